// gemm_skinny.hip -- projections for few rows per weight matrix (decode).
//
// C[rows][n] = sum_k A[row][k] * B[n][k] with A bf16 activations and B either
// a bf16 matrix (pooler, unpooler: step A4, A8) or one expert's MXFP4 matrix
// (W13 and W2: steps A5, A6). With a handful of rows per weight matrix the
// work is bound by streaming B from HBM, so a workgroup owns NF fragments of
// 16 B rows for all K and splits K across its NWAVES wavefronts; partial sums
// are added through LDS. Every weight byte is read once.
//
// MXFP4 is decoded in registers: 16 code bytes per lane (32 elements, one
// E8M0 block) become four bf16x8 MFMA operands with the gfx950 scaled FP4
// conversion, so no bf16 copy of a weight ever reaches memory ("Muse Spark
// Open on Gaudi 2", section "What it taught about Gaudi", shows the cost of
// unpacking touched expert slices to bf16 in memory).
//
// Reduction order inside a 128-element chunk: lane group g = lane/16 owns
// elements [32g, 32g+32); MFMA j takes elements 32g+8j .. +7 from each group,
// for both operands, so A and B always pair the same k.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

template <int BFMT, int EPI, int NF, int MB, int NWAVES, int U>
__global__ __launch_bounds__(64 * NWAVES) void skinny_kernel(SkinnyArgs p) {
  constexpr int NFO = (EPI == EPI_SWIGLU) ? NF / 2 : NF;  // output fragments
  __shared__ float red[NWAVES][MB][NF][256];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 15, g = lane >> 4;

  // ---- rows of this workgroup ----
  int row_begin, row_end, expert = 0;
  if (p.grouped) {
    if (static_cast<int>(blockIdx.y) >= p.counters[0]) return;
    expert = p.active[blockIdx.y];
    row_begin = p.offsets[expert];
    row_end = p.offsets[expert + 1];
  } else {
    row_begin = blockIdx.y * 16 * MB;
    row_end = min(p.m_total, row_begin + 16 * MB);
  }

  // ---- B rows of this lane, one per fragment ----
  const size_t K = static_cast<size_t>(p.K);
  const uint4* brow_q[NF];
  const uint8_t* brow_s[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int r;
    if (EPI == EPI_SWIGLU) {
      const int half = f / (NF / 2), fg = f % (NF / 2);
      r = half * p.inter + (blockIdx.x * (NF / 2) + fg) * 16 + nl;
    } else {
      r = (blockIdx.x * NF + f) * 16 + nl;
    }
    if (BFMT == B_MXFP4) {
      const size_t rr = static_cast<size_t>(expert) * p.b_rows_per_expert + r;
      brow_q[f] = reinterpret_cast<const uint4*>(p.b_codes + rr * (K / 2));
      brow_s[f] = p.b_scales + rr * (K / 32);
    } else {
      brow_q[f] = reinterpret_cast<const uint4*>(p.b_bf16 + static_cast<size_t>(r) * K);
      brow_s[f] = nullptr;
    }
  }

  const int nchunks = p.K / 128;
  const int c_beg = wave * nchunks / NWAVES, c_end = (wave + 1) * nchunks / NWAVES;

  for (int pass_row = row_begin; pass_row < row_end; pass_row += 16 * MB) {
    // ---- A rows of this lane ----
    const uint4* arow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int pos = pass_row + mb * 16 + nl;
      arow[mb] = nullptr;
      if (pos < row_end) {
        const int ar = p.a_gather ? p.sorted[pos] / p.topk : pos;
        arow[mb] = reinterpret_cast<const uint4*>(p.a + static_cast<size_t>(ar) * K);
      }
    }

    f32x4 acc[MB][NF];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mb][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one chunk = 128 reduction elements; each lane group covers 32 of them
    auto run = [&](int kc, auto u_tag) {
      constexpr int UU = decltype(u_tag)::value;
      uint4 av[UU][MB][4];
      uint4 bq[UU][NF][(BFMT == B_MXFP4) ? 1 : 4];
      uint32_t bs[UU][NF];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const int c = kc + u;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (BFMT == B_MXFP4) {
            bq[u][f][0] = brow_q[f][c * 4 + g];
            bs[u][f] = brow_s[f][c * 4 + g];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) bq[u][f][j] = brow_q[f][c * 16 + g * 4 + j];
            bs[u][f] = 0;
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            av[u][mb][j] = arow[mb] ? arow[mb][c * 16 + g * 4 + j] : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < UU; ++u) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float sc = (BFMT == B_MXFP4) ? e8m0_to_f32(bs[u][f]) : 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x8 b;
            if (BFMT == B_MXFP4) {
              const uint4 q = bq[u][f][0];
              const uint32_t d = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
              b = mxfp4x8_to_bf16(d, sc);
            } else {
              b = as_bf16x8(bq[u][f][j]);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][f] = mfma16x16x32(as_bf16x8(av[u][mb][j]), b, acc[mb][f]);
          }
        }
      }
    };
    int kc = c_beg;
    for (; kc + U <= c_end; kc += U) run(kc, std::integral_constant<int, U>{});
    for (; kc < c_end; ++kc) run(kc, std::integral_constant<int, 1>{});

    // ---- add the waves' partial sums through LDS ----
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][mb][f][(4 * g + i) * 16 + nl] = acc[mb][f][i];
    __syncthreads();

    for (int idx = tid; idx < MB * NFO * 256; idx += 64 * NWAVES) {
      const int n = idx & 15, m = (idx >> 4) & 15, fo = (idx >> 8) % NFO, mb = idx / (256 * NFO);
      const int pos = pass_row + mb * 16 + m;
      if (pos >= row_end) continue;
      float s0 = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVES; ++w) s0 += red[w][mb][fo][m * 16 + n];
      if (EPI == EPI_SWIGLU) {
        float s1 = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) s1 += red[w][mb][fo + NF / 2][m * 16 + n];
        const int col = (blockIdx.x * (NF / 2) + fo) * 16 + n;
        const float silu = s0 / (1.0f + expf(-s0));
        static_cast<uint16_t*>(p.out)[static_cast<size_t>(pos) * p.ldo + col] = f32_to_bf16(silu * s1);
      } else if (EPI == EPI_F32_SCATTER) {
        const int col = (blockIdx.x * NF + fo) * 16 + n;
        static_cast<float*>(p.out)[static_cast<size_t>(p.sorted[pos]) * p.ldo + col] = s0;
      } else {
        const int col = (blockIdx.x * NF + fo) * 16 + n;
        static_cast<uint16_t*>(p.out)[static_cast<size_t>(pos) * p.ldo + col] = f32_to_bf16(s0);
      }
    }
    __syncthreads();
  }
}

template <int BFMT, int EPI, int NF, int MB>
hipError_t launch_cfg(const SkinnyArgs& a, dim3 grid, hipStream_t st) {
  constexpr int U = (BFMT == B_MXFP4) ? 4 : 2;
  skinny_kernel<BFMT, EPI, NF, MB, 8, U><<<grid, dim3(512), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

// Dense bf16 projection: out[m][n] = bf16(sum_k a[m][k] * b[n][k]).
hipError_t launch_dense_skinny(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N,
                               int K, hipStream_t st) {
  SkinnyArgs p{};
  p.a = a;
  p.b_bf16 = b;
  p.out = out;
  p.ldo = N;
  p.K = K;
  p.m_total = M;
  const int nf = (N % 32 == 0 && N >= 8192) ? 2 : 1;
  const int mb = M > 16 ? 2 : 1;
  const dim3 grid(N / (16 * nf), (M + 16 * mb - 1) / (16 * mb));
  if (nf == 2)
    return mb == 2 ? launch_cfg<B_BF16, EPI_BF16, 2, 2>(p, grid, st) : launch_cfg<B_BF16, EPI_BF16, 2, 1>(p, grid, st);
  return mb == 2 ? launch_cfg<B_BF16, EPI_BF16, 1, 2>(p, grid, st) : launch_cfg<B_BF16, EPI_BF16, 1, 1>(p, grid, st);
}

// Gate/up projection of every route row against its expert's W13 plus
// SwiGLU: h[i][n] = bf16(silu(g) * u) for sorted position i.
hipError_t launch_gateup_skinny(const ExpertGemm& x, hipStream_t st) {
  SkinnyArgs p{};
  p.grouped = 1;
  p.a = x.lat;
  p.a_gather = 1;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.offsets = x.offsets;
  p.active = x.active;
  p.counters = x.counters;
  p.b_codes = x.w13_codes;
  p.b_scales = x.w13_scales;
  p.b_rows_per_expert = 2 * x.inter;
  p.K = x.latent;
  p.inter = x.inter;
  p.out = x.h;
  p.ldo = x.inter;
  const dim3 grid(x.inter / 16, x.max_active);
  return launch_cfg<B_MXFP4, EPI_SWIGLU, 2, 1>(p, grid, st);
}

// Down projection of every route row: rows[r][n] (fp32, route-major).
hipError_t launch_down_skinny(const ExpertGemm& x, hipStream_t st) {
  SkinnyArgs p{};
  p.grouped = 1;
  p.a = x.h;
  p.a_gather = 0;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.offsets = x.offsets;
  p.active = x.active;
  p.counters = x.counters;
  p.b_codes = x.w2_codes;
  p.b_scales = x.w2_scales;
  p.b_rows_per_expert = x.latent;
  p.K = x.inter;
  p.out = x.rows;
  p.ldo = x.latent;
  const dim3 grid(x.latent / 32, x.max_active);
  return launch_cfg<B_MXFP4, EPI_F32_SCATTER, 2, 1>(p, grid, st);
}

}  // namespace moe
