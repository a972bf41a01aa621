// gemm_skinny.hip -- projections for few rows per weight matrix (decode).
//
// C[rows][n] = sum_k A[row][k] * B[n][k] with A bf16 activations and B either
// a bf16 matrix (pooler, unpooler: steps A4, A8) or one expert's MXFP4 matrix
// (W13 and W2: steps A5, A6). With a handful of rows per weight matrix the
// work is bound by streaming B from HBM: every weight byte is read once, by
// one wavefront, which owns NF fragments of 16 B rows for its share of K and
// keeps U stages of weight loads in flight (software pipeline). All loads are
// raw buffer loads: a lane without a row gets zeros from an out-of-range
// offset, so the loop has no branches and the loads stay in flight.
//
// The A rows either stream through registers beside B, or (AL) are copied
// once per pass of 16 rows into LDS and read from there by every wavefront of
// the workgroup. A bf16 operand costs four times the registers of a 4-bit one
// (64 bytes per lane and 128-element chunk against 16), so staging A in LDS is
// what leaves room for several weight stages in flight: at one or two rows per
// expert the kernel is bound by how many weight bytes each compute unit keeps
// in flight against HBM latency.
//
// MXFP4 is decoded in registers: 16 code bytes per lane (32 elements, one
// E8M0 block) become four bf16x8 MFMA operands through the gfx950 scaled FP4
// conversion, so no bf16 copy of a weight ever reaches memory ("Muse Spark
// Open on Gaudi 2", section "What it taught about Gaudi", shows the cost of
// unpacking touched expert slices to bf16 in memory).
//
// Reduction order inside a 128-element chunk: lane group g = lane/16 owns
// elements [32g, 32g+32) (one E8M0 block); MFMA j takes elements 32g+8j .. +7
// from each group, for both operands, so A and B always pair the same k.
// The scale bytes of a row for two consecutive chunks are 8 contiguous bytes:
// each lane loads all 8 with one load and picks its own.
#include "device_common.h"
#include "kernels.h"
#include "route_small.h"
#include "router_gemv.h"

#include <algorithm>

namespace moe {

namespace {

constexpr int kWaves = 8;  // wavefronts per workgroup

// The block's pre-norm applied in place to bf16 rows staged in LDS (row r at
// lds + r * stride, K elements): n = bf16(x * s * g) with s = 1/sqrt(mean(x^2)
// + eps), every step as the pre-norm kernel takes it (fp64 sum of squares,
// exact whatever its order; fp64 scale and products; one rounding to bf16).
__device__ inline void normalize_staged_rows(uint8_t* lds, uint32_t stride, int n_rows, int K,
                                             const uint16_t* __restrict__ gain, double eps) {
  __shared__ double part[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < n_rows; ++r) {
    uint16_t* row = reinterpret_cast<uint16_t*>(lds + static_cast<size_t>(r) * stride);
    double ss = 0.0;
    for (int h = threadIdx.x * 8; h < K; h += 64 * kWaves * 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + h);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double a = bf16_bits_to_f64(w[j] & 0xFFFFu), b = bf16_bits_to_f64(w[j] >> 16);
        ss += a * a;
        ss += b * b;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += part[w];
    const double s = 1.0 / sqrt(tot / static_cast<double>(K) + eps);
    for (int h = threadIdx.x * 8; h < K; h += 64 * kWaves * 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(row + h);
      const uint4 gq = *reinterpret_cast<const uint4*>(gain + h);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w}, g[4] = {gq.x, gq.y, gq.z, gq.w};
      uint32_t nb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double n0 = bf16_bits_to_f64(w[j] & 0xFFFFu) * s * bf16_bits_to_f64(g[j] & 0xFFFFu);
        const double n1 = bf16_bits_to_f64(w[j] >> 16) * s * bf16_bits_to_f64(g[j] >> 16);
        nb[j] = static_cast<uint32_t>(f64_to_bf16(n0)) | (static_cast<uint32_t>(f64_to_bf16(n1)) << 16);
      }
      *reinterpret_cast<uint4*>(row + h) = uint4{nb[0], nb[1], nb[2], nb[3]};
    }
    __syncthreads();  // (part is rewritten for the next row)
  }
}

template <int BFMT, int MB, int NF, int SC, bool AL>
struct Stage {
  uint4 a[AL ? 1 : SC][MB][4];
  uint4 bq[SC][NF][is_fp4(BFMT) ? 1 : 4];
  uint32_t bs[NF][SC];  // per chunk: its 4 E8M0 bytes, or the dword of its 8 E4M3 bytes holding the lane's two
};

// SC consecutive 128-element chunks of one wavefront: B codes (or bf16 rows)
// and, for MXFP4, the 4*SC scale bytes of each B row that cover those chunks;
// the A rows too unless they are staged in LDS.
// Workgroup = kWaves wavefronts = (kWaves / KS) output groups x KS splits of
// K. A group is 16*NFO output columns (NF fragments of 16 B rows). Each
// wavefront streams its rows over its share of K, SC chunks per stage, with
// U stages of loads in flight; with KS > 1 the split partial sums are added
// in split order through LDS.
// AL: dynamic LDS holds the pass's A rows (p.pass_rows <= 16 * MB of them),
// row stride 2*K + 16 bytes (the 16 rows one ds_read_b128 touches start in
// distinct banks); lanes of rows past the pass's last row read that last row
// (their outputs are not stored).
template <int BFMT, int EPI, int NF, int MB, int U, int KS, int SC, bool AL>
__device__ __forceinline__ void stream_body(const SkinnyArgs& p, int bx, int by) {
  constexpr int NFO = (EPI == EPI_SWIGLU) ? NF / 2 : NF;  // output fragments
  constexpr int GPB = kWaves / KS;                         // groups per workgroup
  __shared__ float red[KS > 1 ? kWaves : 1][MB][NF][256];
  extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int ks = wave % KS;
  const int group = bx * GPB + wave / KS;
  const bool group_ok = group < p.n_groups;

  // ---- rows of this workgroup ----
  // MXFP4 weights are per expert (grouped rows); bf16 weights are one dense matrix
  constexpr bool kGrouped = is_fp4(BFMT);
  constexpr int SB = scale_block(BFMT);  // elements per scale byte
  int row_begin, row_end, expert = 0;
  if constexpr (kGrouped) {
    // one 16-byte entry: expert (-1 past the touched experts) and its rows
    const int4 w = *reinterpret_cast<const int4*>(p.active + 4 * by);
    expert = w.x;
    row_begin = w.y;
    row_end = w.z;
    // (the rows of a touched expert are >= 0, so the test needs all three
    // words and the entry arrives in one load). An entry that is not a
    // touched expert of this call (-1 past the last one; anything outside
    // [0, E) or past the routes in a workspace that no grouping has written)
    // is skipped: no descriptor ever reaches outside the weights.
    if ((expert | row_begin | row_end) < 0 || expert >= p.n_experts || row_end > p.n_routes ||
        row_begin >= row_end)
      return;
  } else {
    row_begin = by * 16 * MB;
    row_end = min(p.m_total, row_begin + 16 * MB);
  }

  // ---- B: one descriptor per expert (or for the dense matrix); per-lane row offsets ----
  const uint32_t K = static_cast<uint32_t>(p.K);
  rsrc_t bq_r, bs_r;
  if (is_fp4(BFMT)) {
    const size_t rows = static_cast<size_t>(p.b_rows_per_expert);
    bq_r = make_rsrc(p.b_codes + expert * rows * (K / 2), static_cast<uint32_t>(rows * (K / 2)));
    bs_r = make_rsrc(p.b_scales + expert * rows * (K / SB), static_cast<uint32_t>(rows * (K / SB)));
  } else {
    bq_r = make_rsrc(p.b_bf16, static_cast<uint32_t>(static_cast<size_t>(p.n_groups) * 16 * NF * K * 2));
    bs_r = bq_r;
  }
  uint32_t bq_off[NF], bs_off[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int r;
    if (EPI == EPI_SWIGLU) {
      r = (f / NFO) * p.inter + (group * NFO + f % NFO) * 16 + nl;
    } else {
      r = (group * NF + f) * 16 + nl;
    }
    if (is_fp4(BFMT)) {
      bq_off[f] = group_ok ? r * (K / 2) + g * 16 : kOutOfRange;
      // NVFP4: lane group g reads dword g/2 of each chunk's 8 scale bytes
      bs_off[f] = group_ok ? r * (K / SB) + (BFMT == B_NVFP4 ? 4 * (g >> 1) : 0) : kOutOfRange;
    } else {
      bq_off[f] = group_ok ? r * K * 2 + g * 64 : kOutOfRange;
      bs_off[f] = 0;
    }
  }
  const rsrc_t a_r = make_rsrc(p.a, p.a_bytes);
  const int sps = p.K / (128 * SC) / KS;  // stages per split, a multiple of U (host)
  const int s_beg = ks * sps;
  const uint32_t a_stride = 2 * K + 16;   // AL: LDS row stride in bytes

  const int pass_rows = AL ? p.pass_rows : 16 * MB;  // rows per pass over the weights
  // A touched expert has at least one row, and so has a dense workgroup: the
  // first pass needs no test, and its weight loads (which depend only on the
  // expert) are issued before anything waits for the row range.
  int pass_row = row_begin;
  bool first_pass = true;
  do {
    uint32_t a_off[MB];
    if (!AL) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int pos = pass_row + mb * 16 + nl;
        a_off[mb] = kOutOfRange;
        if (pos < row_end) {
          const int ar = p.a_gather ? p.sorted[pos] / p.topk : pos;
          a_off[mb] = static_cast<uint32_t>(ar) * K * 2 + g * 64;
        }
      }
    }
    uint32_t a_lrow[MB];  // AL: byte offset of this lane's A row (per row fragment) in LDS

    auto load = [&](Stage<BFMT, MB, NF, SC, AL>& b, int st) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (is_fp4(BFMT)) {
#pragma unroll
          for (int h = 0; h < SC; ++h) b.bq[h][f][0] = buf_load16<kAuxStream>(bq_r, bq_off[f] + (SC * st + h) * 64);
          if (BFMT == B_NVFP4) {  // 8 scale bytes per chunk: the lane's dword of each
#pragma unroll
            for (int h = 0; h < SC; ++h) b.bs[f][h] = buf_load4<kAuxStream>(bs_r, bs_off[f] + (SC * st + h) * 8);
          } else if (SC == 2) {
            const uint2 v = buf_load8b<kAuxStream>(bs_r, bs_off[f] + st * 8);
            b.bs[f][0] = v.x;
            b.bs[f][SC - 1] = v.y;
          } else {
            b.bs[f][0] = buf_load4<kAuxStream>(bs_r, bs_off[f] + st * 4);
          }
        } else {
#pragma unroll
          for (int h = 0; h < SC; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) b.bq[h][f][j] = buf_load16<kAuxStream>(bq_r, bq_off[f] + (SC * st + h) * 256 + j * 16);
#pragma unroll
          for (int h = 0; h < SC; ++h) b.bs[f][h] = 0;
        }
      }
      if (!AL) {
#pragma unroll
        for (int h = 0; h < SC; ++h)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) b.a[h][mb][j] = buf_load16<kAuxDefault>(a_r, a_off[mb] + (SC * st + h) * 256 + j * 16);
      }
    };

    f32x4 acc[MB][NF];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mb][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Stage<BFMT, MB, NF, SC, AL>& b, int st) {
#pragma unroll
      for (int h = 0; h < SC; ++h) {
        bf16x8 av[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (AL) {
              const uint32_t off = a_lrow[mb] + ((SC * st + h) * 128 + g * 32 + j * 8) * 2;
              av[mb][j] = as_bf16x8(*reinterpret_cast<const uint4*>(a_lds + off));
            } else {
              av[mb][j] = as_bf16x8(b.a[AL ? 0 : h][mb][j]);
            }
          }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          // MXFP4: the lane group's 32 elements share byte g of the chunk's
          // dword; NVFP4: its two 16-element blocks have bytes 2g and 2g+1 of
          // the chunk's 8 bytes (the E4M3 value alone: the per-tensor scale
          // multiplies the accumulator, so every decoded weight is exact in bf16)
          float sc_lo = 0.f, sc_hi = 0.f;
          if (BFMT == B_MXFP4) {
            sc_lo = sc_hi = e8m0_to_f32((b.bs[f][h] >> (8 * g)) & 0xFFu);
          } else if (BFMT == B_NVFP4) {
            const uint32_t w = b.bs[f][h] >> (16 * (g & 1));
            sc_lo = e4m3_to_f32(w & 0xFFu);
            sc_hi = e4m3_to_f32((w >> 8) & 0xFFu);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x8 bv;
            if (is_fp4(BFMT)) {
              const uint4 q = b.bq[h][f][0];
              const uint32_t d = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
              bv = BFMT == B_NVFP4 ? nvfp4x8_to_bf16(d, j < 2 ? sc_lo : sc_hi) : mxfp4x8_to_bf16(d, sc_lo);
            } else {
              bv = as_bf16x8(b.bq[h][f][j]);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][f] = mfma16x16x32(av[mb][j], bv, acc[mb][f]);
          }
        }
      }
    };

    // AL: the A rows into LDS in 16-byte pieces (out-of-range pieces load
    // zeros and are not stored). Rows known without the row range (dense
    // rows, or every token row once) have their first pieces issued before
    // the weight stages, so they arrive first and the barrier does not wait
    // for the weights; the others are read behind the first stages.
    const int pr = static_cast<int>(K / 8);  // pieces per row
    const bool a_early = !kGrouped || p.a_tokens;
    const bool a_fill = AL && (!p.a_tokens || first_pass);
    constexpr int kPre = 2, kFill = 4;
    uint4 pre[kPre];
    if (a_fill && a_early) {
      const int early_total = (p.a_tokens ? p.a_tokens : min(pass_rows, row_end - pass_row)) * pr;
#pragma unroll
      for (int q = 0; q < kPre; ++q) {
        const int i = static_cast<int>(threadIdx.x) + q * 64 * kWaves;
        const int row = i / pr;
        const int ar = p.a_tokens ? row : pass_row + row;
        pre[q] = buf_load16<kAuxDefault>(
            a_r, i < early_total ? static_cast<uint32_t>(ar) * K * 2 + static_cast<uint32_t>(i - row * pr) * 16
                                 : kOutOfRange);
      }
    }

    Stage<BFMT, MB, NF, SC, AL> buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(buf[u], s_beg + u);

    // from here on the row range of the pass is needed
    const int n_rows = min(pass_rows, row_end - pass_row);
    // with every token row staged, the LDS row of sorted position i is its token
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = min(mb * 16 + nl, n_rows - 1);
      a_lrow[mb] = static_cast<uint32_t>(p.a_tokens ? p.sorted[pass_row + r] / p.topk : r) * a_stride;
    }
    const int a_total = (p.a_tokens ? p.a_tokens : n_rows) * pr;
    auto a_src = [&](int i) -> uint32_t {
      if (i >= a_total) return kOutOfRange;
      const int row = i / pr;
      const int ar = p.a_tokens ? row : p.a_gather ? p.sorted[pass_row + row] / p.topk : pass_row + row;
      return static_cast<uint32_t>(ar) * K * 2 + static_cast<uint32_t>(i - row * pr) * 16;
    };
    auto a_store = [&](int i, const uint4& v) {
      if (i < a_total) {
        const int row = i / pr;
        *reinterpret_cast<uint4*>(a_lds + row * a_stride + (i - row * pr) * 16) = v;
      }
    };

    if (a_fill) {
      if (a_early) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) a_store(threadIdx.x + q * 64 * kWaves, pre[q]);
      }
      for (int base = static_cast<int>(threadIdx.x) + (a_early ? kPre * 64 * kWaves : 0); base < a_total;
           base += kFill * 64 * kWaves) {
        uint4 v[kFill];
#pragma unroll
        for (int q = 0; q < kFill; ++q) v[q] = buf_load16<kAuxDefault>(a_r, a_src(base + q * 64 * kWaves));
#pragma unroll
        for (int q = 0; q < kFill; ++q) a_store(base + q * 64 * kWaves, v[q]);
      }
      __syncthreads();
      if constexpr (AL && !kGrouped) {
        if (p.pre_gain) {  // the block's pre-norm of the staged rows (one pass holds them all)
          normalize_staged_rows(a_lds, a_stride, n_rows, static_cast<int>(K), p.pre_gain, p.pre_eps);
          __syncthreads();
        }
      }
    }

    for (int s0 = s_beg; s0 + U < s_beg + sps; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(buf[u], s0 + u);
        load(buf[u], s0 + U + u);
        // keep each refill right after the compute that frees its registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) compute(buf[u], s_beg + sps - U + u);

    // ---- add the K splits (in split order) ----
    if (KS > 1) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wave][mb][f][(4 * g + i) * 16 + nl] = acc[mb][f][i];
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float s = 0.f;
#pragma unroll
              for (int q = 0; q < KS; ++q) s += red[wave + q][mb][f][(4 * g + i) * 16 + nl];
              acc[mb][f][i] = s;
            }
      }
    }

    // ---- epilogue ----
    // NVFP4: the tensor's global scale, applied to the fp32 sums
    const float gs = (BFMT == B_NVFP4) ? p.b_global[expert] : 1.0f;
    if (ks == 0 && group_ok) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int fo = 0; fo < NFO; ++fo) {
          const int col = (group * NFO + fo) * 16 + nl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = pass_row + mb * 16 + 4 * g + i;
            if (mb * 16 + 4 * g + i >= n_rows) continue;
            const float s0 = acc[mb][fo][i] * gs;
            if (EPI == EPI_SWIGLU) {
              const float s1 = acc[mb][fo + NFO][i] * gs;
              const float silu = s0 / (1.0f + expf(-s0));
              static_cast<uint16_t*>(p.out)[static_cast<size_t>(pos) * p.ldo + col] = f32_to_bf16(silu * s1);
            } else if (EPI == EPI_F32_SCATTER) {
              static_cast<float*>(p.out)[static_cast<size_t>(p.sorted[pos]) * p.ldo + col] = s0;
            } else {
              static_cast<uint16_t*>(p.out)[static_cast<size_t>(pos) * p.ldo + col] = f32_to_bf16(s0);
            }
          }
        }
      }
      // fp32 route rows: sum of squares over this group's columns, per row
      if (EPI == EPI_F32_SCATTER && p.ssp) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float q = 0.f;
#pragma unroll
            for (int f = 0; f < NF; ++f) q += (acc[mb][f][i] * gs) * (acc[mb][f][i] * gs);
            q = row16_sum_f32(q);
            const int pos = pass_row + mb * 16 + 4 * g + i;
            if (nl == 0 && mb * 16 + 4 * g + i < n_rows)
              p.ssp[static_cast<size_t>(p.sorted[pos]) * p.n_groups + group] = q;
          }
        }
      }
    }
    // the next pass rewrites the reduction buffer and the staged A rows
    if (KS > 1 || (AL && !p.a_tokens)) __syncthreads();
    pass_row += pass_rows;
    first_pass = false;
  } while (pass_row < row_end);
}

// The expert kernels keep two workgroups per CU (at most 128 VGPRs).
template <int BFMT, int EPI, int NF, int MB, int U, int KS, int SC, bool AL>
__global__ __launch_bounds__(64 * kWaves, is_fp4(BFMT) ? 4 : 1) void stream_kernel(SkinnyArgs p) {
  stream_body<BFMT, EPI, NF, MB, U, KS, SC, AL>(p, blockIdx.x, blockIdx.y);
}

// The router (T <= 16 tokens) and the pooler read only the layer input, so
// one launch runs both: workgroups 0 .. E-1 compute one expert's logits each
// (router_gemv.h, eight wavefronts), the rest are the pooler's streaming
// workgroups. The router's 8 MiB then streams beside the pooler's weights
// instead of in a launch of its own. The router reads the same bf16 input,
// or (xf set) the fp32 output of the block's pre-norm. For T <= 8 tokens the
// router workgroups also take the top K and group the routes (one of them,
// those that find all logits stored; route_small.h), under the pooler's
// stream, so routing needs no launch of its own either.
struct RouterArgs {
  const uint16_t* x;
  const float* xf;
  const float* wr;
  float* logits;
  int T, H, E;
  RouteFuse rf;  // rf.tagged set: the router workgroups also route (route_small.h)
  // the block's pre-norm folded in (XIN_PRENORM): x is the residual stream
  const uint16_t* pre_gain;
  double pre_eps;
  float* nf32_out;     // workgroup 0 stores the pre-norm's outputs (fp32, bf16)
  uint16_t* nbf16_out;
};

enum { XIN_BF16 = 0, XIN_F32 = 1, XIN_PRENORM = 2 };

template <int TMAX, int U, int KS, int SC, bool AL, int XIN>
__global__ __launch_bounds__(64 * kWaves) void pool_router_kernel(SkinnyArgs p, RouterArgs r) {
  __shared__ double part[kWaves][TMAX];
  if (static_cast<int>(blockIdx.x) < r.E) {
    const uint32_t gen =
        r.rf.tagged ? __hip_atomic_load(r.rf.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint32_t tag = route_tag(gen);
    if constexpr (XIN == XIN_PRENORM)
      router_prenorm_body<TMAX, kWaves>(r.x, r.pre_gain, r.pre_eps, r.wr, r.logits, r.T, r.H, r.E,
                                        blockIdx.x, part, r.rf.tagged, tag,
                                        blockIdx.x == 0 ? r.nf32_out : nullptr, r.nbf16_out);
    else if constexpr (XIN == XIN_F32)
      router_gemv_body<TMAX, kWaves, float>(r.xf, r.wr, r.logits, r.T, r.H, r.E, blockIdx.x, part,
                                            r.rf.tagged, tag);
    else
      router_gemv_body<TMAX, kWaves>(r.x, r.wr, r.logits, r.T, r.H, r.E, blockIdx.x, part,
                                     r.rf.tagged, tag);
    if (r.rf.tagged) route_when_complete<kWaves>(r.rf, gen, r.T, r.E);
    return;
  }
  stream_body<B_BF16, EPI_BF16, 1, 1, U, KS, SC, AL>(p, blockIdx.x - r.E, 0);
}

// Launch shape of one projection: A through LDS, and the number of
// wavefronts below which K is split. The weight stages in flight (at most
// UMAX) and the largest K split (KSMAX) are template parameters of the
// launchers, so only reachable kernel shapes are compiled.
struct Tune {
  bool al;
  int split_waves = 8192;  // split K while fewer wavefronts than this stream the weights
};

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr size_t kAlLdsBudget = 40 * 1024;

template <int TMAX, int U, int KS, int SC, bool AL>
hipError_t launch_fused(const SkinnyArgs& a, const RouterArgs& r, int gx, size_t lds, hipStream_t st) {
  if (r.pre_gain) {
    // (the pooler normalises its staged rows: A in LDS, one pass)
    if constexpr (AL)
      MOE_LAUNCH((pool_router_kernel<TMAX, U, KS, SC, AL, XIN_PRENORM>), dim3(gx + r.E),
                 dim3(64 * kWaves), lds, st, a, r);
    else
      return hipErrorInvalidValue;
  } else if (r.xf) {
    MOE_LAUNCH((pool_router_kernel<TMAX, U, KS, SC, AL, XIN_F32>), dim3(gx + r.E), dim3(64 * kWaves), lds,
               st, a, r);
  } else {
    MOE_LAUNCH((pool_router_kernel<TMAX, U, KS, SC, AL, XIN_BF16>), dim3(gx + r.E), dim3(64 * kWaves), lds,
               st, a, r);
  }
  return hipGetLastError();
}

template <int BFMT, int EPI, int NF, int MB, int U, int KS, int SC>
hipError_t launch_al(const SkinnyArgs& a, int ny, bool al, const RouterArgs* fuse, hipStream_t st) {
  const dim3 grid((a.n_groups + kWaves / KS - 1) / (kWaves / KS), ny);
  const dim3 block(64 * kWaves);
  const size_t lds = al ? static_cast<size_t>(a.pass_rows) * (2 * static_cast<size_t>(a.K) + 16) : 0;
  if constexpr (BFMT == B_BF16 && EPI == EPI_BF16 && NF == 1 && MB == 1) {
    if (fuse) {
      if (fuse->T <= 1)
        return al ? launch_fused<1, U, KS, SC, true>(a, *fuse, grid.x, lds, st)
                  : launch_fused<1, U, KS, SC, false>(a, *fuse, grid.x, lds, st);
      return al ? launch_fused<16, U, KS, SC, true>(a, *fuse, grid.x, lds, st)
                : launch_fused<16, U, KS, SC, false>(a, *fuse, grid.x, lds, st);
    }
  }
  if (al) {
    MOE_LAUNCH((stream_kernel<BFMT, EPI, NF, MB, U, KS, SC, true>), grid, block, lds, st, a);
  } else {
    MOE_LAUNCH((stream_kernel<BFMT, EPI, NF, MB, U, KS, SC, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int BFMT, int EPI, int NF, int MB, int UMAX, int KS, int SC>
hipError_t launch_ks(const SkinnyArgs& a, int ny, int sps, const Tune& t, const RouterArgs* fuse,
                     hipStream_t st) {
  static_assert(UMAX >= 1 && UMAX <= 2, "weight stages in flight");
  // the pipeline depth must divide the stages of a split
  if constexpr (UMAX == 2)
    if (sps % 2 == 0) return launch_al<BFMT, EPI, NF, MB, 2, KS, SC>(a, ny, t.al, fuse, st);
  return launch_al<BFMT, EPI, NF, MB, 1, KS, SC>(a, ny, t.al, fuse, st);
}

// Split K across the wavefronts of a workgroup when there are few output
// groups, so that about t.split_waves wavefronts stream the weights. a_rows bounds
// the rows of one pass (for the LDS size of A).
template <int BFMT, int EPI, int NF, int MB, int UMAX, int KSMAX>
hipError_t launch_u(SkinnyArgs a, int ny, Tune t, int a_rows, hipStream_t st,
                    const RouterArgs* fuse = nullptr, bool al_one_pass = false) {
  // AL: rows per pass such that the staged rows fit the LDS budget of a
  // workgroup (several workgroups per compute unit); an expert with more
  // rows streams its weights once per pass.
  const size_t row_bytes = 2 * static_cast<size_t>(a.K) + 16;
  a.pass_rows = static_cast<int>(std::min<size_t>(std::min(16 * MB, std::max(1, a_rows)),
                                                  std::max<size_t>(1, kAlLdsBudget / row_bytes)));
  if (a.pass_rows * row_bytes + sizeof(float) * kWaves * MB * NF * 256 > kMaxLds) t.al = false;
  // (dense rows are few and the weights large: staging only pays when all
  // rows fit one pass)
  if (al_one_pass && a.pass_rows < std::min(16 * MB, std::max(1, a_rows))) t.al = false;
  if (!t.al) a.pass_rows = 16 * MB;
  // a gather whose tokens all fit one pass stages every token row once
  a.a_tokens = (t.al && a.a_gather && a_rows <= a.pass_rows) ? a_rows : 0;
  const int nchunks = a.K / 128;
  if (nchunks % 2) {  // odd chunk count (K = 128 * odd): one-chunk stages, no split
    return launch_ks<BFMT, EPI, NF, MB, UMAX, 1, 1>(a, ny, nchunks, t, fuse, st);
  }
  const int nstages = nchunks / 2;
  const int64_t groups = static_cast<int64_t>(a.n_groups) * ny;
  int ks = 1;
  while (ks < kWaves && ks < KSMAX && groups * ks < t.split_waves && nstages % (2 * ks) == 0) ks *= 2;
  const int sps = nstages / ks;
  if constexpr (KSMAX >= 8)
    if (ks == 8) return launch_ks<BFMT, EPI, NF, MB, UMAX, 8, 2>(a, ny, sps, t, fuse, st);
  if constexpr (KSMAX >= 4)
    if (ks == 4) return launch_ks<BFMT, EPI, NF, MB, UMAX, 4, 2>(a, ny, sps, t, fuse, st);
  if constexpr (KSMAX >= 2)
    if (ks == 2) return launch_ks<BFMT, EPI, NF, MB, UMAX, 2, 2>(a, ny, sps, t, fuse, st);
  return launch_ks<BFMT, EPI, NF, MB, UMAX, 1, 2>(a, ny, sps, t, fuse, st);
}

// Weight stages in flight of the dense projections with one 16-row fragment
// (A staged in LDS).
constexpr int kDenseU = 2;
// The router + pooler launch keeps one weight stage in flight: at two its
// registers (163) allow one workgroup per CU, and the pooler's workgroups
// wait for the router's; at one (123) both share the CUs (T = 1 layer
// 91.4 -> 89.4 us).
constexpr int kPoolRouterU = 1;
// The expert projections: two weight stages in flight, K split at most four
// ways, A staged in LDS.
constexpr int kExpertU = 2;
constexpr int kExpertKs = 4;

}  // namespace

// The block's pre-norm folds into the router + pooler launch for one token
// whose row the pooler stages in LDS (the row it normalises); the router
// then runs its one-token body (125 VGPRs with the fold, two workgroups per
// CU; its 16-token body would take 243).
bool prenorm_fold_ok(int T, int H) {
  const size_t row_bytes = 2 * static_cast<size_t>(H) + 16;
  return T == 1 && row_bytes <= kAlLdsBudget && row_bytes + sizeof(float) * kWaves * 256 <= kMaxLds;
}

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
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(M) * K * 2);
  p.n_groups = N / 16;
  const int mb = M > 16 ? 2 : 1;
  const int ny = (M + 16 * mb - 1) / (16 * mb);
  // one 16-row fragment: A staged in LDS, two weight stages in flight; two
  // fragments: A in registers
  // (A in registers: one fragment of weight rows keeps two stages in flight,
  // T = 32 pooler 33.3 -> 30.9 us; two fragments keep one, two measured 66 us)
  const Tune t1{true}, t2{false};
  // two fragments of A rows against two of weight rows per wavefront halve
  // the A loads per weight byte; taken while that still leaves 256 groups
  // (T = 32 unpooler 31.1 -> 25.4 us; the pooler, 128 groups, slowed down)
  if (mb == 2 && N % 32 == 0 && N / 32 >= 256) {
    p.n_groups = N / 32;
    return launch_u<B_BF16, EPI_BF16, 2, 2, 1, kWaves>(p, ny, t2, M, st, nullptr, true);
  }
  return mb == 2 ? launch_u<B_BF16, EPI_BF16, 1, 2, 2, kWaves>(p, ny, t2, M, st, nullptr, true)
                 : launch_u<B_BF16, EPI_BF16, 1, 1, kDenseU, kWaves>(p, ny, t1, M, st, nullptr, true);
}

// The pooler (T <= 16 rows) with the router logits in the same launch; the
// router reads xf (fp32) when given, else x. With pre (the block's pre-norm
// folded in) x is the residual stream, and both the router and the pooler
// normalise it themselves.
hipError_t launch_pool_router(const uint16_t* x, const uint16_t* pooler, uint16_t* lat, int T, int L,
                              int H, const float* wr, float* logits, int E, hipStream_t st,
                              const float* xf, const RouteFuse* rf, const PreNormFold* pre) {
  SkinnyArgs p{};
  p.a = x;
  p.b_bf16 = pooler;
  p.out = lat;
  p.ldo = L;
  p.K = H;
  p.m_total = T;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(T) * H * 2);
  p.n_groups = L / 16;
  RouterArgs r{x, xf, wr, logits, T, H, E, RouteFuse{}, nullptr, 0.0, nullptr, nullptr};
  if (rf) {
    if (T > kWaves || T * rf->K > 64) return hipErrorInvalidValue;  // one wavefront per token, 64 routes
    r.rf = *rf;
  }
  if (pre) {
    if (!prenorm_fold_ok(T, H)) return hipErrorInvalidValue;
    r.pre_gain = pre->gain;
    r.pre_eps = pre->eps;
    r.nf32_out = pre->nf32_out;
    r.nbf16_out = pre->nbf16_out;
    p.pre_gain = pre->gain;
    p.pre_eps = pre->eps;
  }
  const Tune t{true};
  return launch_u<B_BF16, EPI_BF16, 1, 1, kPoolRouterU, kWaves>(p, 1, t, T, st, &r, true);
}

// Gate/up projection of every route row against its expert's W13 plus
// SwiGLU: h[i][n] = bf16(silu(g) * u) for sorted position i. An expert has
// at most one row per token.
hipError_t launch_gateup_skinny(const ExpertGemm& x, hipStream_t st) {
  SkinnyArgs p{};
  p.a = x.lat;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.latent * 2);
  p.a_gather = 1;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.active = x.active;
  p.b_codes = x.w13_codes;
  p.b_scales = x.w13_scales;
  p.b_rows_per_expert = 2 * x.inter;
  p.K = x.latent;
  p.inter = x.inter;
  p.out = x.h;
  p.ldo = x.inter;
  p.n_groups = x.inter / 16;
  p.b_global = x.w13_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  const Tune t{true};
  return x.nvfp4 ? launch_u<B_NVFP4, EPI_SWIGLU, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, x.tokens, st)
                 : launch_u<B_MXFP4, EPI_SWIGLU, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, x.tokens, st);
}

// Down projection of every route row: rows[r][n] (fp32, route-major).
hipError_t launch_down_skinny(const ExpertGemm& x, hipStream_t st) {
  SkinnyArgs p{};
  p.a = x.h;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.topk * x.inter * 2);
  p.a_gather = 0;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.active = x.active;
  p.b_codes = x.w2_codes;
  p.b_scales = x.w2_scales;
  p.b_rows_per_expert = x.latent;
  p.K = x.inter;
  p.out = x.rows;
  p.ldo = x.latent;
  p.n_groups = x.latent / 32;
  p.ssp = x.ssp;
  p.b_global = x.w2_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  // (T = 32, about 163 touched experts: four K splits take the down
  // projection from 441 to 422 us in a harness, while gate/up is fastest
  // unsplit)
  const Tune t{true, 131072};
  return x.nvfp4 ? launch_u<B_NVFP4, EPI_F32_SCATTER, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, x.tokens, st)
                 : launch_u<B_MXFP4, EPI_F32_SCATTER, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, x.tokens, st);
}

}  // namespace moe
