// stream_body.h -- the streaming projection body (decode regime), shared by
// the per-step launches (gemm_skinny.hip) and the persistent decode layer
// (decode_layer.hip).
//
// C[rows][n] = sum_k A[row][k] * B[n][k] with A bf16 activations and B either
// a bf16 matrix (pooler, unpooler: steps A4, A8) or one expert's 4-bit matrix
// (W13 and W2: steps A5, A6); every weight byte is read once, by one
// wavefront (see gemm_skinny.hip for the design and its measurements).
//
// Two template parameters serve the persistent layer, where one launch
// hands data between workgroups:
//  - COH: the A rows, the work list and the route order are read, and the
//    outputs written, with device-coherent (sc1) accesses, the form that
//    device-scope atomic loads and stores take on gfx950, so that a value
//    another workgroup stored (and waited for) before signalling is seen;
//  - Hook: called once per call after the first weight stages are issued and
//    before anything reads A or the row range, so a workgroup can prefetch
//    its weights and then wait for the data it depends on.
#pragma once
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};


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
//
// B_NVFP4_FEW (AL only; p.pass_rows <= 4 * MB): a fragment holds 4 rows, and
// MFMA row 4c + q carries pass row q restricted to block group c (elements
// [32c, 32c+32) of each chunk: the E4M3 blocks 2c and 2c+1, whose codes lane
// group c holds): lane (nl, g) reads row nl%4 where g == nl/4 and a row of
// zeros (after the staged rows in LDS) elsewhere. B_NVFP4_ONE is the same
// with one row per fragment (q = 0 only), which needs a quarter of the FMAs. The codes are decoded at
// unit scale, so MFMAs j = 0, 1 (chained) leave in lane (nl, g), register q,
// row q's sum over block 2g of activation times E2M1 value, and MFMAs 2, 3
// that over block 2g+1: the lane multiplies them by its own two block scales
// and adds them to its accumulators, and after the last chunk the four lane
// groups' sums are added across lanes (in a fixed order). Per 8 weights this
// is one conversion plus two fp32 FMAs, against four multiplies and two
// roundings when every decoded weight is scaled.
template <int BFMT, int EPI, int NF, int MB, int U, int KS, int SC, bool AL, bool COH = false,
          class Hook = NoHook>
__device__ __forceinline__ void stream_body(const SkinnyArgs& p, int bx, int by,
                                            const Hook& hook = Hook{}) {
  constexpr bool kHook = !std::is_same<Hook, NoHook>::value;
  constexpr int kAuxA = aux_for(COH);
  constexpr int kFR = few_rows(BFMT);  // few-rows forms: rows per fragment
  constexpr bool kFew = kFR > 0;
  static_assert(!kFew || AL, "the few-rows forms read their zero row from LDS");
  static_assert(EPI != EPI_ROUTE_SUM || (AL && NF == 1 && MB == 1 && !is_fp4(BFMT)),
                "the route sum: dense weights, one fragment, A rows staged in LDS");
  constexpr bool kRouteSum = EPI == EPI_ROUTE_SUM;
  constexpr int NFO = (EPI == EPI_SWIGLU) ? NF / 2 : NF;  // output fragments
  constexpr int GPB = kWaves / KS;                         // groups per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];
  // the K-split partial sums: [kWaves][MB][NF][256] floats in the dynamic LDS
  // after the staged A rows (p.red_off)
  float(*red)[MB][NF][256] = reinterpret_cast<float(*)[MB][NF][256]>(a_lds + p.red_off);
  // (the wavefront index made scalar: the K split, the output group and the
  // stage offsets then stay in scalar registers)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    int4 w;
    if constexpr (COH) {
      w = int4{ld_i32<true>(p.active + 4 * by), ld_i32<true>(p.active + 4 * by + 1),
               ld_i32<true>(p.active + 4 * by + 2), 0};
    } else {
      w = *reinterpret_cast<const int4*>(p.active + 4 * by);
    }
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
    // (the split into light and heavy experts: a heavy one is the row tiles')
    if (p.max_rows > 0 && row_end - row_begin > p.max_rows) return;
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
      bs_off[f] = group_ok ? r * (K / SB) + (is_nvfp4(BFMT) ? 4 * (g >> 1) : 0) : kOutOfRange;
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
          const int ar = p.a_gather ? ld_i32<COH>(p.sorted + pos) / p.topk : pos;
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
          if (is_nvfp4(BFMT)) {  // 8 scale bytes per chunk: the lane's dword of each
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
            for (int j = 0; j < 4; ++j) b.a[h][mb][j] = buf_load16<kAuxA>(a_r, a_off[mb] + (SC * st + h) * 256 + j * 16);
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
        if constexpr (kFew) {
          // block 2g (MFMAs 0, 1), then block 2g+1 (MFMAs 2, 3), each for
          // every fragment, so that only half the A and decoded B operands
          // are live at a time
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            bf16x8 a0[MB], a1[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const uint32_t off = a_lrow[mb] + ((SC * st + h) * 128 + g * 32 + half * 16) * 2;
              a0[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(a_lds + off));
              a1[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(a_lds + off + 16));
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              const uint4 q = b.bq[h][f][0];
              const int w = static_cast<int>(b.bs[f][h] >> (16 * (g & 1)));  // blocks 2g, 2g+1: bytes 0, 1
              const float sc = half ? __builtin_amdgcn_cvt_f32_fp8(w, 1) : __builtin_amdgcn_cvt_f32_fp8(w, 0);
              const bf16x8 b0 = mxfp4x8_to_bf16(half ? q.z : q.x, 1.0f);
              const bf16x8 b1 = mxfp4x8_to_bf16(half ? q.w : q.y, 1.0f);
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 d = mfma16x16x32(a1[mb], b1, mfma16x16x32(a0[mb], b0, z));
#pragma unroll
                for (int i = 0; i < kFR; ++i) acc[mb][f][i] = fmaf(d[i], sc, acc[mb][f][i]);
              }
            }
          }
          continue;
        }
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

    // AL: the A rows into LDS in 16-byte pieces, copied straight into LDS
    // right behind the weight stages, in whole 64-piece groups of a row: no
    // registers hold them and nothing waits before they are issued. (Read
    // into registers early instead, the pieces were spilled in the NVFP4
    // kernels, and a spilled load makes the pass wait for it before it issues
    // its weight loads; copied straight, the T = 1 layer went 91.1 -> 90.1 us
    // and T = 32 963 -> 960 us.) Gathered rows (without whole-token
    // staging) are copied so for NVFP4 only, their route order for the pass
    // (one word per row) loaded before the weight stages so that reading it
    // waits for it alone (T = 32 gate/up 639 -> 631 us; MXFP4's went 573 ->
    // 575 us and keeps the register path). With K not a multiple of 512, or
    // under a hook, the rows go through registers after the weight stages
    // are issued (out-of-range pieces load zeros and are not stored).
    const int pr = static_cast<int>(K / 8);  // pieces per row
    // (with a hook, A is not ready before it returns)
    const bool a_fill = AL && (!p.a_tokens || first_pass);
    const bool a_direct =
        a_fill && !kHook && K % 512 == 0 && (p.a_tokens || !p.a_gather || is_nvfp4(BFMT));
    constexpr int kFill = 4;
    const int pass_n = min(pass_rows, row_end - pass_row);  // rows of this pass (>= 1)
    int a_tok = 0;  // gather: lane r < pass_n holds the route of pass row r
    if (a_direct && p.a_gather && !p.a_tokens) a_tok = ld_i32<COH>(p.sorted + pass_row + min(lane, pass_n - 1));

    Stage<BFMT, MB, NF, SC, AL> buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(buf[u], s_beg + u);
    if (first_pass) hook();  // the weights are on their way; now wait for A
    if (a_direct) {
      const int rows = p.a_tokens ? p.a_tokens : pass_n;
      const int gpr = static_cast<int>(K / 512);  // 64-piece groups per row
      const uint32_t lds0 = static_cast<uint32_t>(
          reinterpret_cast<size_t>((__attribute__((address_space(3))) uint8_t*)(a_lds)));
      for (int q = wave; q < rows * gpr; q += kWaves) {
        const int row = q / gpr, piece = (q - row * gpr) * 64;
        const int ar = p.a_tokens ? row
                       : p.a_gather ? __builtin_amdgcn_readlane(a_tok, row) / p.topk
                                    : pass_row + row;
        lds_copy16(a_r, static_cast<uint32_t>(ar) * K * 2 + static_cast<uint32_t>(piece + lane) * 16,
                   __builtin_amdgcn_readfirstlane(lds0 + row * a_stride + piece * 16));
      }
    }

    // from here on the row range of the pass is needed
    const int n_rows = min(pass_rows, row_end - pass_row);
    // with every token row staged, the LDS row of sorted position i is its token
    const uint32_t zero_off = static_cast<uint32_t>(p.pass_rows) * a_stride;  // few-rows forms
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int slot = kFew ? mb * kFR + (nl & 3) : mb * 16 + nl;
      const int r = min(slot, n_rows - 1);
      a_lrow[mb] = static_cast<uint32_t>(p.a_tokens ? ld_i32<COH>(p.sorted + pass_row + r) / p.topk : r) * a_stride;
      if (kFew && ((nl >> 2) != g || (nl & 3) >= kFR || slot >= n_rows)) a_lrow[mb] = zero_off;
    }
    const int a_total = (p.a_tokens ? p.a_tokens : n_rows) * pr;
    auto a_src = [&](int i) -> uint32_t {
      if (i >= a_total) return kOutOfRange;
      const int row = i / pr;
      const int ar = p.a_tokens ? row : p.a_gather ? ld_i32<COH>(p.sorted + pass_row + row) / p.topk : pass_row + row;
      return static_cast<uint32_t>(ar) * K * 2 + static_cast<uint32_t>(i - row * pr) * 16;
    };
    auto a_store = [&](int i, const uint4& v) {
      if (i < a_total) {
        const int row = i / pr;
        *reinterpret_cast<uint4*>(a_lds + row * a_stride + (i - row * pr) * 16) = v;
      }
    };

    // EPI_ROUTE_SUM: the post-norm scale of each A row (one pass holds them
    // all), c = w / sqrt(ss / K + eps), ss the row's sum of squares added from
    // the down projection's partial sums in the combine's order (wavefront q
    // takes rows q and q + 8); loaded here, behind the weight and row loads
    __shared__ float c_lds[kRouteSum ? 16 : 1];
    float cq[2] = {0.f, 0.f}, cw[2] = {0.f, 0.f};
    if constexpr (kRouteSum) {
      const int nb = static_cast<int>(K) / 32;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wave + 8 * j;
        if (r < n_rows) {
          for (int c = lane; c < nb; c += 64) cq[j] += ld_f32<COH>(p.ssp + static_cast<size_t>(pass_row + r) * nb + c);
          cw[j] = ld_f32<COH>(p.route_w + pass_row + r);
        }
      }
    }

    if (a_fill) {
      if (a_direct) wait_vm_keep<0>();  // the copies have landed
      for (int base = static_cast<int>(threadIdx.x); !a_direct && base < a_total; base += kFill * 64 * kWaves) {
        uint4 v[kFill];
#pragma unroll
        for (int q = 0; q < kFill; ++q) v[q] = buf_load16<kAuxA>(a_r, a_src(base + q * 64 * kWaves));
#pragma unroll
        for (int q = 0; q < kFill; ++q) a_store(base + q * 64 * kWaves, v[q]);
      }
      if (kFew && first_pass) {  // the row of zeros (no pass writes it again)
        for (int i = static_cast<int>(threadIdx.x); i < pr; i += 64 * kWaves)
          *reinterpret_cast<uint4*>(a_lds + zero_off + i * 16) = uint4{0u, 0u, 0u, 0u};
      }
      if constexpr (kRouteSum) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wave + 8 * j;
          const float ss = wave_sum_f32(cq[j]);
          if (lane == 0 && r < n_rows) c_lds[r] = cw[j] * (1.0f / sqrtf(ss / static_cast<float>(K) + p.norm_eps));
        }
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

    // few-rows forms: add the four block groups' sums (lane groups 0 + 1,
    // 2 + 3, then the two); every lane group then holds rows mb*kFR .. +kFR-1
    if constexpr (kFew) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < kFR; ++i) {
            const float v = acc[mb][f][i] + __shfl_xor(acc[mb][f][i], 16, 64);
            acc[mb][f][i] = v + __shfl_xor(v, 32, 64);
          }
    }

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
    const float gs = is_nvfp4(BFMT) ? p.b_global[expert] : 1.0f;
    // pass row of this lane's output i of fragment mb (few-rows forms: lane
    // group 0 stores, the others hold the same sums)
    auto out_row = [&](int mb, int i) {
      return kFew ? (g == 0 && i < kFR ? mb * kFR + i : pass_rows) : mb * 16 + 4 * g + i;
    };
    if (kRouteSum) {
      // out[t][col] = bf16(sum over the token's routes of c_r * D[r][col]):
      // fragment row r = 4g + i is route row pass_row + r (one pass from row
      // 0, so token pass_row / K + r / K); the lane adds its rows of token t,
      // then the four lane groups are added (groups 0 + 1 and 2 + 3, then the
      // two), and lane group 0 stores
      if (ks == 0 && group_ok) {
        const int col = group * 16 + nl;
        const int n_tok = (n_rows + p.topk - 1) / p.topk;
        for (int t = 0; t < n_tok; ++t) {
          float v = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            if (r < n_rows && r / p.topk == t) v += c_lds[r] * acc[0][0][i];
          }
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);
          if (g == 0)
            st_val<COH>(static_cast<uint16_t*>(p.out) + static_cast<size_t>(pass_row / p.topk + t) * p.ldo + col,
                            f32_to_bf16(v));
        }
      }
    } else if (ks == 0 && group_ok) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int fo = 0; fo < NFO; ++fo) {
          const int col = (group * NFO + fo) * 16 + nl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = pass_row + out_row(mb, i);
            if (out_row(mb, i) >= n_rows) continue;
            const float s0 = acc[mb][fo][i] * gs;
            if (EPI == EPI_SWIGLU) {
              const float s1 = acc[mb][fo + NFO][i] * gs;
              const float silu = s0 / (1.0f + expf(-s0));
              st_val<COH>(static_cast<uint16_t*>(p.out) + static_cast<size_t>(pos) * p.ldo + col,
                          f32_to_bf16(silu * s1));
            } else if (is_scatter(EPI)) {
              const size_t route = static_cast<size_t>(ld_i32<COH>(p.sorted + pos));
              st_val<COH>(static_cast<float*>(p.out) + route * p.ldo + col, s0);
              if constexpr (EPI == EPI_F32_SCATTER_SCALED) {  // bf16(gain * row)
                const float gv = bf16_to_f32(p.gain[(p.gain_per_expert ? static_cast<size_t>(expert) * p.ldo : 0) + col]);
                st_val<COH>(p.out_scaled + route * p.ldo + col, f32_to_bf16(s0 * gv));
              }
            } else {
              st_val<COH>(static_cast<uint16_t*>(p.out) + static_cast<size_t>(pos) * p.ldo + col, f32_to_bf16(s0));
            }
          }
        }
      }
      // fp32 route rows: sum of squares over this group's columns, per row
      if (is_scatter(EPI) && p.ssp) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float q = 0.f;
#pragma unroll
            for (int f = 0; f < NF; ++f) q += (acc[mb][f][i] * gs) * (acc[mb][f][i] * gs);
            q = row16_sum_f32(q);
            const int pos = pass_row + out_row(mb, i);
            if (nl == 0 && out_row(mb, i) < n_rows)
              st_val<COH>(p.ssp + static_cast<size_t>(ld_i32<COH>(p.sorted + pos)) * p.n_groups + group, q);
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


}  // namespace moe
