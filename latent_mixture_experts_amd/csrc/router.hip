// router.hip -- router logits in fp64 and wavefront top-K (steps A1, A2).
//
// "Muse Spark Open on Gaudi 2", section "What was built": the router is fp32
// over 256 experts and keeps 8. Each logit is the fp32 rounding of
// sum_h x[t][h] * router[e][h]; every product of a bf16 and an fp32 value is
// exact in fp64 and the sum is accumulated in fp64, so the rounded logit
// does not depend on the summation order except in vanishingly rare cases.
// Ties in the top-K go to the lower expert id.
#include "device_common.h"
#include "kernels.h"
#include "router_gemv.h"

namespace moe {

// partial[s][t][e] = sum over h in [s*hs, (s+1)*hs) of x[t][h] * router[e][h],
// on fp64 MFMA (16x16x4): one wavefront per 64 tokens (16 for few tokens)
// x 64 experts of one split of H, 4 x 4 (1 x 4) output fragments of 16 x 16. Operands come straight from
// memory, 8 consecutive h per lane (16 bytes of x, 32 bytes of router) per
// 32-element block: lane group kk = lane / 16 owns h = 8kk .. 8kk+7 of the
// block and MFMA step s takes element 8kk + s, for both operands. The next
// block's loads are issued before the current block's MFMAs.
typedef __attribute__((ext_vector_type(4))) double f64x4;
// up to this T: 16 tokens per wavefront (against 64: the layer 10 us faster
// at T = 17-32, 8-11 us at T = 48-192, the same at T = 256 and 512)
constexpr int kRouterFewTokens = 192;

// XT: uint16_t (bf16 input: 16 bytes per lane and block) or float (the
// block's fp32 pre-norm output: 32 bytes); either times fp32 is exact in fp64.
// MF: token fragments of 16 per wavefront (4, or 1 for few tokens, so that
// the wavefronts' MFMA chains are a quarter as long and their count covers
// more of the GPU, and a 32-token call pads nothing).
template <typename XT, int MF>
__global__ __launch_bounds__(64) void router_mfma_kernel(
    const XT* __restrict__ x, const float* __restrict__ wr,
    double* __restrict__ partial, int T, int H, int E, int hs) {
  constexpr int XB = sizeof(XT);  // bytes per input element
  const int lane = threadIdx.x, i = lane & 15, kk = lane >> 4;
  const int t0 = blockIdx.x * 16 * MF, e0 = blockIdx.y * 64, sp = blockIdx.z;
  const int nt = min(16 * MF, T - t0), ne = min(64, E - e0);
  const rsrc_t x_r = make_rsrc(x + static_cast<size_t>(t0) * H, static_cast<uint32_t>(nt * H * XB));
  const rsrc_t w_r = make_rsrc(wr + static_cast<size_t>(e0) * H, static_cast<uint32_t>(ne * H * 4));
  const int hbeg = sp * hs;
  uint32_t xo[MF], wo[4];
#pragma unroll
  for (int m = 0; m < MF; ++m) {
    const int t = 16 * m + i;
    xo[m] = t < nt ? static_cast<uint32_t>((t * H + hbeg + kk * 8) * XB) : kOutOfRange;
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = 16 * n + i;
    wo[n] = e < ne ? static_cast<uint32_t>((e * H + hbeg + kk * 8) * 4) : kOutOfRange;
  }
  f64x4 acc[MF][4];
#pragma unroll
  for (int m = 0; m < MF; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f64x4{0.0, 0.0, 0.0, 0.0};

  uint4 xa[2][MF][XB / 2], wb[2][4][2];
  auto load = [&](int buf, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
      for (int q = 0; q < XB / 2; ++q) xa[buf][m][q] = buf_load16<kAuxDefault>(x_r, xo[m] + c * XB + q * 16);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      wb[buf][n][0] = buf_load16<kAuxDefault>(w_r, wo[n] + c * 4);
      wb[buf][n][1] = buf_load16<kAuxDefault>(w_r, wo[n] + c * 4 + 16);
    }
  };
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      double a[MF], b[4];
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        if constexpr (XB == 2) {
          const uint4 q = xa[buf][m][0];
          const uint32_t d = s < 2 ? q.x : s < 4 ? q.y : s < 6 ? q.z : q.w;
          a[m] = static_cast<double>(__uint_as_float((s & 1) ? (d & 0xFFFF0000u) : (d << 16)));
        } else {
          const uint4 q = xa[buf][m][s >> 2];
          const uint32_t d = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
          a[m] = static_cast<double>(__uint_as_float(d));
        }
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint4 q = wb[buf][n][s >> 2];
        const uint32_t d = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
        b[n] = static_cast<double>(__uint_as_float(d));
      }
#pragma unroll
      for (int m = 0; m < MF; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], b[n], acc[m][n], 0, 0, 0);
    }
  };
  load(0, 0);
  for (int c = 0; c < hs; c += 64) {
    load(1, min(c + 32, hs - 32));
    compute(0);
    if (c + 32 >= hs) break;
    load(0, min(c + 64, hs - 32));
    compute(1);
  }
  // D fragment layout of the fp64 16x16x4 MFMA: register r of a lane holds
  // row kk + 4 r (token), column i (expert)
#pragma unroll
  for (int m = 0; m < MF; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * m + kk + 4 * r;
      if (t >= nt) continue;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int e = 16 * n + i;
        if (e < ne) partial[(static_cast<size_t>(sp) * T + t0 + t) * E + e0 + e] = acc[m][n][r];
      }
    }
}

// One workgroup per token. The four wavefronts each add a quarter of the
// split partials (loads batched, sums in split order), wave 0 adds the four
// quarters in order and rounds to fp32, then runs K rounds of a wave-wide
// max over 64-bit rank keys (lane owns experts lane, lane+64, lane+128,
// lane+192). Weights: softmax over the selected logits in fp64, to fp32.
__global__ __launch_bounds__(256) void topk_kernel(
    const double* __restrict__ partial, int S, int T, int E, int K,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ double quarter[4][256];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x;
  const int s_beg = wave * S / 4, s_end = (wave + 1) * S / 4;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    double v = 0.0;
    if (e < E) {
      int s = s_beg;
      for (; s + 8 <= s_end; s += 8) {
        double p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = partial[(static_cast<size_t>(s + i) * T + t) * E + e];
#pragma unroll
        for (int i = 0; i < 8; ++i) v += p[i];
      }
      for (; s < s_end; ++s) v += partial[(static_cast<size_t>(s) * T + t) * E + e];
    }
    quarter[wave][lane + 64 * c] = v;
  }
  __syncthreads();
  if (wave != 0) return;
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    key[c] = 0;
    if (e < E) {
      const double v = ((quarter[0][e] + quarter[1][e]) + quarter[2][e]) + quarter[3][e];
      const float f = static_cast<float>(v);
      logits[static_cast<size_t>(t) * E + e] = f;
      key[c] = rank_key(f, e);
    }
  }
  wave_topk(key, K, lane, ids + static_cast<size_t>(t) * K, w + static_cast<size_t>(t) * K);
}


// Router logits for a few tokens (T <= 16) in one pass: one workgroup of
// four wavefronts per expert (router_gemv.h).
template <int TMAX, typename XT>
__global__ __launch_bounds__(256) void router_gemv_kernel(
    const XT* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ logits, int T, int H, int E) {
  __shared__ double part[4][TMAX];
  router_gemv_body<TMAX, 4, XT>(x, wr, logits, T, H, E, blockIdx.x, part);
}

template <typename XT>
hipError_t router_gemv(const XT* x, const float* wr, float* logits, int T, int H, int E,
                       hipStream_t st) {
  if (T <= 1)
    MOE_LAUNCH((router_gemv_kernel<1, XT>), dim3(E), dim3(256), 0, st, x, wr, logits, T, H, E);
  else if (T <= 4)
    MOE_LAUNCH((router_gemv_kernel<4, XT>), dim3(E), dim3(256), 0, st, x, wr, logits, T, H, E);
  else
    MOE_LAUNCH((router_gemv_kernel<16, XT>), dim3(E), dim3(256), 0, st, x, wr, logits, T, H, E);
  return hipGetLastError();
}

template <typename XT>
hipError_t router_logits(const XT* x, const float* wr, double* partial, int T, int H, int E,
                         int splits, hipStream_t st) {
  const int hs = H / splits;
  if (T <= kRouterFewTokens)
    MOE_LAUNCH((router_mfma_kernel<XT, 1>), dim3((T + 15) / 16, (E + 63) / 64, splits), dim3(64), 0,
               st, x, wr, partial, T, H, E, hs);
  else
    MOE_LAUNCH((router_mfma_kernel<XT, 4>), dim3((T + 63) / 64, (E + 63) / 64, splits), dim3(64), 0,
               st, x, wr, partial, T, H, E, hs);
  return hipGetLastError();
}

hipError_t launch_router_gemv(const uint16_t* x, const float* wr, float* logits, int T, int H,
                              int E, hipStream_t st) {
  return router_gemv(x, wr, logits, T, H, E, st);
}
hipError_t launch_router_logits(const uint16_t* x, const float* wr, double* partial, int T, int H,
                                int E, int splits, hipStream_t st) {
  return router_logits(x, wr, partial, T, H, E, splits, st);
}
hipError_t launch_router_logits(const float* x, const float* wr, double* partial, int T, int H,
                                int E, int splits, hipStream_t st) {
  return router_logits(x, wr, partial, T, H, E, splits, st);
}

hipError_t launch_topk(const double* partial, int S, int T, int E, int K, float* logits,
                       int32_t* ids, float* w, hipStream_t st) {
  MOE_LAUNCH((topk_kernel), dim3(T), dim3(256), 0, st, partial, S, T, E, K, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
