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

namespace moe {

// partial[s][t][e] = sum over h in [s*hs, (s+1)*hs) of x[t][h] * router[e][h].
// Block: TT tokens x 64 experts x one split of H; 256 threads, each holding
// an RT x RE block of fp64 accumulators; 32-wide h chunks staged in LDS.
template <int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr,
    double* __restrict__ partial, int T, int H, int E, int hs) {
  constexpr int RT = TT >= 64 ? 4 : 1;
  constexpr int RE = TT >= 16 ? 4 : 1;
  constexpr int NE = 64 / RE;
  static_assert((TT / RT) * NE == 256, "thread layout");
  __shared__ double xs[32][TT + 1];
  __shared__ double ws[32][64 + 1];

  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * 64, s = blockIdx.z;
  const int tid = threadIdx.x, ti = tid / NE, ej = tid % NE;
  double acc[RT][RE];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < RE; ++b) acc[a][b] = 0.0;

  const int hbeg = s * hs, hend = hbeg + hs;
  for (int hc = hbeg; hc < hend; hc += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      const int e = i >> 5, h = i & 31;
      ws[h][e] = (e0 + e < E) ? static_cast<double>(wr[static_cast<size_t>(e0 + e) * H + hc + h]) : 0.0;
    }
    for (int i = tid; i < TT * 32; i += 256) {
      const int t = i >> 5, h = i & 31;
      xs[h][t] = (t0 + t < T) ? static_cast<double>(bf16_to_f32(x[static_cast<size_t>(t0 + t) * H + hc + h])) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int h = 0; h < 32; ++h) {
      double xv[RT], wv[RE];
#pragma unroll
      for (int a = 0; a < RT; ++a) xv[a] = xs[h][ti * RT + a];
#pragma unroll
      for (int b = 0; b < RE; ++b) wv[b] = ws[h][ej + NE * b];
#pragma unroll
      for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b = 0; b < RE; ++b) acc[a][b] = __builtin_fma(xv[a], wv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < RT; ++a) {
    const int t = t0 + ti * RT + a;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < RE; ++b) {
      const int e = e0 + ej + NE * b;
      if (e < E) partial[(static_cast<size_t>(s) * T + t) * E + e] = acc[a][b];
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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


// Router logits for a few tokens (T <= 16) in one pass: one workgroup per
// expert, its four wavefronts each take a quarter of H. Each lane issues all
// of its router loads (16 bytes each) and activation loads first, then
// accumulates in fp64; lanes reduce across the wavefront, the wavefronts in
// order through LDS, and the sum is rounded once to fp32.
template <int TMAX>
__global__ __launch_bounds__(256) void router_gemv_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ logits, int T, int H, int E) {
  constexpr int NV = TMAX == 1 ? 8 : (TMAX <= 4 ? 4 : 2);  // 16-byte router loads per lane per pass
  __shared__ double part[4][TMAX];
  const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = H / 4, h0 = wave * hq;
  double acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
  const float* row = wr + static_cast<size_t>(e) * H;
  for (int hp = 0; hp < hq; hp += NV * 256) {
    float4 wv[NV];
    uint2 xv[NV][TMAX];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int h = h0 + hp + u * 256 + lane * 4;
      const bool ok = hp + u * 256 + lane * 4 < hq;
      wv[u] = ok ? *reinterpret_cast<const float4*>(row + h) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < TMAX; ++t)
        xv[u][t] = (ok && t < T) ? *reinterpret_cast<const uint2*>(x + static_cast<size_t>(t) * H + h) : uint2{0, 0};
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        acc[t] = __builtin_fma(static_cast<double>(__uint_as_float(xv[u][t].x << 16)), static_cast<double>(wv[u].x), acc[t]);
        acc[t] = __builtin_fma(static_cast<double>(__uint_as_float(xv[u][t].x & 0xFFFF0000u)), static_cast<double>(wv[u].y), acc[t]);
        acc[t] = __builtin_fma(static_cast<double>(__uint_as_float(xv[u][t].y << 16)), static_cast<double>(wv[u].z), acc[t]);
        acc[t] = __builtin_fma(static_cast<double>(__uint_as_float(xv[u][t].y & 0xFFFF0000u)), static_cast<double>(wv[u].w), acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    double v = acc[t];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0) part[wave][t] = v;
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < T) {
    const int t = threadIdx.x;
    const double v = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    logits[static_cast<size_t>(t) * E + e] = static_cast<float>(v);
  }
}

hipError_t launch_router_gemv(const uint16_t* x, const float* wr, float* logits, int T, int H,
                              int E, hipStream_t st) {
  if (T <= 1)
    MOE_LAUNCH((router_gemv_kernel<1>), dim3(E), dim3(256), 0, st, x, wr, logits, T, H, E);
  else if (T <= 4)
    MOE_LAUNCH((router_gemv_kernel<4>), dim3(E), dim3(256), 0, st, x, wr, logits, T, H, E);
  else
    MOE_LAUNCH((router_gemv_kernel<16>), dim3(E), dim3(256), 0, st, x, wr, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, double* partial,
                                int T, int H, int E, int tt, int splits, hipStream_t st) {
  const int hs = H / splits;
  const dim3 block(256);
  const int ne = (E + 63) / 64;
  if (tt == 4) {
    MOE_LAUNCH((router_logits_kernel<4>), dim3((T + 3) / 4, ne, splits), block, 0, st, x, wr, partial, T, H, E, hs);
  } else if (tt == 16) {
    MOE_LAUNCH((router_logits_kernel<16>), dim3((T + 15) / 16, ne, splits), block, 0, st, x, wr, partial, T, H, E, hs);
  } else {
    MOE_LAUNCH((router_logits_kernel<64>), dim3((T + 63) / 64, ne, splits), block, 0, st, x, wr, partial, T, H, E, hs);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const double* partial, int S, int T, int E, int K, float* logits,
                       int32_t* ids, float* w, hipStream_t st) {
  MOE_LAUNCH((topk_kernel), dim3(T), dim3(256), 0, st, partial, S, T, E, K, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
