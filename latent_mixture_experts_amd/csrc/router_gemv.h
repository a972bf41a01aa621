// router_gemv.h -- router logits for a few tokens in one pass (step A1).
//
// "Muse Spark Open on Gaudi 2", section "What was built": an fp32 router over
// 256 experts. Each logit is the fp32 rounding of the fp64 sum of the exact
// products x[t][h] * router[e][h].
//
// One workgroup of NW wavefronts per expert, each wavefront taking H / NW
// consecutive h. Each lane issues all of its router loads (16 bytes each)
// and activation loads first, then accumulates in fp64; lanes reduce across
// the wavefront, the wavefronts in order through LDS (part[NW][TMAX]), and
// the sum is rounded once to fp32. Shared by the stand-alone router launch
// and the launch that runs it beside the pooler.
#pragma once
#include "device_common.h"

namespace moe {

template <int TMAX, int NW>
__device__ __forceinline__ void router_gemv_body(const uint16_t* __restrict__ x,
                                                 const float* __restrict__ wr,
                                                 float* __restrict__ logits, int T, int H, int E,
                                                 int e, double (*part)[TMAX]) {
  constexpr int NV = TMAX == 1 ? 8 : (TMAX <= 4 ? 4 : 2);  // 16-byte router loads per lane per pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = H / NW, h0 = wave * hq;
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
    double v = part[0][t];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += part[w][t];
    logits[static_cast<size_t>(t) * E + e] = static_cast<float>(v);
  }
}

}  // namespace moe
