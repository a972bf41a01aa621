// router_gemv.h -- router logits for a few tokens in one pass (step A1).
//
// "Muse Spark Open on Gaudi 2", section "What was built": an fp32 router over
// 256 experts. Each logit is the fp32 rounding of the fp64 sum of the exact
// products x[t][h] * router[e][h].
//
// The input is bf16 (the layer's input) or fp32 (the block's pre-norm
// output); products of an fp32 router weight with either are exact in fp64.
// One workgroup of NW wavefronts per expert, each wavefront taking H / NW
// consecutive h. Each lane issues all of its router loads (16 bytes each)
// and activation loads first, then accumulates in fp64; lanes reduce across
// the wavefront, the wavefronts in order through LDS (part[NW][TMAX]), and
// the sum is rounded once to fp32. Shared by the stand-alone router launch
// and the launch that runs it beside the pooler (which may also store each
// logit tagged with its call's tag, for the routing done in that launch).
#pragma once
#include "device_common.h"

namespace moe {

// four consecutive inputs as stored (bf16: two words; fp32: four), and
// element j of them widened exactly to fp64
template <typename XT> struct X4;
template <> struct X4<uint16_t> {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { v = uint2{0u, 0u}; }
  __device__ __forceinline__ double get(int j) const {
    const uint32_t d = j < 2 ? v.x : v.y;
    return static_cast<double>(__uint_as_float((j & 1) ? (d & 0xFFFF0000u) : (d << 16)));
  }
};
template <> struct X4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void zero() { v = float4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ double get(int j) const {
    return static_cast<double>(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w);
  }
};

// XT: uint16_t (bf16 input) or float (the fp32 output of the block's pre-norm)
template <int TMAX, int NW, typename XT = uint16_t>
__device__ __forceinline__ void router_gemv_body(const XT* __restrict__ x,
                                                 const float* __restrict__ wr,
                                                 float* __restrict__ logits, int T, int H, int E,
                                                 int e, double (*part)[TMAX],
                                                 uint64_t* __restrict__ tagged = nullptr,
                                                 uint32_t tag = 0) {
  // 16-byte router loads per lane per pass (halved for fp32 inputs, whose
  // four values per load take twice the registers of bf16 ones)
  constexpr int NV0 = TMAX == 1 ? 8 : (TMAX <= 4 ? 4 : 2);
  constexpr int NV = sizeof(XT) == 4 && NV0 > 1 ? NV0 / 2 : NV0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = H / NW, h0 = wave * hq;
  double acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
  const float* row = wr + static_cast<size_t>(e) * H;
  for (int hp = 0; hp < hq; hp += NV * 256) {
    float4 wv[NV];
    X4<XT> xv[NV][TMAX];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int h = h0 + hp + u * 256 + lane * 4;
      const bool ok = hp + u * 256 + lane * 4 < hq;
      wv[u] = ok ? *reinterpret_cast<const float4*>(row + h) : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (ok && t < T)
          xv[u][t].load(x + static_cast<size_t>(t) * H + h);
        else
          xv[u][t].zero();
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        acc[t] = __builtin_fma(xv[u][t].get(0), static_cast<double>(wv[u].x), acc[t]);
        acc[t] = __builtin_fma(xv[u][t].get(1), static_cast<double>(wv[u].y), acc[t]);
        acc[t] = __builtin_fma(xv[u][t].get(2), static_cast<double>(wv[u].z), acc[t]);
        acc[t] = __builtin_fma(xv[u][t].get(3), static_cast<double>(wv[u].w), acc[t]);
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
    const float lv = static_cast<float>(v);
    logits[static_cast<size_t>(t) * E + e] = lv;
    if (tagged)
      __hip_atomic_store(tagged + static_cast<size_t>(t) * E + e,
                         (static_cast<uint64_t>(tag) << 32) | __float_as_uint(lv), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The block's pre-norm folded into the router (few tokens): x is the bf16
// residual stream and the router's input is n = fp32(x * s * g), s =
// 1/sqrt(mean(x^2) + eps), computed here exactly as the pre-norm kernel does
// (fp64 sum of squares, exact whatever its order; fp64 scale and products;
// one rounding to fp32). A first pass over each token's row gives s, the
// second takes the dot products with n formed on the fly. Workgroup
// `write_views` also stores n as fp32 and as bf16 (the pre-norm's outputs).
template <int TMAX, int NW>
__device__ __forceinline__ void router_prenorm_body(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ gain, double eps,
                                                    const float* __restrict__ wr,
                                                    float* __restrict__ logits, int T, int H, int E,
                                                    int e, double (*part)[TMAX],
                                                    uint64_t* __restrict__ tagged, uint32_t tag,
                                                    float* __restrict__ nf32_out,
                                                    uint16_t* __restrict__ nbf16_out) {
  constexpr int NV = TMAX == 1 ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // ---- pass 1: each token's scale ----
  double ss[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    ss[t] = 0.0;
    if (t < T) {
      for (int h = threadIdx.x * 8; h < H; h += NW * 64 * 8) {
        const uint4 q = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + h);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double a = bf16_bits_to_f64(w[j] & 0xFFFFu), b = bf16_bits_to_f64(w[j] >> 16);
          ss[t] += a * a;
          ss[t] += b * b;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    double v = ss[t];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0) part[wave][t] = v;
  }
  __syncthreads();
  double s[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += part[w][t];
    s[t] = 1.0 / sqrt(v / static_cast<double>(H) + eps);
  }
  __syncthreads();
  // ---- pass 2: logits over n = fp32(x * s * g) ----
  const int hq = H / NW, h0 = wave * hq;
  double acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0;
  const float* row = wr + static_cast<size_t>(e) * H;
  const bool views = nf32_out != nullptr;
  for (int hp = 0; hp < hq; hp += NV * 256) {
    float4 wv[NV];
    uint2 gv[NV];
    uint2 xv[NV][TMAX];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int h = h0 + hp + u * 256 + lane * 4;
      const bool ok = hp + u * 256 + lane * 4 < hq;
      wv[u] = ok ? *reinterpret_cast<const float4*>(row + h) : float4{0.f, 0.f, 0.f, 0.f};
      gv[u] = ok ? *reinterpret_cast<const uint2*>(gain + h) : uint2{0u, 0u};
#pragma unroll
      for (int t = 0; t < TMAX; ++t)
        xv[u][t] = (ok && t < T) ? *reinterpret_cast<const uint2*>(x + static_cast<size_t>(t) * H + h)
                                 : uint2{0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int h = h0 + hp + u * 256 + lane * 4;
      const bool ok = hp + u * 256 + lane * 4 < hq;
      const double g[4] = {bf16_bits_to_f64(gv[u].x & 0xFFFFu), bf16_bits_to_f64(gv[u].x >> 16),
                           bf16_bits_to_f64(gv[u].y & 0xFFFFu), bf16_bits_to_f64(gv[u].y >> 16)};
      const double wd[4] = {static_cast<double>(wv[u].x), static_cast<double>(wv[u].y),
                            static_cast<double>(wv[u].z), static_cast<double>(wv[u].w)};
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        const double xd[4] = {bf16_bits_to_f64(xv[u][t].x & 0xFFFFu), bf16_bits_to_f64(xv[u][t].x >> 16),
                              bf16_bits_to_f64(xv[u][t].y & 0xFFFFu), bf16_bits_to_f64(xv[u][t].y >> 16)};
        float nf[4];
        uint16_t nb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double n = xd[j] * s[t] * g[j];
          nf[j] = static_cast<float>(n);
          nb[j] = f64_to_bf16(n);
          acc[t] = __builtin_fma(static_cast<double>(nf[j]), wd[j], acc[t]);
        }
        if (views && ok && t < T) {
          *reinterpret_cast<float4*>(nf32_out + static_cast<size_t>(t) * H + h) =
              float4{nf[0], nf[1], nf[2], nf[3]};
          *reinterpret_cast<uint2*>(nbf16_out + static_cast<size_t>(t) * H + h) =
              uint2{nb[0] | (static_cast<uint32_t>(nb[1]) << 16), nb[2] | (static_cast<uint32_t>(nb[3]) << 16)};
        }
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
    const float lv = static_cast<float>(v);
    logits[static_cast<size_t>(t) * E + e] = lv;
    if (tagged)
      __hip_atomic_store(tagged + static_cast<size_t>(t) * E + e,
                         (static_cast<uint64_t>(tag) << 32) | __float_as_uint(lv), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace moe
