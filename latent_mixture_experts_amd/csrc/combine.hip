// combine.hip -- post-expert norm and router-weighted sum (step A7).
//
// "Muse Spark Open on Gaudi 2", section "The latent MoE: A' with a per-expert
// norm": post_expert_norm is applied to each full route row, the rows are
// multiplied by the router weights and summed in fp32; the section "EP and TP
// layout" adds that the norm must see the whole row (a norm of a partial sum
// is wrong). Norm: RMS over the L elements of the row, eps inside the square
// root, then the bf16 gain (one [L] vector, or the gain of the row's expert).
//
// Each route row (fp32, route-major) is read once. The routes are added in
// rank order k = 0..K-1 and y is rounded once to bf16.
#include "combine_cols.h"
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kThreads = 1024;

// One workgroup of 1024 threads per token; thread i holds columns
// 4(i + 1024j) .. +3 of every route row (16-byte loads, NV chunks: L <= 4096
// NV). All K route rows are loaded at once, the K sums of squares are reduced
// together (thread, wavefront, then the wavefronts in order), then
// y = sum_k w_k * s_k * gain * row_k. KT: max routes per token; GPE: one gain
// row per expert.
template <int KT, int NV, int GPE>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ rows, const float* __restrict__ w, const int32_t* __restrict__ ids,
    const uint16_t* __restrict__ gain, int gain_per_expert, float eps, int K, int L,
    uint16_t* __restrict__ y) {
  __shared__ float wave_ss[kThreads / 64][KT];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // every global load is issued before the first use: rows, weights, gains
  constexpr int NG = GPE ? KT : 1;
  float4 v[KT][NV];
  float wk[KT];
  uint2 gk[NG][NV];
  int32_t ek[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const size_t r = static_cast<size_t>(t) * K + k;
    wk[k] = k < K ? w[r] : 0.f;
    ek[k] = (k < K && GPE) ? ids[r] : 0;
    const float* row = rows + r * L;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = 4 * (tid + kThreads * j);
      v[k][j] = (k < K && c < L) ? *reinterpret_cast<const float4*>(row + c) : float4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const uint16_t* gr = gain + static_cast<size_t>(ek[k]) * L;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = 4 * (tid + kThreads * j);
      gk[k][j] = c < L ? *reinterpret_cast<const uint2*>(gr + c) : uint2{0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      ss += v[k][j].x * v[k][j].x + v[k][j].y * v[k][j].y + v[k][j].z * v[k][j].z + v[k][j].w * v[k][j].w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) wave_ss[wave][k] = ss;
  }
  __syncthreads();
  float4 acc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) acc[j] = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    if (k >= K) break;
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < kThreads / 64; ++q) tot += wave_ss[q][k];
    const float ws = wk[k] * (1.0f / sqrtf(tot / static_cast<float>(L) + eps));
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint2 g = gk[GPE ? k : 0][j];
      acc[j].x += ws * (v[k][j].x * bf16_to_f32(static_cast<uint16_t>(g.x)));
      acc[j].y += ws * (v[k][j].y * bf16_to_f32(static_cast<uint16_t>(g.x >> 16)));
      acc[j].z += ws * (v[k][j].z * bf16_to_f32(static_cast<uint16_t>(g.y)));
      acc[j].w += ws * (v[k][j].w * bf16_to_f32(static_cast<uint16_t>(g.y >> 16)));
    }
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = 4 * (tid + kThreads * j);
    if (c < L) {
      const uint32_t lo = f32_to_bf16(acc[j].x) | (static_cast<uint32_t>(f32_to_bf16(acc[j].y)) << 16);
      const uint32_t hi = f32_to_bf16(acc[j].z) | (static_cast<uint32_t>(f32_to_bf16(acc[j].w)) << 16);
      *reinterpret_cast<uint2*>(y + static_cast<size_t>(t) * L + c) = uint2{lo, hi};
    }
  }
}
// Few tokens: workgroup (column block of 256, token); combine_cols.h.
template <int GPE>
__global__ __launch_bounds__(256) void combine_cols_kernel(
    const float* __restrict__ rows, const float* __restrict__ ssp, const float* __restrict__ w,
    const int32_t* __restrict__ ids, const uint16_t* __restrict__ gain, float eps, int K, int L,
    uint16_t* __restrict__ y) {
  combine_cols_body<GPE, false>(rows, ssp, w, ids, gain, eps, K, L, y, blockIdx.x, blockIdx.y);
}
}  // namespace

hipError_t launch_combine_cols(const float* rows, const float* ssp, const float* w,
                               const int32_t* ids, const uint16_t* gain, int gain_per_expert,
                               float eps, int T, int K, int L, uint16_t* y, hipStream_t st) {
  const dim3 grid((L + 255) / 256, T), block(256);
  if (gain_per_expert)
    MOE_LAUNCH((combine_cols_kernel<1>), grid, block, 0, st, rows, ssp, w, ids, gain, eps, K, L, y);
  else
    MOE_LAUNCH((combine_cols_kernel<0>), grid, block, 0, st, rows, ssp, w, ids, gain, eps, K, L, y);
  return hipGetLastError();
}

hipError_t launch_combine(const float* rows, const float* w, const int32_t* ids,
                          const uint16_t* gain, int gain_per_expert, float eps, int T, int K,
                          int L, uint16_t* y, hipStream_t st) {
  const dim3 grid(T), block(kThreads);
#define MOE_COMBINE(KT_, NV_, G_) MOE_LAUNCH((combine_kernel<KT_, NV_, G_>), grid, block, 0, st, rows, w, ids, gain, gain_per_expert, eps, K, L, y)
#define MOE_COMBINE_C(KT_, G_)                     \
  if (L <= 4 * kThreads) MOE_COMBINE(KT_, 1, G_); \
  else MOE_COMBINE(KT_, 2, G_);
  if (K <= 4) {
    if (gain_per_expert) { MOE_COMBINE_C(4, 1) } else { MOE_COMBINE_C(4, 0) }
  } else {
    if (gain_per_expert) { MOE_COMBINE_C(8, 1) } else { MOE_COMBINE_C(8, 0) }
  }
#undef MOE_COMBINE_C
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
