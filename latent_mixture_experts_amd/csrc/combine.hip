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
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kThreads = 1024;

// One workgroup of 1024 threads per token. All K route rows are loaded at
// once (each thread keeps its columns of every row in registers), the K sums
// of squares are reduced together, then y = sum_k w_k * s_k * gain * row_k.
// KT: max routes per token; kCols: columns per thread (L <= 1024 * kCols);
// GPE: one gain row per expert.
template <int KT, int kCols, int GPE>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ rows, const float* __restrict__ w, const int32_t* __restrict__ ids,
    const uint16_t* __restrict__ gain, int gain_per_expert, float eps, int K, int L,
    uint16_t* __restrict__ y) {
  __shared__ float wave_ss[kThreads / 64][KT];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // every global load is issued before the first use: rows, weights, gains
  constexpr int NG = GPE ? KT : 1;
  float v[KT][kCols], wk[KT], gk[NG][kCols];
  int32_t ek[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const size_t r = static_cast<size_t>(t) * K + k;
    wk[k] = k < K ? w[r] : 0.f;
    ek[k] = (k < K && GPE) ? ids[r] : 0;
    const float* row = rows + r * L;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      const int c = tid + kThreads * i;
      v[k][i] = (k < K && c < L) ? row[c] : 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const uint16_t* gr = gain + static_cast<size_t>(ek[k]) * L;
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      const int c = tid + kThreads * i;
      gk[k][i] = c < L ? bf16_to_f32(gr[c]) : 0.f;
    }
  }
  float ss[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    ss[k] = 0.f;
#pragma unroll
    for (int i = 0; i < kCols; ++i) ss[k] += v[k][i] * v[k][i];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss[k] += __shfl_xor(ss[k], m, 64);
    if (lane == 0) wave_ss[wave][k] = ss[k];
  }
  __syncthreads();
  float acc[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) acc[i] = 0.f;
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    if (k >= K) break;
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < kThreads / 64; ++q) tot += wave_ss[q][k];
    const float ws = wk[k] * (1.0f / sqrtf(tot / static_cast<float>(L) + eps));
#pragma unroll
    for (int i = 0; i < kCols; ++i) acc[i] += ws * (v[k][i] * gk[GPE ? k : 0][i]);
  }
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    const int c = tid + kThreads * i;
    if (c < L) y[static_cast<size_t>(t) * L + c] = f32_to_bf16(acc[i]);
  }
}
// Few tokens: workgroup (column block of 256, token). The norm scale of each
// route comes from the per-32-column partial sums of squares written by the
// down projection (added in column order), so the workgroups need no row
// beyond their own columns.
template <int GPE>
__global__ __launch_bounds__(256) void combine_cols_kernel(
    const float* __restrict__ rows, const float* __restrict__ ssp, const float* __restrict__ w,
    const int32_t* __restrict__ ids, const uint16_t* __restrict__ gain, float eps, int K, int L,
    uint16_t* __restrict__ y) {
  __shared__ float scale[8];
  const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x * 256 + tid;
  const int nb = L / 32;
  float v[8], gk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const size_t r = static_cast<size_t>(t) * K + k;
    v[k] = (k < K && c < L) ? rows[r * L + c] : 0.f;
    gk[k] = 0.f;
    if (GPE || k == 0) {
      const int e = (GPE && k < K) ? ids[r] : 0;
      gk[k] = (k < K && c < L) ? bf16_to_f32(gain[static_cast<size_t>(e) * L + c]) : 0.f;
    }
  }
  // wave q computes the scale of routes q and q + 4
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = wave + 4 * h;
    if (k < K) {
      const size_t r = static_cast<size_t>(t) * K + k;
      float q = 0.f;
      for (int j = lane; j < nb; j += 64) q += ssp[r * nb + j];
      const float ss = wave_sum_f32(q);
      if (lane == 0) scale[k] = w[r] * (1.0f / sqrtf(ss / static_cast<float>(L) + eps));
    }
  }
  __syncthreads();
  if (c >= L) return;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < K) acc += scale[k] * (v[k] * gk[GPE ? k : 0]);
  y[static_cast<size_t>(t) * L + c] = f32_to_bf16(acc);
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
  const int cpt = (L + kThreads - 1) / kThreads;
#define MOE_COMBINE(KT_, C_, G_) MOE_LAUNCH((combine_kernel<KT_, C_, G_>), grid, block, 0, st, rows, w, ids, gain, gain_per_expert, eps, K, L, y)
#define MOE_COMBINE_C(KT_, G_)    \
  if (cpt <= 1) MOE_COMBINE(KT_, 1, G_); \
  else if (cpt <= 2) MOE_COMBINE(KT_, 2, G_); \
  else if (cpt <= 4) MOE_COMBINE(KT_, 4, G_); \
  else MOE_COMBINE(KT_, 8, G_);
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
