// combine.hip -- post-expert norm and router-weighted sum (step A7).
//
// "Muse Spark Open on Gaudi 2", section "The latent MoE: A' with a per-expert
// norm": post_expert_norm is applied to each full route row, the rows are
// multiplied by the router weights and summed in fp32; the section "EP and TP
// layout" adds that the norm must see the whole row (a norm of a partial sum
// is wrong). Norm: RMS over the L elements of the row, eps inside the square
// root, then the bf16 gain (one [L] vector, or the gain of the row's expert).
//
// One workgroup per token. Each route row (fp32, route-major) is read once:
// the thread keeps its slice of the row in registers while the block reduces
// the sum of squares, then adds w * s * gain * row into its slice of y. The
// routes are added in rank order k = 0..K-1; y is rounded once to bf16.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kMaxPerThread = 32;  // L <= 8192 with 256 threads

__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ rows, const float* __restrict__ w, const int32_t* __restrict__ ids,
    const uint16_t* __restrict__ gain, int gain_per_expert, float eps, int K, int L,
    uint16_t* __restrict__ y) {
  __shared__ float wave_ss[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[kMaxPerThread], v[kMaxPerThread];
#pragma unroll
  for (int i = 0; i < kMaxPerThread; ++i) acc[i] = 0.f;

  for (int k = 0; k < K; ++k) {
    const size_t r = static_cast<size_t>(t) * K + k;
    const float* row = rows + r * L;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerThread; ++i) {
      const int c = tid + 256 * i;
      v[i] = c < L ? row[c] : 0.f;
      ss += v[i] * v[i];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) wave_ss[wave] = ss;
    __syncthreads();
    const float tot = (wave_ss[0] + wave_ss[1]) + (wave_ss[2] + wave_ss[3]);
    __syncthreads();
    const float s = 1.0f / sqrtf(tot / static_cast<float>(L) + eps);
    const float ws = w[r] * s;
    const uint16_t* gr = gain + (gain_per_expert ? static_cast<size_t>(ids[r]) * L : 0);
#pragma unroll
    for (int i = 0; i < kMaxPerThread; ++i) {
      const int c = tid + 256 * i;
      if (c < L) acc[i] += ws * (v[i] * bf16_to_f32(gr[c]));
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxPerThread; ++i) {
    const int c = tid + 256 * i;
    if (c < L) y[static_cast<size_t>(t) * L + c] = f32_to_bf16(acc[i]);
  }
}
}  // namespace

hipError_t launch_combine(const float* rows, const float* w, const int32_t* ids,
                          const uint16_t* gain, int gain_per_expert, float eps, int T, int K,
                          int L, uint16_t* y, hipStream_t st) {
  combine_kernel<<<dim3(T), dim3(256), 0, st>>>(rows, w, ids, gain, gain_per_expert, eps, K, L, y);
  return hipGetLastError();
}

}  // namespace moe
