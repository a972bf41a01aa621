// combine_cols.h -- post-expert norm and router-weighted sum (step A7) for
// few tokens, one column block of one token per workgroup.
//
// "Muse Spark Open on Gaudi 2", section "The latent MoE: A' with a per-expert
// norm": the RMS norm over each full route row, then the router weight and
// the fp32 sum over the routes (k ascending), y rounded once to bf16. The
// norm's sum of squares comes from the per-32-column partial sums the down
// projection wrote (added in column order), so a workgroup reads no column
// beyond its own. Shared by the per-step launch (combine.hip) and the
// persistent decode layer (COH: the rows, partial sums and routing written
// by other workgroups of the launch, and y, go through device-coherent
// accesses).
#pragma once
#include "device_common.h"

namespace moe {

// Workgroup of blockDim.x threads: columns cb * blockDim.x + tid of token t.
template <int GPE, bool COH>
__device__ __forceinline__ void combine_cols_body(const float* __restrict__ rows,
                                                  const float* __restrict__ ssp,
                                                  const float* __restrict__ w,
                                                  const int32_t* __restrict__ ids,
                                                  const uint16_t* __restrict__ gain, float eps,
                                                  int K, int L, uint16_t* __restrict__ y, int cb,
                                                  int t) {
  __shared__ float scale[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = static_cast<int>(blockDim.x) >> 6;
  const int c = cb * static_cast<int>(blockDim.x) + tid;
  const int nb = L / 32;
  float v[8], gk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const size_t r = static_cast<size_t>(t) * K + k;
    v[k] = (k < K && c < L) ? ld_f32<COH>(rows + r * L + c) : 0.f;
    gk[k] = 0.f;
    if (GPE || k == 0) {
      const int e = (GPE && k < K) ? ld_i32<COH>(ids + r) : 0;
      gk[k] = (k < K && c < L) ? bf16_to_f32(gain[static_cast<size_t>(e) * L + c]) : 0.f;
    }
  }
  // wave q computes the scales of routes q, q + nwaves, ...
  for (int k = wave; k < K; k += nwaves) {
    const size_t r = static_cast<size_t>(t) * K + k;
    float q = 0.f;
    for (int j = lane; j < nb; j += 64) q += ld_f32<COH>(ssp + r * nb + j);
    const float ss = wave_sum_f32(q);
    if (lane == 0) scale[k] = ld_f32<COH>(w + r) * (1.0f / sqrtf(ss / static_cast<float>(L) + eps));
  }
  __syncthreads();
  if (c < L) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < K) acc += scale[k] * (v[k] * gk[GPE ? k : 0]);
    st_val<COH>(y + static_cast<size_t>(t) * L + c, f32_to_bf16(acc));
  }
  __syncthreads();  // (scale is rewritten by the workgroup's next item)
}

}  // namespace moe
