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

// Order key: larger value ranks first, NaN after every number, -0 == +0,
// equal values by lower id. 0 is reserved for "not selectable".
__device__ __forceinline__ uint64_t rank_key(float f, int e) {
  uint32_t ok;
  if (f != f) {
    ok = 0;
  } else {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    ok = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(ok + 1u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ok = static_cast<uint32_t>(key >> 32) - 1u;
  if (ok == 0) return __uint_as_float(0x7FC00000u);
  const uint32_t u = (ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok;
  return __uint_as_float(u);
}

// One wavefront per token: sum the split partials in split order, round to
// fp32, then K rounds of a wave-wide max over 64-bit rank keys (each lane
// owns experts lane, lane+64, lane+128, lane+192). Weights: softmax over the
// selected logits in fp64, rounded to fp32.
__global__ __launch_bounds__(256) void topk_kernel(
    const double* __restrict__ partial, int S, int T, int E, int K,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    key[c] = 0;
    if (e < E) {
      double v = 0.0;
      for (int s = 0; s < S; ++s) v += partial[(static_cast<size_t>(s) * T + t) * E + e];
      const float f = static_cast<float>(v);
      logits[static_cast<size_t>(t) * E + e] = f;
      key[c] = rank_key(f, e);
    }
  }
  uint64_t sel[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sel[k] = 0;
    if (k < K) {
      uint64_t best = key[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) best = key[c] > best ? key[c] : best;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = wave_shfl_xor(best, m);
        best = o > best ? o : best;
      }
      const int e = static_cast<int>(~static_cast<uint32_t>(best));
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (lane + 64 * c == e) key[c] = 0;
      sel[k] = best;
    }
  }
  if (lane == 0) {
    const double m = static_cast<double>(key_value(sel[0]));
    double a[8], sum = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K) {
        a[k] = exp(static_cast<double>(key_value(sel[k])) - m);
        sum += a[k];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K) {
        ids[static_cast<size_t>(t) * K + k] = static_cast<int32_t>(~static_cast<uint32_t>(sel[k]));
        w[static_cast<size_t>(t) * K + k] = static_cast<float>(a[k] / sum);
      }
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, double* partial,
                                int T, int H, int E, int tt, int splits, hipStream_t st) {
  const int hs = H / splits;
  const dim3 block(256);
  const int ne = (E + 63) / 64;
  if (tt == 4) {
    router_logits_kernel<4><<<dim3((T + 3) / 4, ne, splits), block, 0, st>>>(x, wr, partial, T, H, E, hs);
  } else if (tt == 16) {
    router_logits_kernel<16><<<dim3((T + 15) / 16, ne, splits), block, 0, st>>>(x, wr, partial, T, H, E, hs);
  } else {
    router_logits_kernel<64><<<dim3((T + 63) / 64, ne, splits), block, 0, st>>>(x, wr, partial, T, H, E, hs);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const double* partial, int S, int T, int E, int K, float* logits,
                       int32_t* ids, float* w, hipStream_t st) {
  topk_kernel<<<dim3((T + 3) / 4), dim3(256), 0, st>>>(partial, S, T, E, K, logits, ids, w);
  return hipGetLastError();
}

}  // namespace moe
