// peaks.hip -- measured ceilings of the MI355X that the benchmark prices the
// layer's kernels against, beside the vendor figures: the HBM bandwidth one
// streaming kernel reaches (a copy, and a read-only reduction), and the bf16
// MFMA issue rate of register-resident operands. Measurement only: the layer
// (libmoe.so) neither links nor calls this library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_peaks.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// dst = src, 16 bytes per lane per step, grid-stride
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

// xor of every 16-byte word (reads n16 * 16 bytes), one word per workgroup out
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {  // four loads in flight per lane
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int t = 0; t < 256; ++t) v ^= red[t];
    sink[blockIdx.x] = v;
  }
}

// Eight independent chains of bf16 MFMA 16x16x32 per wavefront (enough to
// cover the instruction's latency), operands in registers; the sums are
// written out so that nothing is removed.
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * static_cast<float>((lane + i) & 7));
    b[i] = static_cast<__bf16>(0.002f * static_cast<float>((lane * 3 + i) & 7));
  }
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -static_cast<int>(e) - 1000; }

}  // namespace

extern "C" {

int moe_peak_copy(const void* src, void* dst, size_t bytes, int workgroups, void* stream) {
  if (!src || !dst || bytes % 16 || workgroups <= 0) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return status(hipGetLastError());
}

int moe_peak_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  if (!src || !sink || bytes % 16 || workgroups <= 0) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return status(hipGetLastError());
}

int moe_peak_mfma_bf16(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return status(hipGetLastError());
}

double moe_peak_mfma_bf16_flops(int workgroups, int iters) {
  // 4 wavefronts per workgroup, 8 MFMAs per iteration, 2*16*16*32 flops each
  return 4.0 * workgroups * iters * 8.0 * 2.0 * 16 * 16 * 32;
}

}  // extern "C"
