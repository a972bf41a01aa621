// block.hip -- the steps around the layer: the sandwich norms and the residual.
//
// "Soporte de día 0 para Muse Spark Open en vLLM", section "Arquitectura del
// modelo", paragraph on the sandwich norm: a norm before the block and one
// after it, out = x + post_norm(F(norm(x))); section "Nvidia": the router is
// fed by the norm's fp32 output. Both norms are RMS norms over the H-wide row
// with a bf16 gain [H].
//
// One workgroup per token, BT threads; each thread holds 8 consecutive
// elements per 8*BT-element pass. Few tokens: 1024 threads (at T = 1 the
// step is one workgroup and its time the latency of its passes: the block
// at T = 1 107.8 -> 100.2 us); many tokens: 256 (1024 measured slower at
// T = 4096). The sum of squares of bf16 values is taken
// in fp64 (every square is exact; for rows whose squares span less than
// about 2^24 in magnitude the sum is exact whatever its order), the scale
// 1/sqrt(ss/H + eps) in fp64 with IEEE square root and division, and each
// element v*s*g in fp64: the fp32 router input then equals the fp32 rounding
// of the exact formula, which keeps the routing reproducible. bf16 results
// are rounded once from fp64: to fp32 with round-to-odd, then to bf16 with
// round-to-nearest-even (two rounding steps that give the correct single
// rounding because fp32 keeps more than two extra bits).
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kFewTokens = 256;  // up to this T: 1024 threads per token

// sum over the workgroup (fp64), same value in every thread
template <int kBT>
__device__ double block_sum(double v, double* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kBT / 64; ++w) s += lds[w];
  __syncthreads();
  return s;
}

template <int kBT>
__global__ __launch_bounds__(kBT) void pre_norm_kernel(const uint16_t* __restrict__ resid,
                                                      const uint16_t* __restrict__ gain, double eps,
                                                      int H, float* __restrict__ n_f32,
                                                      uint16_t* __restrict__ n_bf16) {
  __shared__ double lds[kBT / 64];
  const size_t row = static_cast<size_t>(blockIdx.x) * H;
  double ss = 0.0;
  for (int h = threadIdx.x * 8; h < H; h += kBT * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(resid + row + h);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = bf16_bits_to_f64(w[j] & 0xFFFFu), b = bf16_bits_to_f64(w[j] >> 16);
      ss += a * a;
      ss += b * b;
    }
  }
  ss = block_sum<kBT>(ss, lds);
  const double s = 1.0 / sqrt(ss / static_cast<double>(H) + eps);
  for (int h = threadIdx.x * 8; h < H; h += kBT * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(resid + row + h);
    const uint4 gq = *reinterpret_cast<const uint4*>(gain + h);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w}, g[4] = {gq.x, gq.y, gq.z, gq.w};
    float nf[8];
    uint32_t nb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double n0 = bf16_bits_to_f64(w[j] & 0xFFFFu) * s * bf16_bits_to_f64(g[j] & 0xFFFFu);
      const double n1 = bf16_bits_to_f64(w[j] >> 16) * s * bf16_bits_to_f64(g[j] >> 16);
      nf[2 * j] = static_cast<float>(n0);
      nf[2 * j + 1] = static_cast<float>(n1);
      nb[j] = static_cast<uint32_t>(f64_to_bf16(n0)) | (static_cast<uint32_t>(f64_to_bf16(n1)) << 16);
    }
    *reinterpret_cast<float4*>(n_f32 + row + h) = float4{nf[0], nf[1], nf[2], nf[3]};
    *reinterpret_cast<float4*>(n_f32 + row + h + 4) = float4{nf[4], nf[5], nf[6], nf[7]};
    *reinterpret_cast<uint4*>(n_bf16 + row + h) = uint4{nb[0], nb[1], nb[2], nb[3]};
  }
}

template <int kBT>
__global__ __launch_bounds__(kBT) void post_norm_residual_kernel(
    const uint16_t* resid, const uint16_t* __restrict__ f, const uint16_t* __restrict__ gain,
    double eps, int H, uint16_t* out) {  // (out may be resid: each element is read, then written)
  __shared__ double lds[kBT / 64];
  const size_t row = static_cast<size_t>(blockIdx.x) * H;
  double ss = 0.0;
  for (int h = threadIdx.x * 8; h < H; h += kBT * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(f + row + h);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = bf16_bits_to_f64(w[j] & 0xFFFFu), b = bf16_bits_to_f64(w[j] >> 16);
      ss += a * a;
      ss += b * b;
    }
  }
  ss = block_sum<kBT>(ss, lds);
  const double s = 1.0 / sqrt(ss / static_cast<double>(H) + eps);
  for (int h = threadIdx.x * 8; h < H; h += kBT * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(f + row + h);
    const uint4 rq = *reinterpret_cast<const uint4*>(resid + row + h);
    const uint4 gq = *reinterpret_cast<const uint4*>(gain + h);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w}, r[4] = {rq.x, rq.y, rq.z, rq.w},
                   g[4] = {gq.x, gq.y, gq.z, gq.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double v0 = bf16_bits_to_f64(r[j] & 0xFFFFu) +
                        bf16_bits_to_f64(w[j] & 0xFFFFu) * s * bf16_bits_to_f64(g[j] & 0xFFFFu);
      const double v1 = bf16_bits_to_f64(r[j] >> 16) +
                        bf16_bits_to_f64(w[j] >> 16) * s * bf16_bits_to_f64(g[j] >> 16);
      o[j] = static_cast<uint32_t>(f64_to_bf16(v0)) | (static_cast<uint32_t>(f64_to_bf16(v1)) << 16);
    }
    *reinterpret_cast<uint4*>(out + row + h) = uint4{o[0], o[1], o[2], o[3]};
  }
}

// Few tokens: kSplit workgroups per token. Each adds the squares of the
// whole row (the same threads, order and sum in each, so every workgroup of
// the token takes the same scale) and writes its own H / kSplit columns.
// Every load goes out before any is used: the workgroup's own columns of f,
// resid and gain, and the whole row of f (buffer loads: offsets past the
// row return zeros, no branch). Out may be resid (each element is read,
// then written, by one thread). H is a multiple of 4 * kSplit, at most
// kSplit * 4 * kBT * kMine (own columns) and 8 * kBT * kRow (the row).
constexpr int kSplit = 8;
template <int kBT, int kMine, int kRow>
__global__ __launch_bounds__(kBT) void post_norm_split_kernel(
    const uint16_t* resid, const uint16_t* __restrict__ f, const uint16_t* __restrict__ gain,
    double eps, int H, uint16_t* out) {
  __shared__ double lds[kBT / 64];
  const size_t row = static_cast<size_t>(blockIdx.x) * H;
  const uint32_t rb = static_cast<uint32_t>(H) * 2;
  const rsrc_t fr = make_rsrc(f + row, rb), rr = make_rsrc(resid + row, rb), gr = make_rsrc(gain, rb);
  const int w = H / kSplit, c0 = static_cast<int>(blockIdx.y) * w;
  uint2 fq[kMine], rq[kMine], gq[kMine];
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int h = c0 + (static_cast<int>(threadIdx.x) + i * kBT) * 4;
    const uint32_t off = h < c0 + w ? static_cast<uint32_t>(h) * 2 : kOutOfRange;
    fq[i] = buf_load8b<0>(fr, off);
    rq[i] = buf_load8b<0>(rr, off);
    gq[i] = buf_load8b<0>(gr, off);
  }
  uint4 q[kRow];
#pragma unroll
  for (int i = 0; i < kRow; ++i) {
    const int h = (static_cast<int>(threadIdx.x) + i * kBT) * 8;
    q[i] = buf_load16<0>(fr, h < H ? static_cast<uint32_t>(h) * 2 : kOutOfRange);
  }
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kRow; ++i) {
    const uint32_t v[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = bf16_bits_to_f64(v[j] & 0xFFFFu), b = bf16_bits_to_f64(v[j] >> 16);
      ss += a * a;
      ss += b * b;
    }
  }
  ss = block_sum<kBT>(ss, lds);
  const double s = 1.0 / sqrt(ss / static_cast<double>(H) + eps);
  auto one = [&](uint32_t fw, uint32_t rw, uint32_t gw) {
    const double v0 = bf16_bits_to_f64(rw & 0xFFFFu) + bf16_bits_to_f64(fw & 0xFFFFu) * s * bf16_bits_to_f64(gw & 0xFFFFu);
    const double v1 = bf16_bits_to_f64(rw >> 16) + bf16_bits_to_f64(fw >> 16) * s * bf16_bits_to_f64(gw >> 16);
    return static_cast<uint32_t>(f64_to_bf16(v0)) | (static_cast<uint32_t>(f64_to_bf16(v1)) << 16);
  };
#pragma unroll
  for (int i = 0; i < kMine; ++i) {
    const int h = c0 + (static_cast<int>(threadIdx.x) + i * kBT) * 4;
    if (h < c0 + w)
      *reinterpret_cast<uint2*>(out + row + h) =
          uint2{one(fq[i].x, rq[i].x, gq[i].x), one(fq[i].y, rq[i].y, gq[i].y)};
  }
}

}  // namespace

hipError_t launch_pre_norm(const uint16_t* resid, const uint16_t* gain, double eps, int T, int H,
                           float* n_f32, uint16_t* n_bf16, hipStream_t st) {
  if (T <= kFewTokens)
    MOE_LAUNCH((pre_norm_kernel<1024>), dim3(T), dim3(1024), 0, st, resid, gain, eps, H, n_f32, n_bf16);
  else
    MOE_LAUNCH((pre_norm_kernel<256>), dim3(T), dim3(256), 0, st, resid, gain, eps, H, n_f32, n_bf16);
  return hipGetLastError();
}

hipError_t launch_post_norm_residual(const uint16_t* resid, const uint16_t* f, const uint16_t* gain,
                                     double eps, int T, int H, uint16_t* out, hipStream_t st) {
  // (T = 1, H = 8192: one workgroup of 1024 threads per token took 5.8 us)
  if (T <= kFewTokens && H % (4 * kSplit) == 0 && H <= kSplit * 4 * 256 && H <= 8 * 256 * 4)
    MOE_LAUNCH((post_norm_split_kernel<256, 1, 4>), dim3(T, kSplit), dim3(256), 0, st, resid, f, gain, eps, H,
               out);
  else if (T <= kFewTokens)
    MOE_LAUNCH((post_norm_residual_kernel<1024>), dim3(T), dim3(1024), 0, st, resid, f, gain, eps, H, out);
  else
    MOE_LAUNCH((post_norm_residual_kernel<256>), dim3(T), dim3(256), 0, st, resid, f, gain, eps, H, out);
  return hipGetLastError();
}

}  // namespace moe
