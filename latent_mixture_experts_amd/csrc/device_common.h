// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resources (gfx9-family descriptor word 3). A load whose byte
// offset lies outside [0, bytes) returns zeros and touches no memory, which
// lets a lane without a row load "nothing" without a branch.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kAuxStream = 0;  // weights: default policy (non-temporal measured slower)
constexpr int kAuxDefault = 0;

// Values one workgroup of a launch stores and another, possibly on another
// XCD, reads while the launch runs (the persistent decode layer): device-
// scope relaxed atomic loads and stores, which gfx950 issues as sc1
// accesses, coherent across the XCDs' L2 caches; the buffer-load form takes
// the same bit, 16, in its cache-policy operand.
// loads and stores of values another workgroup of the same launch writes
template <bool COH>
__device__ __forceinline__ int32_t ld_i32(const int32_t* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH>
__device__ __forceinline__ float ld_f32(const float* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH, typename T>
__device__ __forceinline__ void st_val(T* p, T v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
constexpr int aux_for(bool coh) { return coh ? 16 : 0; }  // 16: sc1 on gfx950 buffer accesses

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Tile order over the 8 XCDs (workgroup b runs on XCD b % 8, each XCD with
// its own L2). Logical tiles are dealt to the XCDs in chunks of `chunk`
// consecutive tiles, round-robin: a chunk (the column tiles of one row tile,
// which share its activation rows) stays in one L2, and when only a prefix
// of the logical tiles has work (a grid sized for the most tiles that can
// exist) every XCD gets its share of that prefix. The grid is a multiple of
// 8 * chunk (xcd_grid), which makes the map a bijection on the grid.
__host__ __device__ __forceinline__ int xcd_tile_of(int block, int chunk) {
  const int j = block >> 3;
  return ((j / chunk) * 8 + (block & 7)) * chunk + j % chunk;
}
__device__ __forceinline__ int xcd_tile(int chunk) { return xcd_tile_of(static_cast<int>(blockIdx.x), chunk); }
inline int xcd_grid(int n, int chunk) { return (n + 8 * chunk - 1) / (8 * chunk) * (8 * chunk); }

// The prefill dense kernel's tile order: workgroup `block` of a grid of
// `grid` (a multiple of 8) runs the tile (row tile, column tile) returned, or
// (-1, -1) for a padding workgroup. Each XCD (block % 8) takes a contiguous
// range of the logical tiles, and the logical order walks group_m row tiles
// at a time, column-tile major within a group.
struct TileRC {
  int mt, nt;
};
__host__ __device__ __forceinline__ TileRC dense_tile_of(int block, int grid, int n_row_tiles,
                                                         int n_col_tiles, int group_m) {
  const int per = grid / 8;
  const int logical = (block % 8) * per + block / 8;
  if (logical >= n_row_tiles * n_col_tiles) return TileRC{-1, -1};
  const int in_group = group_m * n_col_tiles;
  const int first_m = logical / in_group * group_m;
  const int gsize = n_row_tiles - first_m < group_m ? n_row_tiles - first_m : group_m;
  return TileRC{first_m + (logical % in_group) % gsize, (logical % in_group) / gsize};
}

template <int AUX>
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  return uint4{v[0], v[1], v[2], v[3]};
}

template <int AUX>
__device__ __forceinline__ uint2 buf_load8b(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
  return uint2{v[0], v[1]};
}

template <int AUX>
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ uint32_t buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, AUX);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16 bytes as an MFMA bf16x8 operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Eight MXFP4 elements (one dword of codes, element 2j in the low nibble of
// byte j) times the E8M0 scale 2^(s-127), as bf16. The hardware conversion
// takes the scale as an fp32 value; 2^(s-127) is built from its exponent
// bits (s in 1..254 gives a normal fp32 power of two).
__device__ __forceinline__ bf16x8 mxfp4x8_to_bf16(uint32_t codes, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight NVFP4 elements (E2M1 codes of one word) times an arbitrary fp32
// scale. The scaled conversions apply only the power of two of their scale
// (measured: scale 1.5 gives 1.0, 0.3 gives 0.25), which is exact for E8M0
// scales. Here the power of two goes through the conversion to fp32 and the
// significand in [1, 2) (at most 4 significant bits for an E4M3 scale)
// multiplies in fp32; the product of an E2M1 value and that significand has
// at most 5 significant bits, so the bf16 result is exact. Per two elements:
// one conversion, two multiplies, one rounding to a bf16 pair. A zero scale
// gives zeros (through a zero significand).
__device__ __forceinline__ bf16x8 nvfp4x8_to_bf16(uint32_t codes, float scale) {
  const uint32_t sb = __float_as_uint(scale);
  const float p2 = __uint_as_float(sb & 0x7F800000u);  // power of two
  const float mf = (sb & 0x7FFFFFFFu) ? __uint_as_float((sb & 0x807FFFFFu) | 0x3F800000u) : 0.0f;
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p2, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p2, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p2, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p2, 3);
  auto bf = [mf](float x) { return static_cast<__bf16>(x * mf); };
  return bf16x8{bf(v0[0]), bf(v0[1]), bf(v1[0]), bf(v1[1]), bf(v2[0]), bf(v2[1]), bf(v3[0]), bf(v3[1])};
}

__device__ __forceinline__ double bf16_bits_to_f64(uint32_t b) {
  return static_cast<double>(__uint_as_float(b << 16));
}

// round-to-nearest-even of a double to bf16 bits: truncate to fp32 and put
// the sticky bit (inexact) into the last place (round to odd), then round
// that to nearest even at bf16 precision. Values beyond the bf16 range go
// to infinity; NaN becomes the quiet NaN.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  if (v != v) return 0x7FC0u;
  const float t = __double2float_rz(v);
  uint32_t u = __float_as_uint(t);
  if (static_cast<double>(t) != v) u |= 1u;
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float((s & 0xFFu) << 23);
}

// OCP FP8 E4M3 ("fn": bias 7, exponent 0 subnormal, S.1111.111 NaN, no
// infinities) to fp32: the NVFP4 block scale, byte 0 of b, by the gfx950
// fp8 conversion (which follows that format: checked on the GPU against the
// format's definition for all 256 bytes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(b), 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16). Lane l supplies row
// l%16 of A and column l%16 of B, each with the 8 reduction elements of lane
// group l/16; it receives D rows 4*(l/16) .. +3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
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


// Wave-wide max / min of a 32-bit value, uniform result. Within each row of
// 16 lanes: DPP quad_perm xor-1 and xor-2 steps, then row rotations by 4 and
// 8 lanes; the four row results are combined through readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// Sum over the 16 lanes of each row (lanes 16r .. 16r+15); every lane of the
// row receives the same sum, added in a fixed pattern.
__device__ __forceinline__ float row16_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  return v;
}

// Wave-wide sum, uniform result: row sums, then the four rows in order.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = row16_sum_f32(v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return ((a + b) + c) + d;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Top K of 256 rank keys per wavefront; lane owns experts lane, lane+64,
// lane+128, lane+192 (keys are distinct: the low half holds the inverted
// id). Each lane first sorts its four keys; a round then takes the wave max
// of the heads' value halves, and when several lanes hold that value, the
// largest low half among them (the lowest expert id); the lane that owns
// the selected key pops its head. The ids go out in rank order with the
// router weights: softmax over the selected logits in fp64 (sum in rank
// order), rounded to fp32.
__device__ __forceinline__ void wave_topk(uint64_t key[4], int K, int lane, int32_t* ids,
                                          float* w) {
  auto cswap = [](uint64_t& a, uint64_t& b) {  // a >= b afterwards
    const bool sw = b > a;
    const uint64_t t = sw ? b : a;
    b = sw ? a : b;
    a = t;
  };
  cswap(key[0], key[1]);
  cswap(key[2], key[3]);
  cswap(key[0], key[2]);
  cswap(key[1], key[3]);
  cswap(key[1], key[2]);
  uint32_t mine_hi = 0, mine_lo = 0, first_hi = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      const uint32_t hv = static_cast<uint32_t>(key[0] >> 32), lv = static_cast<uint32_t>(key[0]);
      const uint32_t mx = wave_max_u32(hv);
      const uint64_t tied = __ballot(hv == mx);
      uint32_t lo;
      if (__builtin_expect(__popcll(tied) == 1, 1))  // uniform: one lane holds the value
        lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(lv, __builtin_ctzll(tied)));
      else
        lo = wave_max_u32(hv == mx ? lv : 0u);
      if (hv == mx && lv == lo) {
        key[0] = key[1];
        key[1] = key[2];
        key[2] = key[3];
        key[3] = 0;
      }
      if (lane == k) {
        mine_hi = mx;
        mine_lo = lo;
      }
      if (k == 0) first_hi = mx;
    }
  }
  // lane k < K computes a_k = exp(l_k - l_0); every lane adds them in rank
  // order; lane k writes its id and a_k / sum.
  double a = 0.0;
  if (lane < K)
    a = exp(static_cast<double>(key_value(static_cast<uint64_t>(mine_hi) << 32)) -
            static_cast<double>(key_value(static_cast<uint64_t>(first_hi) << 32)));
  double sum = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < K) sum += readlane_f64(a, k);
  if (lane < K) {
    ids[lane] = static_cast<int32_t>(~mine_lo);
    w[lane] = static_cast<float>(a / sum);
  }
}
// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS
// address lds + 16 * l (lds uniform over the wavefront). Issued as inline
// assembly so that the compiler does not make every later LDS read wait for
// it; the kernel waits for it explicitly (vmcnt) before the stage barrier.
__device__ __forceinline__ void lds_copy16(rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(r), "s"(lds) : "memory");
}

// s_waitcnt vmcnt(N) (N < 16) that the compiler's own wait insertion sees:
// waits until at most the N most recent vector-memory instructions are
// outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_keep() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace moe
