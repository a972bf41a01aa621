// gemm_dense.hip -- pooler and unpooler projections over many rows (prefill).
//
// out[m][n] = bf16(sum_k a[m][k] * b[n][k]) with a and b bf16 (steps A4 and
// A8: the pooler, 8192 -> 4096, and the unpooler, 4096 -> 8192, each shared
// by all experts: "Soporte de dia 0 para Muse Spark Open en vLLM", section
// "Arquitectura del modelo", paragraph "MoE latente"), on bf16 MFMA 16x16x32
// with fp32 accumulation.
//
// Workgroup tile: 128 rows x 256 columns, eight wavefronts in a 2 x 4 grid,
// each computing 64 x 64 (4 x 4 fragments). Both operands are copied
// straight from global memory into LDS (buffer loads with the LDS
// destination: no registers hold them in flight), 64 reduction elements per
// stage in a ring of three stages, so the copies run two stages ahead of the
// MFMAs. An LDS row is the 128 bytes of one stage; 16-byte piece c of row r
// sits at position r*8 + (c ^ ((r/2) % 8)), so the 16 rows one ds_read_b128
// touches start in distinct banks. One workgroup per CU (144 KiB of LDS);
// workgroup ids are remapped so that each XCD runs a contiguous range of
// tiles, ordered in groups of 4 row tiles (the tiles running together on an
// XCD share A rows and B tiles in its L2).
//
// Reduction order inside a 32-element block: lane group g = lane/16 owns
// elements 8g .. 8g+7, for both operands.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kDW = 8;      // wavefronts per workgroup (2 x 4)
constexpr int kDM = 128;    // tile rows (A)
constexpr int kDN = 256;    // tile columns (rows of B)
constexpr int kDK = 64;     // reduction elements per stage
constexpr int kDRing = 3;   // stages held in LDS
constexpr int kDGM = 4;     // row tiles per group of the tile order
constexpr int kDAOps = kDM * kDK * 2 / 1024 / kDW;  // 1-KiB A copies per wavefront and stage (2)
constexpr int kDBOps = kDN * kDK * 2 / 1024 / kDW;  // 1-KiB B copies per wavefront and stage (4)

// LDS element index of piece c (8 bf16) of row r.
__device__ __forceinline__ int dpos(int r, int c) { return (r * 8 + (c ^ ((r >> 1) & 7))) * 8; }

__global__ __launch_bounds__(64 * kDW) void dense_kernel(const uint16_t* __restrict__ a,
                                                       const uint16_t* __restrict__ b,
                                                       uint16_t* __restrict__ out, int M, int N,
                                                       int K, int n_col_tiles, int kslice,
                                                       float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint16_t As[kDRing][kDM * kDK];
  __shared__ __attribute__((aligned(1024))) uint16_t Bs[kDRing][kDN * kDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;

  // Grouped order: kDGM row tiles at a time, column-tile major within a
  // group, so the 32 tiles an XCD runs at once cover 4 row tiles x 8 column
  // tiles (B read once per 4 row tiles) instead of 1 x 32 (the whole B per
  // row tile: the 4096 x 8192 x 4096 unpooler 314 -> 240 us). The grid is
  // padded to a multiple of 8; padding workgroups get no tile.
  const int n_row_tiles = (M + kDM - 1) / kDM;
  const TileRC tile = dense_tile_of(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x),
                                    n_row_tiles, n_col_tiles, kDGM);
  if (tile.mt < 0) return;
  const int mt = tile.mt, nt = tile.nt;
  const int row0 = mt * kDM, col0 = nt * kDN;
  if (row0 >= M) return;
  const int nrows = min(kDM, M - row0);
  const rsrc_t a_r = make_rsrc(a + static_cast<size_t>(row0) * K, static_cast<uint32_t>(nrows * K * 2));
  const rsrc_t b_r = make_rsrc(b + static_cast<size_t>(col0) * K, static_cast<uint32_t>(kDN * K * 2));

  // K split (blockIdx.y): this workgroup sums elements koff .. koff+kslice-1
  const int koff = static_cast<int>(blockIdx.y) * kslice;
  // copies of this wavefront: A blocks kDAOps*wave + i, B blocks kDBOps*wave + i;
  // block q holds LDS positions 64q .. 64q+63 (rows 8q .. 8q+7)
  uint32_t aoff[kDAOps], boff[kDBOps];
#pragma unroll
  for (int i = 0; i < kDAOps; ++i) {
    const int r = (kDAOps * wave + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = r < nrows ? static_cast<uint32_t>(r * K * 2 + koff * 2 + c * 16) : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < kDBOps; ++i) {
    const int r = (kDBOps * wave + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    boff[i] = static_cast<uint32_t>(r * K * 2 + koff * 2 + c * 16);
  }
  const uint32_t lds_a = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) uint16_t*)(&As[0][0])));
  const uint32_t lds_b = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) uint16_t*)(&Bs[0][0])));
  auto issue = [&](int st, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kDAOps; ++i)
      lds_copy16(a_r, aoff[i] + st * (kDK * 2),
                 __builtin_amdgcn_readfirstlane(lds_a + slot * (kDM * kDK * 2) + (kDAOps * wave + i) * 1024));
#pragma unroll
    for (int i = 0; i < kDBOps; ++i)
      lds_copy16(b_r, boff[i] + st * (kDK * 2),
                 __builtin_amdgcn_readfirstlane(lds_b + slot * (kDN * kDK * 2) + (kDBOps * wave + i) * 1024));
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) __attribute__((always_inline)) {
    const uint16_t* as = As[slot];
    const uint16_t* bs = Bs[slot];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = s * 4 + g;
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) av[m] = as_bf16x8(*reinterpret_cast<const uint4*>(&as[dpos(wm * 64 + m * 16 + nl, c)]));
#pragma unroll
      for (int f = 0; f < 4; ++f) bv[f] = as_bf16x8(*reinterpret_cast<const uint4*>(&bs[dpos(wn * 64 + f * 16 + nl, c)]));
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[m][f] = mfma16x16x32(av[m], bv[f], acc[m][f]);
    }
  };

  // Stage s lives in slot s % 3. Copies past the last stage repeat it into a
  // slot that is no longer read, so the loop has no conditional loads.
  const int nst = kslice / kDK;
  issue(0, 0);
  issue(min(1, nst - 1), 1);
  wait_vm_keep<kDAOps + kDBOps>();
  __syncthreads();
  int slot = 0;
  for (int st = 0; st < nst; ++st) {
    const int s2 = slot >= 1 ? slot - 1 : slot + 2;  // (st + 2) % 3
    issue(min(st + 2, nst - 1), s2);
    compute(slot);
    wait_vm_keep<kDAOps + kDBOps>();
    __syncthreads();
    slot = slot == 2 ? 0 : slot + 1;
  }
  wait_vm_keep<0>();  // no copy may still target this workgroup's LDS

#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + m * 16 + 4 * g + i;
      if (r >= nrows) continue;
      const size_t o = static_cast<size_t>(row0 + r) * N + col0 + wn * 64 + nl;
      if (part) {  // fp32 partial sums of this split
        float* dst = part + static_cast<size_t>(blockIdx.y) * M * N + o;
#pragma unroll
        for (int f = 0; f < 4; ++f) dst[f * 16] = acc[m][f][i];
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) out[o + f * 16] = f32_to_bf16(acc[m][f][i]);
      }
    }
}

// out = bf16(sum over the S splits' fp32 partial sums, in split order);
// four consecutive elements per thread (M * N is a multiple of 256).
__global__ __launch_bounds__(256) void dense_split_sum_kernel(const float* __restrict__ part, int S,
                                                              size_t n, uint16_t* __restrict__ out) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int s = 1; s < S; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(part + static_cast<size_t>(s) * n + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const uint32_t lo = f32_to_bf16(acc.x) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
  const uint32_t hi = f32_to_bf16(acc.z) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
  *reinterpret_cast<uint2*>(out + i) = uint2{lo, hi};
}

}  // namespace

// K splits of the LDS-staged kernel for M x N x K: 1 when its tiles fill at
// least half of the CUs, else the fewest (2, 4, 8 or 16) that bring tiles x
// splits to 256, each split a multiple of the stage; 0 when it does not apply.
int dense_splits(int M, int N, int K) {
  if (N % kDN || K % kDK || K < kDK) return 0;
  const int tiles = ((M + kDM - 1) / kDM) * (N / kDN);
  if (tiles >= 128) return 1;
  for (int s = 2; s <= 16; s *= 2)
    if (tiles * s >= 256 && K % (kDK * s) == 0) return s;
  return 0;
}

bool dense_lds_ok(int M, int N, int K) { return dense_splits(M, N, K) == 1; }

// The dense kernel's grid for an M x N output, and the tile each of its
// workgroups runs (for the host-side check of the tile order).
int dense_grid(int M, int N) {
  const int n = ((M + kDM - 1) / kDM) * (N / kDN);
  return (n + 7) / 8 * 8;
}
TileRC dense_tile_host(int block, int M, int N) {
  return dense_tile_of(block, dense_grid(M, N), (M + kDM - 1) / kDM, N / kDN, kDGM);
}

// part: S * M * N fp32 of workspace when S = dense_splits(M, N, K) > 1.
hipError_t launch_dense_lds(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N, int K,
                            hipStream_t st, float* part) {
  const int S = dense_splits(M, N, K);
  if (S < 1 || (S > 1 && !part)) return hipErrorInvalidValue;
  const int n_col_tiles = N / kDN;
  // a step's timing events: its start at the first launch, its stop at the last
  StageEvents& ev = stage_events();
  const StageEvents saved = ev;
  if (S > 1) ev.stop = nullptr;
  MOE_LAUNCH((dense_kernel), dim3(dense_grid(M, N), S), dim3(64 * kDW), 0, st, a, b, out, M, N, K,
             n_col_tiles, K / S, S > 1 ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (S > 1 && e == hipSuccess) {
    ev.start = nullptr;
    ev.stop = saved.stop;
    const size_t mn = static_cast<size_t>(M) * N;
    MOE_LAUNCH((dense_split_sum_kernel), dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, st,
               part, S, mn, out);
    e = hipGetLastError();
  }
  ev = saved;
  return e;
}

}  // namespace moe
