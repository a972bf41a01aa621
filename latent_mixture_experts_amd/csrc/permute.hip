// permute.hip -- grouping of routes by expert (step A3).
//
// "Muse Spark Open on Gaudi 2", section "The latent MoE: A' with a per-expert
// norm": every (token, route) pair becomes its own row, and an expert's cost
// is paid per touched expert slice. Route r = t*K + k is listed under its
// expert; the grouping is a stable counting sort, so the result is unique:
// offsets[e] = routes of experts < e, and within an expert the routes keep
// ascending r.
//
// One workgroup of 16 wavefronts. Wave w owns a contiguous segment of routes
// and walks it in chunks of 64. Lanes holding the same expert id find each
// other with eight ballots (one per bit of the id); the rank of a lane among
// them is a popcount, and the highest such lane bumps the per-wave counter.
// Pass 1 counts, a scan turns the per-wave counts into base positions, and
// pass 2 repeats the walk to scatter.
//
// Besides offsets and sorted_routes it writes the work lists of the expert
// GEMMs: the touched experts in ascending id with their row ranges
// (active[i] = {expert, first row, end row, 0}, i < n_active; the entries
// after them, up to the min(E, T*K) that the streaming expert kernels'
// grid covers, hold expert -1, so a workgroup reads only its own entry) and the row tiles (expert, first row) of
// tile_m rows (tiles[], n_tiles).
#include "device_common.h"
#include "kernels.h"
#include "route_small.h"

namespace moe {

namespace {
constexpr int kWaves = 16;

// Exclusive scan over v for threads 0..255 (all 1024 threads must call);
// returns the scan value for thread < 256 and writes the total to *total.
__device__ int block_scan_256(int v, int* lds_wave_sums, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (tid < 256 && lane == 63) lds_wave_sums[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave && w < 4; ++w) base += lds_wave_sums[w];
  if (tid == 0) *total = lds_wave_sums[0] + lds_wave_sums[1] + lds_wave_sums[2] + lds_wave_sums[3];
  __syncthreads();
  return base + incl - v;
}

// Row tiles of tile_m rows for thread tid's expert (cnt routes from sorted
// row off; all 1024 threads call): the (expert, first row) pairs go to tiles
// in expert order, or with pair_order, experts with an even number of tiles
// first, then those with an odd number above one, then single-tile experts.
// The expert kernels deal row tiles to the XCDs in aligned pairs, so an
// expert whose two tiles start at an even index has both on one XCD at once,
// reading its weights through that XCD's L2 once (measured with 32768 routes
// over 256 experts, 121 of them with two tiles: gate/up HBM bytes 1.48 ->
// 1.33x the algorithmic ones, 2304 -> 2232 us; with 16 routes per expert,
// nearly all single tiles, the extra scans only cost time). Returns the
// number of tiles (in every thread).
__device__ int write_tiles(int tid, int E, int cnt, int off, int tile_m, bool pair_order,
                           int32_t* __restrict__ tiles, int* lds_wave_sums, int* lds_tot) {
  const int nt = tid < E ? (cnt + tile_m - 1) / tile_m : 0;
  if (!pair_order) {
    const int tb = block_scan_256(nt, lds_wave_sums, &lds_tot[0]);
    if (tid < E) {
      for (int j = 0; j < nt; ++j) {
        tiles[2 * (tb + j)] = tid;
        tiles[2 * (tb + j) + 1] = off + j * tile_m;
      }
    }
    return lds_tot[0];
  }
  const int cls = nt >= 2 ? (nt & 1) : 2;
  const int s0 = block_scan_256(cls == 0 ? nt : 0, lds_wave_sums, &lds_tot[0]);
  const int s1 = block_scan_256(cls == 1 ? nt : 0, lds_wave_sums, &lds_tot[1]);
  const int s2 = block_scan_256(cls == 2 ? nt : 0, lds_wave_sums, &lds_tot[2]);
  const int tb = cls == 0 ? s0 : cls == 1 ? lds_tot[0] + s1 : lds_tot[0] + lds_tot[1] + s2;
  if (tid < E) {
    for (int j = 0; j < nt; ++j) {
      tiles[2 * (tb + j)] = tid;
      tiles[2 * (tb + j) + 1] = off + j * tile_m;
    }
  }
  return lds_tot[0] + lds_tot[1] + lds_tot[2];
}
}  // namespace

// The whole grouping, run by one workgroup of 1024 threads. ids may point to
// global memory or LDS. Ids are clamped into [0, E) (ids from the caller of
// a routed forward are not checked otherwise); with ids_copy the clamped ids
// are also written there, for the steps after the grouping.
__device__ void permute_block(const int32_t* ids, int R, int E, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted_routes, int32_t* __restrict__ active,
                              int32_t* __restrict__ counters, int32_t* __restrict__ tiles,
                              int tile_m, int32_t* __restrict__ ids_copy = nullptr,
                              bool pair_order = false) {
  __shared__ int hist[kWaves][256];
  __shared__ int wave_sums[4];
  __shared__ int totals[2];
  __shared__ int tile_tot[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < kWaves * 256; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();

  const int seg = ((R + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int rbeg = wave * seg;
  const int rend = min(R, rbeg + seg);

  // pass 1: per-wave counts
  for (int base = rbeg; base < rend; base += 64) {
    const int r = base + lane;
    const bool valid = r < rend;
    const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
    if (valid && ids_copy) ids_copy[r] = e;
    const uint64_t mask = same_id_mask(e, valid);
    if (valid && (63 - __clzll(static_cast<long long>(mask))) == lane)
      hist[wave][e] += __popcll(mask);
  }
  __syncthreads();

  // per-expert totals; hist becomes the prefix over waves
  int tot = 0;
  if (tid < E) {
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w][tid];
      hist[w][tid] = tot;
      tot += c;
    }
  }
  int dummy;
  const int off = block_scan_256(tid < E ? tot : 0, wave_sums, &dummy);
  if (tid < E) {
    offsets[tid] = off;
    for (int w = 0; w < kWaves; ++w) hist[w][tid] += off;
  }
  if (tid == 0) offsets[E] = R;
  __syncthreads();

  // pass 2: scatter
  for (int base = rbeg; base < rend; base += 64) {
    const int r = base + lane;
    const bool valid = r < rend;
    const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
    const uint64_t mask = same_id_mask(e, valid);
    if (valid) {
      const int rank = __popcll(mask & ((1ull << lane) - 1ull));
      sorted_routes[hist[wave][e] + rank] = r;
      if ((63 - __clzll(static_cast<long long>(mask))) == lane) hist[wave][e] += __popcll(mask);
    }
  }

  // work lists: touched experts, and row tiles of tile_m rows
  const int cnt = tid < E ? tot : 0;
  const int act = block_scan_256(cnt > 0 ? 1 : 0, wave_sums, &totals[0]);
  if (tid < E && cnt > 0) {
    active[4 * act] = tid;
    active[4 * act + 1] = off;
    active[4 * act + 2] = off + cnt;
    active[4 * act + 3] = 0;
  }
  if (tid < E && tid >= totals[0]) active[4 * tid] = -1;
  const int n_tiles = write_tiles(tid, E, cnt, off, tile_m, pair_order, tiles, wave_sums, tile_tot);
  if (tid == 0) {
    counters[0] = totals[0];
    counters[1] = n_tiles;
  }
}


// The grouping of many routes over several workgroups, in two launches.
// Chunk c (kChunk consecutive routes, 16 wavefronts of 128) is counted per
// expert by workgroup c of the first launch; in the second, workgroup c
// derives every expert's global start (an exclusive scan over the experts of
// the counts of all chunks) and the routes of its expert in earlier chunks,
// and scatters its chunk as the single-workgroup grouping does: routes keep
// ascending order within an expert, so the result is the same. Workgroup 0
// also writes offsets and the work lists.
constexpr int kChunk = kWaves * 128;

// per-wave counts of this workgroup's chunk into hist (each wavefront its
// own row, so no two lanes update one entry at once)
__device__ inline void count_chunk(const int32_t* ids, int R, int E, int (*hist)[256],
                                    int32_t* __restrict__ ids_copy) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kWaves * 256; i += 1024) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int rbeg = static_cast<int>(blockIdx.x) * kChunk + wave * 128;
  const int rend = min(R, rbeg + 128);
  for (int base = rbeg; base < rend; base += 64) {
    const int r = base + lane;
    const bool valid = r < rend;
    const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
    if (valid && ids_copy) ids_copy[r] = e;
    const uint64_t mask = same_id_mask(e, valid);
    if (valid && (63 - __clzll(static_cast<long long>(mask))) == lane) hist[wave][e] += __popcll(mask);
  }
  __syncthreads();
}

__global__ __launch_bounds__(1024) void permute_count_kernel(const int32_t* __restrict__ ids, int R,
                                                             int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ ids_copy) {
  __shared__ int hist[kWaves][256];
  count_chunk(ids, R, E, hist, ids_copy);
  const int tid = threadIdx.x;
  if (tid < E) {
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) tot += hist[w][tid];
    counts[static_cast<size_t>(blockIdx.x) * E + tid] = tot;
  }
}

__global__ __launch_bounds__(1024) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, const int32_t* __restrict__ counts, int G,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_routes, int32_t* __restrict__ active,
    int32_t* __restrict__ counters, int32_t* __restrict__ tiles, int tile_m, bool pair_order) {
  __shared__ int hist[kWaves][256];
  __shared__ int wave_sums[4];
  __shared__ int totals[2];
  __shared__ int tile_tot[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = static_cast<int>(blockIdx.x);
  // (the clamped ids were copied by the counting launch)
  count_chunk(ids, R, E, hist, nullptr);
  // every expert's routes in earlier chunks and in all chunks
  int before = 0, total = 0;
  if (tid < E) {
    for (int g = 0; g < G; ++g) {
      const int n = counts[static_cast<size_t>(g) * E + tid];
      before += g < c ? n : 0;
      total += n;
    }
  }
  int dummy;
  const int off = block_scan_256(tid < E ? total : 0, wave_sums, &dummy);
  if (tid < E) {  // hist becomes each wavefront's first position per expert
    int run = off + before;
    for (int w = 0; w < kWaves; ++w) {
      const int n = hist[w][tid];
      hist[w][tid] = run;
      run += n;
    }
  }
  __syncthreads();
  const int rbeg = c * kChunk + wave * 128;
  const int rend = min(R, rbeg + 128);
  for (int base = rbeg; base < rend; base += 64) {
    const int r = base + lane;
    const bool valid = r < rend;
    const int e = valid ? min(max(ids[r], 0), E - 1) : 0;
    const uint64_t mask = same_id_mask(e, valid);
    if (valid) {
      const int rank = __popcll(mask & ((1ull << lane) - 1ull));
      sorted_routes[hist[wave][e] + rank] = r;
      if ((63 - __clzll(static_cast<long long>(mask))) == lane) hist[wave][e] += __popcll(mask);
    }
  }
  if (c != 0) return;
  // offsets and the work lists (as the single-workgroup grouping writes them)
  if (tid < E) offsets[tid] = off;
  if (tid == 0) offsets[E] = R;
  const int cnt = tid < E ? total : 0;
  const int act = block_scan_256(cnt > 0 ? 1 : 0, wave_sums, &totals[0]);
  if (tid < E && cnt > 0) {
    active[4 * act] = tid;
    active[4 * act + 1] = off;
    active[4 * act + 2] = off + cnt;
    active[4 * act + 3] = 0;
  }
  if (tid < E && tid >= totals[0]) active[4 * tid] = -1;
  const int n_tiles = write_tiles(tid, E, cnt, off, tile_m, pair_order, tiles, wave_sums, tile_tot);
  if (tid == 0) {
    counters[0] = totals[0];
    counters[1] = n_tiles;
  }
}

__global__ __launch_bounds__(1024) void permute_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_routes, int32_t* __restrict__ active,
    int32_t* __restrict__ counters, int32_t* __restrict__ tiles, int tile_m,
    int32_t* __restrict__ ids_copy, bool pair_order) {
  permute_block(ids, R, E, offsets, sorted_routes, active, counters, tiles, tile_m, ids_copy, pair_order);
}

// Few tokens (T <= 16): top-K of every token (one wavefront per token) and
// the grouping of its routes in one launch; the ids go through LDS.
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ logits, int T, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_routes,
    int32_t* __restrict__ active, int32_t* __restrict__ counters, int32_t* __restrict__ tiles,
    int tile_m) {
  __shared__ int32_t ids_lds[kWaves * 8];
  __shared__ float w_lds[kWaves * 8];
  __shared__ __attribute__((aligned(16))) int32_t hist[512];
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (t < T) {
    uint64_t key[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      key[c] = e < E ? rank_key(logits[static_cast<size_t>(t) * E + e], e) : 0;
    }
    wave_topk(key, K, lane, ids_lds + t * K, w_lds + t * K);
  }
  __syncthreads();
  const int R = T * K;
  if (static_cast<int>(threadIdx.x) < R) {
    ids[threadIdx.x] = ids_lds[threadIdx.x];
    w[threadIdx.x] = w_lds[threadIdx.x];
  }
  if (R <= 64 && tile_m >= 64) {
    if (threadIdx.x < 64) permute_wave(ids_lds, R, E, offsets, sorted_routes, active, counters, tiles, hist);
  } else {
    permute_block(ids_lds, R, E, offsets, sorted_routes, active, counters, tiles, tile_m);
  }
}

hipError_t launch_route_small(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                              int32_t* offsets, int32_t* sorted_routes, int32_t* active,
                              int32_t* counters, int32_t* tiles, int tile_m, hipStream_t st) {
  MOE_LAUNCH((route_small_kernel), dim3(1), dim3(1024), 0, st, logits, T, E, K, ids, w, offsets,
                                                      sorted_routes, active, counters, tiles,
                                                      tile_m);
  return hipGetLastError();
}

// At most 64 routes with one row tile per touched expert: the grouping by
// one wavefront (the caller's ids clamped into [0, E) first).
__global__ __launch_bounds__(64) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_routes, int32_t* __restrict__ active,
    int32_t* __restrict__ counters, int32_t* __restrict__ tiles, int32_t* __restrict__ ids_copy) {
  __shared__ int32_t ids_lds[64];
  __shared__ __attribute__((aligned(16))) int32_t hist[512];
  const int lane = threadIdx.x;
  if (lane < R) {
    const int e = min(max(ids[lane], 0), E - 1);
    ids_lds[lane] = e;
    if (ids_copy) ids_copy[lane] = e;
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  permute_wave(ids_lds, R, E, offsets, sorted_routes, active, counters, tiles, hist);
}

// Two launches pay off from a few chunks on (measured: 4096 routes take
// 11.6 us in one workgroup and 12.7 us in two launches; 32768 routes 66 us
// and 16.5 us).
int permute_chunks(int R) { return R > 3 * kChunk ? (R + kChunk - 1) / kChunk : 0; }

hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* offsets, int32_t* sorted_routes,
                          int32_t* active, int32_t* counters, int32_t* tiles, int tile_m,
                          hipStream_t st, int32_t* ids_copy, int32_t* chunk_counts) {
  const int G = permute_chunks(R);
  // row tiles in pairs per expert when the routes average half a tile per expert or more
  const bool pair_order = 2 * static_cast<int64_t>(R) >= static_cast<int64_t>(E) * tile_m;
  if (G > 0 && chunk_counts) {
    // (a step's timing events: its start at the first launch, its stop at the second)
    StageEvents& ev = stage_events();
    const StageEvents saved = ev;
    ev.stop = nullptr;
    MOE_LAUNCH((permute_count_kernel), dim3(G), dim3(1024), 0, st, ids, R, E, chunk_counts, ids_copy);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
      ev.start = nullptr;
      ev.stop = saved.stop;
      const int32_t* ids_read = ids_copy ? ids_copy : ids;
      MOE_LAUNCH((permute_scatter_kernel), dim3(G), dim3(1024), 0, st, ids_read, R, E, chunk_counts, G,
                 offsets, sorted_routes, active, counters, tiles, tile_m, pair_order);
      e = hipGetLastError();
    }
    ev = saved;
    return e;
  }
  if (R <= 64 && tile_m >= 64)
    MOE_LAUNCH((permute_small_kernel), dim3(1), dim3(64), 0, st, ids, R, E, offsets, sorted_routes,
                                                        active, counters, tiles, ids_copy);
  else
    MOE_LAUNCH((permute_kernel), dim3(1), dim3(1024), 0, st, ids, R, E, offsets, sorted_routes,
                                                  active, counters, tiles, tile_m, ids_copy, pair_order);
  return hipGetLastError();
}

}  // namespace moe
