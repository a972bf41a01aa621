// route_small.h -- top-K and grouping of a few tokens' routes by one
// workgroup (steps A2 and A3).
//
// "Muse Spark Open on Gaudi 2", section "The latent MoE: A' with a per-expert
// norm": each token keeps its K best experts, every (token, route) pair
// becomes a row, and the rows are grouped by expert (a stable counting sort:
// offsets[e] = routes of experts < e, routes ascending within an expert).
//
// Besides the grouping kernels, the launch that runs the router beside the
// pooler uses route_when_complete: every router workgroup, once its logits
// are written, checks whether all experts' logits of this call are; each
// workgroup that finds them all complete routes (they all write the same
// values). Nothing waits, so no workgroup depends on another being
// scheduled.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace moe {

// Lanes (of those with `valid`) that hold the same id e as this lane.
__device__ __forceinline__ uint64_t same_id_mask(int e, bool valid) {
  uint64_t mask = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    mask &= bit ? bb : ~bb;
  }
  return mask;
}

// The grouping of at most 64 routes by one wavefront, without barriers.
// Lane r holds route r. The per-expert counts are added up in LDS and
// scanned over the experts (lane j holds experts 4j .. 4j+3; row scans by
// DPP shifts, then the rows before): offsets[v] is the number of routes with
// an id below v, and a second scan of the touched flags gives each touched
// expert its work-list index. Route r goes to offsets[id] + (# earlier
// routes with the same id, from eight ballots of the id bits). Every touched
// expert has one row tile (tile_m >= 64). hist: 512 ints of LDS; E <= 256.
template <bool COH = false>
__device__ inline void permute_wave(const int32_t* ids, int R, int E, int32_t* __restrict__ offsets,
                                    int32_t* __restrict__ sorted_routes, int32_t* __restrict__ active,
                                    int32_t* __restrict__ counters, int32_t* __restrict__ tiles,
                                    int32_t* hist) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < R;
  const int e = valid ? ids[lane] : 0;
  // (one wavefront: each step's LDS accesses complete before the next reads)
  reinterpret_cast<int4*>(hist)[lane] = int4{0, 0, 0, 0};
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  if (valid) atomicAdd(&hist[e], 1);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const int4 h = reinterpret_cast<const int4*>(hist)[lane];
  // exclusive scans of the counts and of the touched flags over the experts
  auto scan = [&](int c) {  // c: this lane's total; returns the lanes-before total
    int incl = c;
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31),
              r2 = __builtin_amdgcn_readlane(incl, 47);
    const int row = lane >> 4;
    return incl - c + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  };
  const int tx = h.x > 0, ty = h.y > 0, tz = h.z > 0, tw = h.w > 0;
  const int o0 = scan(h.x + h.y + h.z + h.w), q0 = scan(tx + ty + tz + tw);
  const int o[4] = {o0, o0 + h.x, o0 + h.x + h.y, o0 + h.x + h.y + h.z};
  const int q[4] = {q0, q0 + tx, q0 + tx + ty, q0 + tx + ty + tz};
  const int n_active = __builtin_amdgcn_readlane(q0 + tx + ty + tz + tw, 63);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (4 * lane + j < E) st_val<COH>(offsets + 4 * lane + j, o[j]);
    hist[4 * lane + j] = o[j];
    hist[256 + 4 * lane + j] = q[j];
  }
  if (lane == 0) st_val<COH>(offsets + E, R);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const uint64_t same = same_id_mask(e, valid);
  const uint64_t lower = (1ull << lane) - 1ull;
  const int first = hist[e];
  if (valid) st_val<COH>(sorted_routes + first + __popcll(same & lower), static_cast<int32_t>(lane));
  if (valid && (same & lower) == 0) {  // the expert's first route
    const int idx = hist[256 + e];
    st_val<COH>(active + 4 * idx, e);
    st_val<COH>(active + 4 * idx + 1, first);
    st_val<COH>(active + 4 * idx + 2, static_cast<int32_t>(first + __popcll(same)));
    st_val<COH>(active + 4 * idx + 3, 0);
    st_val<COH>(tiles + 2 * idx, e);
    st_val<COH>(tiles + 2 * idx + 1, first);
  }
  // the streaming kernels read min(E, R) entries (one per possible touched expert)
  for (int v = n_active + lane; v < min(E, R); v += 64) st_val<COH>(active + 4 * v, -1);
  if (lane == 0) {
    st_val<COH>(counters, n_active);
    st_val<COH>(counters + 1, n_active);
  }
}

// Tag of one call's router logits: a bijective hash of the generation word
// (advanced by every call that routes this way), never 0, so neither a
// zero-filled workspace nor the previous call's words carry it.
__device__ __forceinline__ uint32_t route_tag(uint32_t gen) {
  uint32_t x = gen + 0x9E3779B9u;
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x | 1u;
}

// Called by every router workgroup (NW wavefronts, T <= NW, T * K <= 64)
// after its threads t < T have stored the tagged logit of token t for
// expert e: tagged[t * E + e] = tag << 32 | logit bits, tag = route_tag(gen)
// for the generation word's value gen at the launch. The workgroup reads
// all T * E tagged words; if each carries this call's tag, every logit is
// there, and the workgroup takes each token's top K (wave t for token t,
// from the words it holds), writes ids and weights, groups the routes and
// stores gen + 1 for the next call. Several workgroups may find the logits
// complete; they compute from the same words and write the same values.
//
// A workgroup that finds a tag missing does not leave: it polls the
// generation word until a workgroup that found all tags has stored gen + 1
// (then the routing is done), and if that has not happened within kGrace it
// reads the tagged words again and routes itself once all tags are there.
// So routing needs only that every stored word becomes visible to every
// workgroup in finite time, which device-scope atomic stores guarantee; no
// ordering between one workgroup's stores and another's loads is assumed.
// The waits are bounded: past kGiveUp the workgroup sets bit 0 of
// status (left for the caller to read) and leaves without routing.
// (Measured alternatives: an election by compare-and-swap, or an arrival
// counter so that only the last workgroup reads the words, put a
// device-scope round trip on every call's critical path, and under the
// pooler's stream each such round trip takes microseconds.)
//
// Data travels only inside those 64-bit words (stored and loaded at device
// scope), so no fence (no L2 write-back or invalidation) is needed.
template <int NW>
__device__ void route_when_complete(const RouteFuse& f, uint32_t gen, int T, int E) {
  constexpr uint64_t kGrace = 100000;      // ~40 us at the 100 MHz constant clock (s_memrealtime)
  constexpr uint64_t kGiveUp = 10000000;   // ~100 ms
  __shared__ int32_t ids_lds[64];
  __shared__ float w_lds[64];
  __shared__ __attribute__((aligned(16))) int32_t hist[512];
  __shared__ int done_lds;
  const uint32_t tag = route_tag(gen);
  const int lane = threadIdx.x & 63, t = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's tagged words are stored
  __syncthreads();
  uint64_t key[4];
  auto read_all = [&]() -> bool {
    int ok = 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      key[c] = 0;
      const int e = lane + 64 * c;
      if (t < T && e < E) {
        const uint64_t v = __hip_atomic_load(f.tagged + static_cast<size_t>(t) * E + e,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok &= static_cast<uint32_t>(v >> 32) == tag;
        key[c] = rank_key(__uint_as_float(static_cast<uint32_t>(v)), e);
      }
    }
    return __syncthreads_and(ok);
  };
  if (!read_all()) {
    // wait (bounded) for another workgroup's routing, then route here if none came
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool mine = false;
    for (;;) {
      if (threadIdx.x == 0) {
        const uint32_t g = __hip_atomic_load(f.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t dt = __builtin_amdgcn_s_memrealtime() - t0;
        done_lds = g != gen ? 1 : dt > kGiveUp ? 2 : dt > kGrace ? 3 : 0;
      }
      __syncthreads();
      const int d = done_lds;
      __syncthreads();
      if (d == 1) return;
      if (d == 2) {
        if (threadIdx.x == 0) __hip_atomic_fetch_or(f.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      if (d == 3 && read_all()) {
        mine = true;
        break;
      }
      // (a short sleep: the waiting workgroups end, and with them the launch,
      // soon after the routing workgroup stores gen + 1; 32 instead of 1
      // measured the T = 1 layer 1.1 us slower, T = 4 0.7 us, T = 8 0.4 us)
      __builtin_amdgcn_s_sleep(1);
    }
    if (!mine) return;
  }
  if (t < T) wave_topk(key, f.K, lane, ids_lds + t * f.K, w_lds + t * f.K);
  __syncthreads();
  const int R = T * f.K;
  if (static_cast<int>(threadIdx.x) < R) {
    f.ids[threadIdx.x] = ids_lds[threadIdx.x];
    f.w[threadIdx.x] = w_lds[threadIdx.x];
  }
  if (threadIdx.x < 64) permute_wave(ids_lds, R, E, f.offsets, f.sorted, f.active, f.counters, f.tiles, hist);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(f.gen, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
