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

// The grouping of at most 64 routes by one wavefront, without barriers. Lane r holds route r. Eight ballots of the id bits give, for any
// id v, the lanes whose id is below v (most significant bit first), so the
// position of route r is (# routes with a lower id) + (# earlier routes with
// the same id), and offsets[v] is (# routes with an id below v). Every
// touched expert then has one row tile (tile_m >= 64).
__device__ inline void permute_wave(const int32_t* ids, int R, int E, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ sorted_routes, int32_t* __restrict__ active,
                             int32_t* __restrict__ counters, int32_t* __restrict__ tiles) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < R;
  const int e = valid ? ids[lane] : 0;
  const uint64_t vmask = __ballot(valid);
  uint64_t bits[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) bits[b] = __ballot(valid && ((e >> b) & 1));
  auto below = [&](int v) {  // lanes whose id is below v
    uint64_t lt = 0, eq = vmask;
#pragma unroll
    for (int b = 7; b >= 0; --b) {
      if ((v >> b) & 1) {
        lt |= eq & ~bits[b];
        eq &= bits[b];
      } else {
        eq &= ~bits[b];
      }
    }
    return lt;
  };
  const uint64_t lt = below(e);
  const uint64_t same = same_id_mask(e, valid);
  const uint64_t lower = (1ull << lane) - 1ull;
  const bool leader = valid && (same & lower) == 0;
  const uint64_t leaders = __ballot(leader);
  if (valid) sorted_routes[__popcll(lt) + __popcll(same & lower)] = lane;
  if (leader) {
    const int idx = __popcll(lt & leaders);
    active[4 * idx] = e;
    active[4 * idx + 1] = __popcll(lt);
    active[4 * idx + 2] = __popcll(lt) + __popcll(same);
    active[4 * idx + 3] = 0;
    tiles[2 * idx] = e;
    tiles[2 * idx + 1] = __popcll(lt);
  }
  // the streaming kernels read min(E, R) entries (one per possible touched expert)
  for (int v = __popcll(leaders) + lane; v < min(E, R); v += 64) active[4 * v] = -1;
  for (int v = lane; v <= E; v += 64) offsets[v] = v == E ? R : __popcll(below(v));
  if (lane == 0) {
    counters[0] = __popcll(leaders);
    counters[1] = __popcll(leaders);
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
// (Measured alternatives: an election by compare-and-swap, or an arrival
// counter so that only the last workgroup reads the words, add a
// device-scope round trip, and under the pooler's stream each such round
// trip takes microseconds.)
//
// Ordering: everything one workgroup learns from another travels in one
// 64-bit word, stored and loaded at device scope (sc1), so no fence (and no
// L2 write-back or invalidation) is needed for data. A workgroup waits for
// its own stores to complete (vmcnt 0) before its barrier and its loads, so
// of any two workgroups at least one sees the other's words: the last to
// store sees all, so at least one workgroup routes.
template <int NW>
__device__ void route_when_complete(const RouteFuse& f, uint32_t gen, int T, int E) {
  __shared__ int32_t ids_lds[64];
  __shared__ float w_lds[64];
  const uint32_t tag = route_tag(gen);
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's tagged words are stored
  __syncthreads();
  uint64_t key[4];
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
  if (!__syncthreads_and(ok)) return;
  if (t < T) wave_topk(key, f.K, lane, ids_lds + t * f.K, w_lds + t * f.K);
  __syncthreads();
  const int R = T * f.K;
  if (static_cast<int>(threadIdx.x) < R) {
    f.ids[threadIdx.x] = ids_lds[threadIdx.x];
    f.w[threadIdx.x] = w_lds[threadIdx.x];
  }
  if (threadIdx.x < 64) permute_wave(ids_lds, R, E, f.offsets, f.sorted, f.active, f.counters, f.tiles);
  if (threadIdx.x == 0) __hip_atomic_store(f.gen, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
