// decode_layer.hip -- the whole latent MoE layer for one or two tokens in a
// single launch (steps A1-A8): the persistent decode layer.
//
// "RadixArk team serves Meta's Muse Spark Open on one TPU host", section "A
// single program for a serving step": one program runs the decode step and
// pipelines its weight loads so that transfers do not stall the compute;
// "Muse Spark Open on Gaudi 2", section "What it taught about Gaudi": at
// batch 1 the host's launches, not the device, set the decode time. Here the
// five launches of the per-step path (router + pooler, gate/up, down,
// combine, unpooler) become phases of one grid.
//
// Grid: G workgroups, all resident at once (the grid is the device's
// capacity at this kernel's occupancy, two workgroups of 512 threads per
// CU). Work items of a phase are dealt to the workgroups in turn (item i to
// workgroup i mod G); the item shapes are those of the per-step kernels,
// whose bodies run here unchanged. G equals the capacity, so a phase of G
// or 2G items takes one or two item times on every workgroup.
//
//   phase 1: router logits (one item per expert; logits also stored tagged
//            with this call's tag) and the pooler's column groups; then
//            workgroup 0, once every tagged logit of this call is visible,
//            takes the top K, groups the routes (work list, route order)
//            and raises the routing flag -- under the pooler's stream;
//   phase 2: gate/up + SwiGLU items (touched expert x column groups);
//   phase 3: down items, fp32 route rows and per-32-column sums of squares;
//   phase 4: post-norm + weighted sum (token x column block);
//   phase 5: unpooler column groups.
//
// Barriers. A workgroup that finishes its items of phase p waits for its
// own stores (vmcnt 0 in every wavefront), then stores this call's tag for
// barrier p in its arrival slot and, once that store is acknowledged, loads
// the slots of its group (workgroups w mod 8: with the dispatcher's round-
// robin over the XCDs, one group per XCD; 64 slots on two 128-byte lines,
// one load). If all carry the tag it stores the tag in the group word and,
// once acknowledged, loads the eight group words; if all carry it, it
// stores the tag in eight release words (one per 128-byte line; workgroup w
// polls word w mod 8). Each check comes after the workgroup's own store is
// acknowledged, so the workgroup whose store is acknowledged last sees every
// store: some workgroup completes each group and the barrier (several may;
// the stores are the same). The checks come before the next phase's weight
// loads: a load issued behind them would return only after them. A
// workgroup starts its phase-(p+1) item by issuing the item's first weight
// stages, and only then waits for the release (the streaming body's hook),
// so the barrier's latency runs under its own weight loads; one with no
// item in phase p+1 waits before it arrives at barrier p+1, so a slot or
// group word never holds tag p+1 before tag p has been seen in all. Should
// the checks all miss (they assume that a load issued after a store is
// acknowledged sees it, which the memory model does not promise for
// relaxed accesses to different addresses), a workgroup still waiting for a
// release after a grace period runs them itself.
// Every value one workgroup writes and another reads (latent rows, routing,
// h, route rows and their sums of squares, y) is stored and loaded with
// device-scope atomic accesses (sc1 on gfx950: device coherent across the
// XCDs' L2 caches), so no cache write-back or invalidation is issued; the
// arrival slots, group words, routing flag and release words are such
// accesses too.
//
// Tags. Every workgroup reads the generation word at its start; the tags of
// the routing and of barriers 1..4 are bijective hashes of it, so slots and
// words left by an earlier call (or any initial contents) carry other tags.
// The workgroup that completes barrier 1 advances the word (every workgroup
// of the call has read it by then).
//
// All waits are bounded (about 10 ms): a wait that gives up sets bit 1 of
// the status word (and a bit naming the wait) and lets its workgroup go on,
// so the launch always completes; the call's output is then invalid (never
// seen in practice: it would need a workgroup of the grid not to be
// scheduled while the others run, that is, other kernels occupying the
// device at the same time).
#include "combine_cols.h"
#include "device_common.h"
#include "kernels.h"
#include "route_small.h"
#include "router_gemv.h"
#include "stream_body.h"

namespace moe {

namespace {

constexpr int kDW = 8;                 // wavefronts per workgroup
constexpr int kRelStride = 32;         // words between group / release words (128 bytes)
constexpr int kGroups = 8;             // barrier groups (w mod 8)
constexpr int kGroupSlots = kDecodeMaxWorkers / kGroups;  // slots per group
// Bounded waits: 10 ms of the 100 MHz constant clock (s_memrealtime).
constexpr uint64_t kWaitTicks = 1000000;
// Status bits (sync[1]): 2 any wait gave up; 4 a wait for the routing flag,
// 8 for a release, 16 workgroup 0's wait for the tagged logits. sync[3]:
// the workgroup count.
enum { kGaveUp = 2, kRouteWait = 4, kReleaseWait = 8, kLogitWait = 16 };

struct DecodeArgs {
  SkinnyArgs pool, gateup, down, unpool;
  int n_pool, gu_gx, n_gu, dn_gx, n_dn, comb_cb, n_comb, n_unpool;
  // router
  const uint16_t* x;
  const float* router;
  float* logits;
  uint64_t* tagged;
  int T, H, E, K, L;
  // routing outputs
  int32_t* ids;
  float* w;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* active;
  int32_t* counters;
  int32_t* tiles;
  // combine
  const float* rows;
  const float* ssp;
  const uint16_t* gain;
  int gpe;
  float eps;
  uint16_t* y;
  // hand-offs
  uint32_t* sync;   // [0] generation word, [1] status, [2] routing flag
  uint32_t* slots;  // arrival slots: group g's at [g * kGroupSlots, ...)
  uint32_t* grp;    // 8 group words, kRelStride apart
  uint32_t* rel;    // 8 release words, kRelStride apart
  int G;
};

__device__ __forceinline__ uint32_t barrier_tag(uint32_t gen, int i) {
  return route_tag(gen * 8u + static_cast<uint32_t>(i));
}

__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void give_up(uint32_t* status, uint32_t bit) {
  __hip_atomic_fetch_or(status, kGaveUp | bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

// Thread 0 polls *word until it holds `tag` (bounded), then the workgroup goes on.
__device__ void wait_word(const uint32_t* word, uint32_t tag, uint32_t* status, uint32_t bit) {
  if (threadIdx.x == 0) {
    const uint64_t t0 = now();
    while (ld_u32(word) != tag) {
      if (now() - t0 > kWaitTicks) {
        give_up(status, bit);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t* slot_of(uint32_t* slots, int w) {
  return slots + (w % kGroups) * kGroupSlots + w / kGroups;
}

// Completion checks of barrier b (wavefront 0 of a workgroup of group g):
// if every slot of the group carries the tag, the group word; then, if every
// group word carries it, the release words (and, at barrier 1, the next
// generation value). Each store is acknowledged (vmcnt 0) before the next
// load.
__device__ void complete(uint32_t* sync, const uint32_t* slots, uint32_t* grp, uint32_t* rel, int G, int g,
                         int b, uint32_t gen, uint32_t tag) {
  const int lane = threadIdx.x;
  const int n = (G - g + kGroups - 1) / kGroups;  // members of group g
  int ok = 1;
  for (int j = lane; j < n; j += 64) ok &= ld_u32(slots + g * kGroupSlots + j) == tag;
  if (!__all(ok)) return;
  if (lane == 0) st_u32(grp + kRelStride * g, tag);
  __builtin_amdgcn_s_waitcnt(0);
  const int ng = G < kGroups ? G : kGroups;
  if (!__all(lane >= ng || ld_u32(grp + kRelStride * lane) == tag)) return;
  if (lane == 0) {
    // (every workgroup has read the generation word once all have arrived at barrier 1)
    if (b == 1) st_u32(sync, gen + 1u);
    st_u32(sync + 8 + b, static_cast<uint32_t>(now()));  // (diagnostics: released)
  }
  if (lane < kGroups) st_u32(rel + kRelStride * lane, tag);
}

// The hook of phase p+1 (and the wait of a workgroup with no item there):
// the wait for the release of barrier p, once per phase (the hook runs in
// the first pass of every item); records that the workgroup has seen it (an
// item whose work-list entry is not a touched expert returns before its
// hook runs). A workgroup still waiting after kGrace runs the completion
// checks itself, so the barrier completes once every slot store has become
// visible, whatever the order in which the arrivals' checks saw them.
struct Barrier {
  uint32_t* sync;
  const uint32_t* slots;
  uint32_t* grp;
  uint32_t* rel;
  int G, wid, b;
  uint32_t gen;
  bool* seen;
  __device__ void operator()() const {
    if (*seen) return;
    constexpr uint64_t kGrace = 5000;  // 50 us: above any measured barrier
    const uint32_t tag = barrier_tag(gen, b);
    if (threadIdx.x < 64) {
      const uint32_t* word = rel + kRelStride * (wid % kGroups);
      const uint64_t t0 = now();
      for (;;) {
        if (__builtin_amdgcn_readfirstlane(ld_u32(word)) == tag) break;  // (uniform: every lane goes on together)
        const uint64_t dt = now() - t0;
        if (dt > kWaitTicks) {
          if (threadIdx.x == 0) give_up(sync + 1, kReleaseWait);
          break;
        }
        if (dt > kGrace) complete(sync, slots, grp, rel, G, wid % kGroups, b, gen, tag);
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    *seen = true;
  }
};

// Arrival of workgroup wid at barrier b: its stores are done (every
// wavefront), then its slot, then (wavefront 0, once the slot store is
// acknowledged) the completion checks.
__device__ void arrive(const DecodeArgs& a, int wid, int b, uint32_t gen) {
  const uint32_t tag = barrier_tag(gen, b);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x >= 64) return;
  if (threadIdx.x == 0) st_u32(slot_of(a.slots, wid), tag);
  __builtin_amdgcn_s_waitcnt(0);
  complete(a.sync, a.slots, a.grp, a.rel, a.G, wid % kGroups, b, gen, tag);
}

// ---- the routing (workgroup 0, after its phase-1 items) -----------------------
// Once every tagged logit of this call is visible: the top K of each token
// (wavefront t for token t) and the grouping of the routes, then the routing
// flag.
template <int TMAX>
__device__ void route(const DecodeArgs& a, uint32_t gen) {
  __shared__ int32_t ids_lds[64];
  __shared__ float w_lds[64];
  __shared__ __attribute__((aligned(16))) int32_t hist[512];
  uint32_t* status = a.sync + 1;
  const int lane = threadIdx.x & 63, t = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t rtag = route_tag(gen);
  const uint64_t t0 = now();
  uint64_t key[4];
  for (;;) {
    int ok = 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      key[c] = 0;
      const int e = lane + 64 * c;
      if (t < a.T && e < a.E) {
        const uint64_t v = __hip_atomic_load(a.tagged + static_cast<size_t>(t) * a.E + e, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        ok &= static_cast<uint32_t>(v >> 32) == rtag;
        key[c] = rank_key(__uint_as_float(static_cast<uint32_t>(v)), e);
      }
    }
    if (__syncthreads_and(ok)) break;
    const bool late = now() - t0 > kWaitTicks;  // (the same clock value need not reach every wavefront:
    if (__syncthreads_or(late)) {               //  decided together)
      if (threadIdx.x == 0) give_up(status, kLogitWait);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (t < a.T) wave_topk(key, a.K, lane, ids_lds + t * a.K, w_lds + t * a.K);
  __syncthreads();
  const int R = a.T * a.K;
  if (static_cast<int>(threadIdx.x) < R) {
    st_val<true>(a.ids + threadIdx.x, ids_lds[threadIdx.x]);
    st_val<true>(a.w + threadIdx.x, w_lds[threadIdx.x]);
  }
  if (threadIdx.x < 64)
    permute_wave<true>(ids_lds, R, a.E, a.offsets, a.sorted, a.active, a.counters, a.tiles, hist);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    st_u32(a.sync + 2, rtag);
    st_u32(a.sync + 3, static_cast<uint32_t>(a.G));
    st_u32(a.sync + 8, static_cast<uint32_t>(now()));  // (diagnostics: routing done)
  }
}

// ---- one workgroup ------------------------------------------------------------
template <int BFMT, int TMAX, bool RS>
__device__ void worker(const DecodeArgs& a, int wid, uint32_t gen) {
  __shared__ double part[kDW][TMAX];
  uint32_t* status = a.sync + 1;
  // (diagnostics: workgroup 0 stamps its start and the end of each of its phases)
  auto stamp = [&](int k) {
    if (wid == 0 && threadIdx.x == 0) st_u32(a.sync + 16 + k, static_cast<uint32_t>(now()));
  };
  stamp(0);
  // phase 1: router items, then pooler items; workgroup 0 then routes
  const uint32_t rtag = route_tag(gen);
  for (int i = wid; i < a.E + a.n_pool; i += a.G) {
    if (i < a.E)
      router_gemv_body<TMAX, kDW>(a.x, a.router, a.logits, a.T, a.H, a.E, i, part, a.tagged, rtag);
    else
      stream_body<B_BF16, EPI_BF16, 1, 1, 1, 8, 2, true, true>(a.pool, i - a.E, 0);
    __syncthreads();
  }
  if (wid == 0) route<TMAX>(a, gen);
  arrive(a, wid, 1, gen);
  stamp(1);
  // phase 2: gate/up (the work list needs the routing; A, the latent rows, barrier 1)
  wait_word(a.sync + 2, rtag, status, kRouteWait);
  bool seen1 = false;
  const Barrier b1{a.sync, a.slots, a.grp, a.rel, a.G, wid, 1, gen, &seen1};
  for (int i = wid; i < a.n_gu; i += a.G) {
    stream_body<BFMT, EPI_SWIGLU, 2, 1, 2, 4, 2, true, true>(a.gateup, i % a.gu_gx, i / a.gu_gx, b1);
    __syncthreads();
  }
  if (!seen1) b1();  // (no item with a touched expert: the hook never ran)
  arrive(a, wid, 2, gen);
  stamp(2);
  // phase 3: down (A, the h rows, barrier 2)
  bool seen2 = false;
  const Barrier b2{a.sync, a.slots, a.grp, a.rel, a.G, wid, 2, gen, &seen2};
  for (int i = wid; i < a.n_dn; i += a.G) {
    // (RS: the gain-scaled bf16 route rows too, the unpooler phase's input)
    stream_body<BFMT, RS ? EPI_F32_SCATTER_SCALED : EPI_F32_SCATTER, 2, 1, 2, 4, 2, true, true>(
        a.down, i % a.dn_gx, i / a.dn_gx, b2);
    __syncthreads();
  }
  if (!seen2) b2();
  arrive(a, wid, 3, gen);
  stamp(3);
  bool seen3 = false;
  const Barrier b3{a.sync, a.slots, a.grp, a.rel, a.G, wid, 3, gen, &seen3};
  if constexpr (RS) {
    // phases 4 and 5 in one: the unpooler against the gain-scaled route rows,
    // each row's post-norm scale and the weighted sum in its epilogue
    // (EPI_ROUTE_SUM; barrier 3: the route rows and their partial sums)
    stamp(4);
    for (int i = wid; i < a.n_unpool; i += a.G) {
      stream_body<B_BF16, EPI_ROUTE_SUM, 1, 1, 1, 8, 2, true, true>(a.unpool, i, 0, b3);
      __syncthreads();
    }
    stamp(5);
    return;
  }
  // phase 4: post-norm + weighted sum (the route rows, barrier 3)
  b3();
  for (int i = wid; i < a.n_comb; i += a.G) {
    if (a.gpe)
      combine_cols_body<1, true>(a.rows, a.ssp, a.w, a.ids, a.gain, a.eps, a.K, a.L, a.y, i % a.comb_cb,
                                 i / a.comb_cb);
    else
      combine_cols_body<0, true>(a.rows, a.ssp, a.w, a.ids, a.gain, a.eps, a.K, a.L, a.y, i % a.comb_cb,
                                 i / a.comb_cb);
  }
  arrive(a, wid, 4, gen);
  stamp(4);
  // phase 5: unpooler (A, y, barrier 4)
  bool seen4 = false;
  const Barrier b4{a.sync, a.slots, a.grp, a.rel, a.G, wid, 4, gen, &seen4};  // (no barrier follows: a workgroup
                                                                //  without items just ends)
  for (int i = wid; i < a.n_unpool; i += a.G) {
    stream_body<B_BF16, EPI_BF16, 1, 1, 1, 8, 2, true, true>(a.unpool, i, 0, b4);
    __syncthreads();
  }
  stamp(5);
}

template <int BFMT, int TMAX, bool RS>
__global__ __launch_bounds__(64 * kDW, 4) void decode_layer_kernel(DecodeArgs a) {
  const uint32_t gen = ld_u32(a.sync);
  worker<BFMT, TMAX, RS>(a, blockIdx.x, gen);
}

template <int BFMT, int TMAX, bool RS>
hipError_t launch_decode(const DecodeArgs& a, size_t lds, hipStream_t st) {
  MOE_LAUNCH((decode_layer_kernel<BFMT, TMAX, RS>), dim3(a.G), dim3(64 * kDW), lds, st, a);
  return hipGetLastError();
}

template <int BFMT, int TMAX, bool RS>
const void* kernel_of() {
  return reinterpret_cast<const void*>(&decode_layer_kernel<BFMT, TMAX, RS>);
}

// One phase's streaming arguments, finalised as the per-step launchers do
// (rows staged in LDS in one pass, plus the row of zeros of the NVFP4
// few-rows forms); false if the phase does not fit the kernel's compiled
// shape (K split ks, u weight stages in flight).
bool finalize(SkinnyArgs& p, int a_rows, int ks, int u, size_t* lds, int zero_rows = 0,
              size_t budget = 40 * 1024, int nf = 2) {
  const size_t row_bytes = 2 * static_cast<size_t>(p.K) + 16;
  const int rows = a_rows < 1 ? 1 : a_rows;
  if (rows > 16 || static_cast<size_t>(rows) * row_bytes > budget) return false;
  p.pass_rows = rows;
  p.a_tokens = p.a_gather ? rows : 0;
  if (p.K % 256) return false;
  const int nstages = p.K / 256;
  if (nstages % ks || (nstages / ks) % u) return false;
  const size_t b = stream_lds_bytes(p, true, ks, 1, nf, zero_rows);
  *lds = b > *lds ? b : *lds;
  return true;
}

}  // namespace

// (the unpooler against the T*K route rows: their LDS budget is the per-step
// launch's, kRouteSumLds; two workgroups per CU take at most 80 KiB each)
constexpr size_t kRouteSumRowsLds = 72 * 1024;

bool decode_layer_ok(int T, int H, int L, int I, int E, int K, bool nvfp4, bool route_sum) {
  if (T < 1 || T > 2 || T * K > 64 || E > 256) return false;
  if (route_sum && !down_scaled_ok(T, I, nvfp4)) return false;  // (MXFP4 or the one-row NVFP4 form)
  SkinnyArgs p{};
  size_t lds = 0;
  p.K = H;
  if (!finalize(p, T, 8, 1, &lds)) return false;
  p.K = L;
  p.a_gather = 1;
  if (!finalize(p, T, 4, 2, &lds, nvfp4 ? 1 : 0)) return false;
  p.K = I;
  p.a_gather = 0;
  if (!finalize(p, T, 4, 2, &lds, nvfp4 ? 1 : 0)) return false;
  p.K = L;
  if (route_sum ? !finalize(p, T * K, 8, 1, &lds, 0, kRouteSumRowsLds, 1) : !finalize(p, T, 8, 1, &lds, 0, 40 * 1024, 1))
    return false;
  return L % 16 == 0 && H % 16 == 0 && I % 16 == 0 && lds <= 80 * 1024;
}

hipError_t launch_decode_layer(const DecodeLayer& d, hipStream_t st) {
  const int T = d.T, H = d.H, L = d.L, I = d.I, E = d.E, K = d.K;
  const bool rs = d.rows16 != nullptr;
  if (!decode_layer_ok(T, H, L, I, E, K, d.nvfp4, rs)) return hipErrorInvalidValue;
  DecodeArgs a{};
  size_t lds = 0;
  // phase 1: the pooler (dense, A = x)
  SkinnyArgs& pl = a.pool;
  pl.a = d.x;
  pl.a_bytes = static_cast<uint32_t>(static_cast<size_t>(T) * H * 2);
  pl.b_bf16 = d.pooler;
  pl.out = d.lat;
  pl.ldo = L;
  pl.K = H;
  pl.m_total = T;
  pl.n_groups = L / 16;
  finalize(pl, T, 8, 1, &lds);
  a.n_pool = pl.n_groups;  // one group per workgroup (K split 8 ways)
  // phase 2: gate/up
  SkinnyArgs& gu = a.gateup;
  gu.a = d.lat;
  gu.a_bytes = static_cast<uint32_t>(static_cast<size_t>(T) * L * 2);
  gu.a_gather = 1;
  gu.sorted = d.sorted;
  gu.topk = K;
  gu.active = d.active;
  gu.b_codes = d.w13_codes;
  gu.b_scales = d.w13_scales;
  gu.b_global = d.w13_global;
  gu.b_rows_per_expert = 2 * I;
  gu.K = L;
  gu.inter = I;
  gu.out = d.h;
  gu.ldo = I;
  gu.n_groups = I / 16;
  gu.n_experts = E;
  gu.n_routes = T * K;
  finalize(gu, T, 4, 2, &lds, d.nvfp4 ? 1 : 0);
  const int max_active = T * K < E ? T * K : E;
  a.gu_gx = gu.n_groups / 2;
  a.n_gu = a.gu_gx * max_active;
  // phase 3: down
  SkinnyArgs& dn = a.down;
  dn.a = d.h;
  dn.a_bytes = static_cast<uint32_t>(static_cast<size_t>(T) * K * I * 2);
  dn.sorted = d.sorted;
  dn.topk = K;
  dn.active = d.active;
  dn.b_codes = d.w2_codes;
  dn.b_scales = d.w2_scales;
  dn.b_global = d.w2_global;
  dn.b_rows_per_expert = L;
  dn.K = I;
  dn.out = d.rows;
  dn.ldo = L;
  dn.n_groups = L / 32;
  dn.ssp = d.ssp;
  dn.out_scaled = d.rows16;
  dn.gain = d.gain;
  dn.gain_per_expert = d.gain_per_expert;
  dn.n_experts = E;
  dn.n_routes = T * K;
  finalize(dn, T, 4, 2, &lds, d.nvfp4 ? 1 : 0);
  a.dn_gx = dn.n_groups / 2;
  a.n_dn = a.dn_gx * max_active;
  // phase 5: unpooler (dense, A = y; rs: A = the T*K gain-scaled route rows)
  SkinnyArgs& up = a.unpool;
  const int up_rows = rs ? T * K : T;
  up.a = rs ? d.rows16 : d.y;
  up.a_bytes = static_cast<uint32_t>(static_cast<size_t>(up_rows) * L * 2);
  up.b_bf16 = d.unpooler;
  up.out = d.out;
  up.ldo = H;
  up.K = L;
  up.m_total = up_rows;
  up.n_groups = H / 16;
  up.topk = K;
  up.ssp = d.ssp;
  up.route_w = d.w;
  up.norm_eps = d.eps;
  if (rs)
    finalize(up, up_rows, 8, 1, &lds, 0, kRouteSumRowsLds, 1);
  else
    finalize(up, T, 8, 1, &lds, 0, 40 * 1024, 1);
  a.n_unpool = up.n_groups;
  // phase 4 and the rest
  a.comb_cb = (L + 64 * kDW - 1) / (64 * kDW);
  a.n_comb = T * a.comb_cb;
  a.x = d.x;
  a.router = d.router;
  a.logits = d.logits;
  a.tagged = d.tagged;
  a.T = T;
  a.H = H;
  a.E = E;
  a.K = K;
  a.L = L;
  a.ids = d.ids;
  a.w = d.w;
  a.offsets = d.offsets;
  a.sorted = d.sorted;
  a.active = d.active;
  a.counters = d.counters;
  a.tiles = d.tiles;
  a.rows = d.rows;
  a.ssp = d.ssp;
  a.gain = d.gain;
  a.gpe = d.gain_per_expert;
  a.eps = d.eps;
  a.y = d.y;
  a.sync = d.sync;
  a.slots = d.slots;
  a.grp = d.grp;
  a.rel = d.rel;
  // the grid: every workgroup resident at once
  // (NVFP4 in the streaming kernels' few-rows forms, as the per-step
  // launches take it for one or two tokens)
  if (d.nvfp4 && T != 1 && rs) return hipErrorInvalidValue;  // (the few-rows form keeps the combine)
  const void* kern = d.nvfp4 ? (T == 1 ? (rs ? kernel_of<B_NVFP4_ONE, 1, true>() : kernel_of<B_NVFP4_ONE, 1, false>())
                                      : kernel_of<B_NVFP4_FEW, 2, false>())
                             : (T == 1 ? (rs ? kernel_of<B_MXFP4, 1, true>() : kernel_of<B_MXFP4, 1, false>())
                                       : (rs ? kernel_of<B_MXFP4, 2, true>() : kernel_of<B_MXFP4, 2, false>()));
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kDW, lds);
  if (e != hipSuccess) return e;
  // (two workgroups per CU: the kernel's register budget; never more than the
  // occupancy query reports)
  const int capacity = cus * (per_cu < 2 ? per_cu : 2);
  if (capacity < 1 || capacity > kDecodeMaxWorkers) return hipErrorInvalidValue;
  a.G = capacity;
  if (d.nvfp4) {
    if (T != 1) return rs ? hipErrorInvalidValue : launch_decode<B_NVFP4_FEW, 2, false>(a, lds, st);
    return rs ? launch_decode<B_NVFP4_ONE, 1, true>(a, lds, st) : launch_decode<B_NVFP4_ONE, 1, false>(a, lds, st);
  }
  if (T != 1) return rs ? launch_decode<B_MXFP4, 2, true>(a, lds, st) : launch_decode<B_MXFP4, 2, false>(a, lds, st);
  return rs ? launch_decode<B_MXFP4, 1, true>(a, lds, st) : launch_decode<B_MXFP4, 1, false>(a, lds, st);
}

}  // namespace moe
