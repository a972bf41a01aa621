// moe_api.hip -- the C ABI declared in include/moe.h: argument checks,
// workspace plan and the launch sequence of the latent MoE layer.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"
#include <algorithm>
#include <atomic>
#include <mutex>
#include "moe.h"

// The workspace of moe_latent_forward_noalloc: one array per GPU, for the
// life of the process. Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;
thread_local moe::StageEvents g_stage_events;

constexpr size_t kAlign = 256;
constexpr int kSmallT = 16;  // routing in two launches (one-pass router, fused top-K + grouping)
constexpr int kPersistentMaxT = 2;  // tokens the persistent decode layer takes

// Projection regime, a function of the shapes only. Tiled (LDS-staged A,
// 128-row tiles) when the weights see many rows: pooler/unpooler for T > 16
// (at T = 32 the streaming kernels re-read their 32 activation rows from L2
// for every weight fragment; the tiled kernel with a 16-way K split took the
// pooler 30.0 -> 23.8 us and the unpooler 25.1 -> 22.0 us, the step 0.960 ->
// 0.948 ms),
// experts when the routes average at least 16 rows per expert; streaming
// kernels otherwise. The tiled kernels need the output widths to be
// multiples of their column tiles and K to be a multiple of 256.
bool dense_tiled(int T, int N, int K) { return T > 16 && N % 128 == 0 && K % 256 == 0; }
bool experts_tiled(const moe_dims* d, int T) {
  return static_cast<int64_t>(T) * d->top_k >= 16 * static_cast<int64_t>(d->n_experts) &&
         d->inter % 256 == 0 && d->latent % 256 == 0;
}
// The LDS-staged expert kernel (128-row tiles, eight wavefronts, two
// workgroups per CU for MXFP4, one for NVFP4) whenever its widths allow (K a
// multiple of 512; MXFP4 at most 4096); the register-staged kernel (64-row
// tiles) otherwise. Measured on the
// skewed T = 512 workload (about 16 routes per expert): 2.03 ms against
// 2.25 ms with the register-staged kernel.
bool experts_lds(const moe_dims* d, int T) {
  return experts_tiled(d, T) &&
         moe::expert_lds_ok(d->latent, d->inter, d->expert_format == MOE_FMT_NVFP4);
}
// The expert projections' two loops on the row-tile regime (moe_dims::
// expert_split_rows): the rows at or below which an expert streams its
// weights on the streaming kernels, 0 for one loop.
constexpr int kDefaultSplitRows = 0;
int split_rows(const moe_dims* d, int T) {
  if (!experts_tiled(d, T) || d->expert_split_rows < 0) return 0;
  return d->expert_split_rows > 0 ? d->expert_split_rows : kDefaultSplitRows;
}
// The router runs in the pooler's launch for T <= 16 (the streaming pooler:
// the tiled one starts above 32 tokens); for T <= 8 tokens with at most 64
// routes its workgroups also route (one wavefront per token, the grouping by
// one wavefront).
bool pool_with_router(int T, const moe_dims*) { return T <= kSmallT; }
// Few route rows on the streaming expert kernels: the post-norm, the
// weighted sum and the unpooler in one launch (the weighted sum after the
// unpooler's products; gemm_skinny.hip, launch_unpool_routes), y not written.
bool route_sum(const moe_dims* d, int T) {
  return T <= kSmallT && !experts_tiled(d, T) && moe::route_sum_ok(T, d->top_k, d->latent, d->hidden) &&
         moe::down_scaled_ok(T, d->inter, d->expert_format == MOE_FMT_NVFP4);
}
bool route_in_router(const moe_dims* d, int T) {
  return pool_with_router(T, d) && T <= 8 && T * d->top_k <= 64;
}
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (!(d->norm_eps >= 0.0f) || !isfinite(d->norm_eps)) return MOE_EINVAL;
  if (d->gain_per_expert != 0 && d->gain_per_expert != 1) return MOE_EINVAL;
  if (d->expert_format != MOE_FMT_MXFP4 && d->expert_format != MOE_FMT_NVFP4) return MOE_EINVAL;
  if (d->expert_split_rows < -1 || d->expert_split_rows > moe::kMaxSplitRows) return MOE_EINVAL;
  if (d->hidden <= 0 || d->latent <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0)
    return MOE_EINVAL;
  if (d->hidden % 128 || d->latent % 128 || d->inter % 128) return MOE_EUNSUPPORTED;
  if (d->latent > 8192 || d->hidden > 65536 || d->inter > 65536) return MOE_EUNSUPPORTED;
  if (d->n_experts > 256 || d->top_k > 8 || d->top_k > d->n_experts) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// The kernels address the token-sized tensors they read through buffer
// descriptors with 32-bit byte offsets, 2^31 marking "out of range": the
// layer input (and the block's pre-norm output) T*H*2 bytes, the latent rows
// and y T*L*2, h T*K*I*2 must each stay below 2^31 bytes (T <= 32767 at the
// real shape, set by h).
int check_tokens(const moe_dims* d, int32_t T) {
  if (T < 0) return MOE_EINVAL;
  const int64_t t = T, lim = int64_t{1} << 31;
  if (t * d->top_k >= (int64_t{1} << 28)) return MOE_EUNSUPPORTED;
  if (t * d->hidden * 2 >= lim || t * d->latent * 2 >= lim ||
      t * d->top_k * d->inter * 2 >= lim)
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Placement of every buffer of one call inside the workspace, and the
// launch shapes that depend on T.
struct Plan {
  int splits, tile_m, max_tiles, max_active;
  size_t sync, tagged;  // generation word; the tagged logits (routing in the router launch)
  size_t partial, logits, ids, w, offsets, sorted, active, counters, tiles, lat, h, rows, ssp, y;
  size_t rows16;             // the gain-scaled bf16 route rows (steps A7 and A8 in one launch)
  size_t dpart;              // fp32 partial sums of a K-split dense projection (prefill, few tiles)
  size_t ccount;             // per-chunk expert counts of a grouping over several workgroups
  size_t nf32, nbf16, fout;  // the block only: pre-norm outputs, the layer's output
  size_t pbar;               // the persistent decode layer: arrival slots, group and release words
  size_t total;
};

// block: also the buffers of moe_block_forward (after all the others, so
// the layer's views keep their offsets)
Plan make_plan(const moe_dims* d, int32_t T, bool block = false) {
  const int H = d->hidden, L = d->latent, I = d->inter, E = d->n_experts, K = d->top_k;
  const size_t R = static_cast<size_t>(T) * K;
  Plan p{};
  // Router (T > 16): split H so that about 2048 wavefronts share the fp64
  // MFMA work (64 tokens x 64 experts each), at most 64 splits; a split is a
  // whole number of 32-element blocks.
  const int nt = (T + 63) / 64, ne = (E + 63) / 64, hc = H / 32;
  int64_t cap = 2048 / (static_cast<int64_t>(nt) * ne);
  if (cap > 64) cap = 64;
  if (cap > hc) cap = hc;
  if (cap < 1) cap = 1;
  p.splits = static_cast<int>(cap);
  while (hc % p.splits) --p.splits;
  // rows per tile of the prefill expert projections (the LDS-staged kernel
  // takes 128-row tiles, the register-staged one 64)
  p.tile_m = experts_lds(d, T) ? moe::kExpertTileRows : moe::kTileRows;
  p.max_active = static_cast<int>(R < static_cast<size_t>(E) ? R : E);
  p.max_tiles = static_cast<int>(R / p.tile_m) + p.max_active + 1;

  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  // first, at a fixed place whatever T: the words that carry over between calls
  p.sync = take(256);
  p.tagged = take(route_in_router(d, T) ? sizeof(uint64_t) * static_cast<size_t>(T) * E : 0);
  p.partial = take(T > kSmallT ? sizeof(double) * p.splits * static_cast<size_t>(T) * E : 0);
  p.logits = take(sizeof(float) * static_cast<size_t>(T) * E);
  p.ids = take(sizeof(int32_t) * R);
  p.w = take(sizeof(float) * R);
  p.offsets = take(sizeof(int32_t) * (E + 1));
  p.sorted = take(sizeof(int32_t) * R);
  p.active = take(sizeof(int32_t) * 4 * E);  // (expert, first row, end row, unused) per touched expert
  p.counters = take(sizeof(int32_t) * 4);
  p.tiles = take(sizeof(int32_t) * 2 * static_cast<size_t>(p.max_tiles));
  p.lat = take(sizeof(uint16_t) * static_cast<size_t>(T) * L);
  p.h = take(sizeof(uint16_t) * R * I);
  p.rows = take(sizeof(float) * R * L);
  p.ssp = take(T <= kSmallT && !experts_tiled(d, T) ? sizeof(float) * R * (L / 32) : 0);
  p.y = take(sizeof(uint16_t) * static_cast<size_t>(T) * L);
  p.rows16 = take(route_sum(d, T) ? sizeof(uint16_t) * R * L : 0);
  size_t dpart = 0;
  if (dense_tiled(T, L, H) && moe::dense_splits(T, L, H) > 1)
    dpart = static_cast<size_t>(moe::dense_splits(T, L, H)) * T * L;
  if (dense_tiled(T, H, L) && moe::dense_splits(T, H, L) > 1)
    dpart = std::max(dpart, static_cast<size_t>(moe::dense_splits(T, H, L)) * T * H);
  p.dpart = take(sizeof(float) * dpart);
  p.ccount = take(sizeof(int32_t) * static_cast<size_t>(moe::permute_chunks(static_cast<int>(R))) * E);
  p.pbar = take(T <= kPersistentMaxT ? 4 * moe::kDecodeMaxWorkers + 16 * 128 : 0);
  const size_t th = block ? static_cast<size_t>(T) * H : 0;
  p.nf32 = take(sizeof(float) * th);
  p.nbf16 = take(sizeof(uint16_t) * th);
  p.fout = take(sizeof(uint16_t) * th);
  p.total = o;
  return p;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(e);
  return MOE_EHIP;
}

template <typename P>
int need_ptr(P* ptr) {
  if (!ptr) return MOE_EINVAL;
  if (!aligned16(ptr)) return MOE_EALIGN;
  return MOE_OK;
}

#define MOE_TRY(expr)              \
  do {                             \
    const int rc_ = (expr);        \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

}  // namespace

namespace moe {
StageEvents& stage_events() { return g_stage_events; }
}  // namespace moe

extern "C" {

size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_tokens) {
  if (check_dims(dims) != MOE_OK || check_tokens(dims, max_tokens) != MOE_OK) return 0;
  return make_plan(dims, max_tokens).total;
}

int moe_route_validate(const moe_dims* dims, int32_t T, const uint16_t* x, const float* router,
                       const int32_t* topk_ids, const float* topk_w,
                       const int32_t* expert_offsets, const int32_t* sorted_routes,
                       const float* logits_out, const void* workspace, size_t workspace_bytes) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(dims, T));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_ptr(x));
  MOE_TRY(need_ptr(router));
  MOE_TRY(need_ptr(topk_ids));
  MOE_TRY(need_ptr(topk_w));
  MOE_TRY(need_ptr(expert_offsets));
  MOE_TRY(need_ptr(sorted_routes));
  if (logits_out) MOE_TRY(need_ptr(logits_out));
  MOE_TRY(need_ptr(workspace));
  if (workspace_bytes < make_plan(dims, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int moe_latent_forward_validate(const moe_dims* dims, int32_t T, const uint16_t* x,
                                const moe_weights* wts, const uint16_t* out,
                                const void* workspace, size_t workspace_bytes) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(dims, T));
  if (T == 0) return MOE_OK;
  if (!wts) return MOE_EINVAL;
  MOE_TRY(need_ptr(x));
  MOE_TRY(need_ptr(wts->router));
  MOE_TRY(need_ptr(wts->pooler));
  MOE_TRY(need_ptr(wts->w13_codes));
  MOE_TRY(need_ptr(wts->w13_scales));
  MOE_TRY(need_ptr(wts->w2_codes));
  MOE_TRY(need_ptr(wts->w2_scales));
  MOE_TRY(need_ptr(wts->norm_gain));
  MOE_TRY(need_ptr(wts->unpooler));
  if (dims->expert_format == MOE_FMT_NVFP4) {
    MOE_TRY(need_ptr(wts->w13_global));
    MOE_TRY(need_ptr(wts->w2_global));
  }
  MOE_TRY(need_ptr(out));
  MOE_TRY(need_ptr(workspace));
  if (workspace_bytes < make_plan(dims, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int moe_route(const moe_dims* dims, int32_t T, const uint16_t* x, const float* router,
              int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_routes,
              float* logits_out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(moe_route_validate(dims, T, x, router, topk_ids, topk_w, expert_offsets, sorted_routes,
                             logits_out, workspace, workspace_bytes));
  if (T == 0) return MOE_OK;
  const Plan p = make_plan(dims, T);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int H = dims->hidden, E = dims->n_experts, K = dims->top_k;
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + p.logits);
  double* partial = reinterpret_cast<double*>(ws + p.partial);
  int32_t* active = reinterpret_cast<int32_t*>(ws + p.active);
  int32_t* counters = reinterpret_cast<int32_t*>(ws + p.counters);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + p.tiles);
  if (T <= kSmallT) {
    MOE_TRY(hip_status(moe::launch_router_gemv(x, router, logits, T, H, E, st)));
    MOE_TRY(hip_status(moe::launch_route_small(logits, T, E, K, topk_ids, topk_w, expert_offsets,
                                               sorted_routes, active, counters, tiles, p.tile_m,
                                               st)));
  } else {
    MOE_TRY(hip_status(moe::launch_router_logits(x, router, partial, T, H, E, p.splits, st)));
    MOE_TRY(hip_status(moe::launch_topk(partial, p.splits, T, E, K, logits, topk_ids, topk_w, st)));
    MOE_TRY(hip_status(moe::launch_permute(topk_ids, T * K, E, expert_offsets, sorted_routes,
                                           active, counters, tiles, p.tile_m, st, nullptr,
                                           reinterpret_cast<int32_t*>(ws + p.ccount))));
  }
  return MOE_OK;
}

}  // extern "C"

namespace {

// The block around the layer: out = resid + post_norm(layer(pre_norm(resid)))
struct Block {
  const uint16_t* resid;
  const uint16_t* pre_gain;
  const uint16_t* post_gain;
  double eps;
};

// The launch sequence of the layer. With given_ids / given_w (routing
// replay) steps 1 and 2 are skipped: the grouping reads the caller's ids
// (clamped into [0, E), copied to the workspace for the combine) and the
// combine reads the caller's weights. With a block, the pre-norm runs first
// (its fp32 output feeds the router, its bf16 output the pooler), the layer
// writes its output to the workspace, and the post-norm plus the residual
// write `out`.
int forward_impl(const moe_dims* dims, int32_t T, const uint16_t* x, const moe_weights* wts,
                 uint16_t* out, void* workspace, void* hip_stream, void* const* stage_events,
                 const int32_t* given_ids, const float* given_w, const Block* blk = nullptr) {
  const Plan p = make_plan(dims, T, blk != nullptr);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int H = dims->hidden, L = dims->latent, I = dims->inter, E = dims->n_experts,
            K = dims->top_k;
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  // Stage i's kernel records events 2i and 2i+1 at its own start and end
  // (hipExtLaunchKernel); a step without a kernel records both back to back.
  bool launched = false;
  auto mark = [&](int i) -> int {
    int rc = MOE_OK;
    if (stage_events && i > 0) {  // close stage i-1
      hipEvent_t a = static_cast<hipEvent_t>(stage_events[2 * (i - 1)]);
      hipEvent_t b = static_cast<hipEvent_t>(stage_events[2 * (i - 1) + 1]);
      if (!launched && a) rc = hip_status(hipEventRecord(a, st));
      if (rc == MOE_OK && !launched && b) rc = hip_status(hipEventRecord(b, st));
    }
    g_stage_events = moe::StageEvents{};
    launched = false;
    if (stage_events && i < MOE_N_STAGES) {
      g_stage_events.start = static_cast<hipEvent_t>(stage_events[2 * i]);
      g_stage_events.stop = static_cast<hipEvent_t>(stage_events[2 * i + 1]);
    }
    return rc;
  };
  auto ran = [&](hipError_t e) -> int {
    launched = true;
    const int rc = hip_status(e);
    if (rc != MOE_OK) g_stage_events = moe::StageEvents{};
    return rc;
  };
  double* partial = static_cast<double*>(at(p.partial));
  float* logits = static_cast<float*>(at(p.logits));
  int32_t* ids = static_cast<int32_t*>(at(p.ids));
  float* w = given_w ? const_cast<float*>(given_w) : static_cast<float*>(at(p.w));
  const bool routed = given_ids != nullptr;
  int32_t* offsets = static_cast<int32_t*>(at(p.offsets));
  int32_t* sorted = static_cast<int32_t*>(at(p.sorted));
  int32_t* active = static_cast<int32_t*>(at(p.active));
  int32_t* counters = static_cast<int32_t*>(at(p.counters));
  int32_t* tiles = static_cast<int32_t*>(at(p.tiles));
  uint16_t* lat = static_cast<uint16_t*>(at(p.lat));
  uint16_t* h = static_cast<uint16_t*>(at(p.h));
  float* rows = static_cast<float*>(at(p.rows));
  const bool tiled = experts_tiled(dims, T);
  // per-32-column sums of squares of the route rows (streaming down kernel, few tokens)
  float* ssp = (T <= kSmallT && !tiled) ? static_cast<float*>(at(p.ssp)) : nullptr;
  uint16_t* y = static_cast<uint16_t*>(at(p.y));

  moe::ExpertGemm eg{};
  eg.lat = lat;
  eg.sorted = sorted;
  eg.offsets = offsets;
  eg.active = active;
  eg.counters = counters;
  eg.tiles = tiles;
  eg.w13_codes = wts->w13_codes;
  eg.w13_scales = wts->w13_scales;
  eg.w2_codes = wts->w2_codes;
  eg.w2_scales = wts->w2_scales;
  eg.h = h;
  eg.rows = rows;
  eg.ssp = ssp;
  eg.tokens = T;
  eg.topk = K;
  eg.latent = L;
  eg.inter = I;
  eg.n_experts = E;
  eg.max_active = p.max_active;
  eg.max_tiles = p.max_tiles;
  eg.nvfp4 = dims->expert_format == MOE_FMT_NVFP4;
  eg.w13_global = wts->w13_global;
  eg.w2_global = wts->w2_global;
  const bool rsum = route_sum(dims, T);
  uint16_t* rows16 = rsum ? static_cast<uint16_t*>(at(p.rows16)) : nullptr;
  eg.rows16 = rows16;
  eg.gain = wts->norm_gain;
  eg.gain_per_expert = dims->gain_per_expert;

  // the block's pre-norm: the router reads its fp32 output, the pooler its bf16 one.
  // With few tokens (every row staged by the pooler in one pass) the
  // router + pooler launch normalises the residual stream itself.
  const float* x_f32 = nullptr;
  uint16_t* layer_out = out;
  moe::PreNormFold pre{};
  const bool pre_folded = blk && !given_ids && T <= kSmallT && moe::prenorm_fold_ok(T, H);
  if (blk) {
    float* nf = static_cast<float*>(at(p.nf32));
    uint16_t* nb = static_cast<uint16_t*>(at(p.nbf16));
    if (pre_folded) {
      pre = moe::PreNormFold{blk->pre_gain, blk->eps, nf, nb};
    } else {
      MOE_TRY(hip_status(moe::launch_pre_norm(blk->resid, blk->pre_gain, blk->eps, T, H, nf, nb, st)));
      x_f32 = nf;
      x = nb;
    }
    layer_out = static_cast<uint16_t*>(at(p.fout));
  }

  MOE_TRY(mark(0));
  // few tokens: the router runs inside the pooler's launch (timed as step 0;
  // step 3 then has no kernel of its own), and for T <= 8 the top K and the
  // grouping too (steps 1 and 2 without kernels)
  const bool with_router = !routed && pool_with_router(T, dims);
  const bool fused_route = with_router && route_in_router(dims, T);
  moe::RouteFuse rf{};
  if (fused_route) {
    uint32_t* sync = static_cast<uint32_t*>(at(p.sync));
    rf = moe::RouteFuse{static_cast<uint64_t*>(at(p.tagged)), sync, sync + 1, K, ids, w, offsets,
                        sorted, active, counters, tiles};
  }
  if (routed) {
    MOE_TRY(mark(1));
    MOE_TRY(mark(2));
    MOE_TRY(ran(moe::launch_permute(given_ids, T * K, E, offsets, sorted, active, counters, tiles,
                                    p.tile_m, st, ids, static_cast<int32_t*>(at(p.ccount)))));
  } else if (T <= kSmallT) {
    MOE_TRY(ran(moe::launch_pool_router(x, wts->pooler, lat, T, L, H, wts->router, logits, E, st,
                                        x_f32, fused_route ? &rf : nullptr,
                                        pre_folded ? &pre : nullptr)));
    MOE_TRY(mark(1));
    if (!fused_route)
      MOE_TRY(ran(moe::launch_route_small(logits, T, E, K, ids, w, offsets, sorted, active,
                                          counters, tiles, p.tile_m, st)));
    MOE_TRY(mark(2));
  } else {
    MOE_TRY(ran(x_f32 ? moe::launch_router_logits(x_f32, wts->router, partial, T, H, E, p.splits, st)
                      : moe::launch_router_logits(x, wts->router, partial, T, H, E, p.splits, st)));
    MOE_TRY(mark(1));
    MOE_TRY(ran(moe::launch_topk(partial, p.splits, T, E, K, logits, ids, w, st)));
    MOE_TRY(mark(2));
    MOE_TRY(ran(moe::launch_permute(ids, T * K, E, offsets, sorted, active, counters, tiles,
                                    p.tile_m, st, nullptr, static_cast<int32_t*>(at(p.ccount)))));
  }
  MOE_TRY(mark(3));
  if (!with_router)
    MOE_TRY(ran(dense_tiled(T, L, H) ? moe::launch_dense_tiled(x, wts->pooler, lat, T, L, H, st,
                                                                static_cast<float*>(at(p.dpart)))
                                   : moe::launch_dense_skinny(x, wts->pooler, lat, T, L, H, st)));
  MOE_TRY(mark(4));
  const bool lds = experts_lds(dims, T);
  eg.split_rows = split_rows(dims, T);
  // the light experts first (two loops): the stage's start event at their
  // launch, its end at the row tiles'
  auto light = [&](hipError_t (*launch)(const moe::ExpertGemm&, hipStream_t)) -> int {
    if (eg.split_rows == 0) return MOE_OK;
    const hipEvent_t stop = g_stage_events.stop;
    g_stage_events.stop = nullptr;
    const int rc = ran(launch(eg, st));
    g_stage_events.start = nullptr;
    if (rc == MOE_OK) g_stage_events.stop = stop;
    return rc;
  };
  MOE_TRY(light(moe::launch_gateup_skinny));
  MOE_TRY(ran(lds ? moe::launch_gateup_expert(eg, st)
                  : tiled ? moe::launch_gateup_tiled(eg, st) : moe::launch_gateup_skinny(eg, st)));
  MOE_TRY(mark(5));
  MOE_TRY(light(moe::launch_down_skinny));
  MOE_TRY(ran(lds ? moe::launch_down_expert(eg, st)
                  : tiled ? moe::launch_down_tiled(eg, st) : moe::launch_down_skinny(eg, st)));
  MOE_TRY(mark(6));
  if (rsum) {  // (step 6 without a kernel of its own: the unpooler's launch takes it)
    MOE_TRY(mark(7));
    MOE_TRY(ran(moe::launch_unpool_routes(rows16, ssp, w, dims->norm_eps, T, K, L, H, wts->unpooler,
                                          layer_out, st)));
  } else {
    MOE_TRY(ran(ssp ? moe::launch_combine_cols(rows, ssp, w, ids, wts->norm_gain, dims->gain_per_expert,
                                               dims->norm_eps, T, K, L, y, st)
                    : moe::launch_combine(rows, w, ids, wts->norm_gain, dims->gain_per_expert,
                                          dims->norm_eps, T, K, L, y, st)));
    MOE_TRY(mark(7));
    MOE_TRY(ran(dense_tiled(T, H, L) ? moe::launch_dense_tiled(y, wts->unpooler, layer_out, T, H, L, st,
                                                                static_cast<float*>(at(p.dpart)))
                                   : moe::launch_dense_skinny(y, wts->unpooler, layer_out, T, H, L, st)));
  }
  MOE_TRY(mark(8));
  if (blk)
    MOE_TRY(hip_status(moe::launch_post_norm_residual(blk->resid, layer_out, blk->post_gain, blk->eps,
                                                      T, H, out, st)));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_latent_forward_timed(const moe_dims* dims, int32_t T, const uint16_t* x,
                             const moe_weights* wts, uint16_t* out, void* workspace,
                             size_t workspace_bytes, void* hip_stream, void* const* stage_events) {
  MOE_TRY(moe_latent_forward_validate(dims, T, x, wts, out, workspace, workspace_bytes));
  if (T == 0) return MOE_OK;
  return forward_impl(dims, T, x, wts, out, workspace, hip_stream, stage_events, nullptr, nullptr);
}

int moe_latent_forward(const moe_dims* dims, int32_t T, const uint16_t* x, const moe_weights* wts,
                       uint16_t* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return moe_latent_forward_timed(dims, T, x, wts, out, workspace, workspace_bytes, hip_stream,
                                  nullptr);
}

int moe_latent_forward_routed_validate(const moe_dims* dims, int32_t T, const uint16_t* x,
                                       const int32_t* topk_ids, const float* topk_w,
                                       const moe_weights* wts, const uint16_t* out,
                                       const void* workspace, size_t workspace_bytes) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(dims, T));
  if (T == 0) return MOE_OK;
  if (!wts) return MOE_EINVAL;
  MOE_TRY(need_ptr(x));
  MOE_TRY(need_ptr(topk_ids));
  MOE_TRY(need_ptr(topk_w));
  MOE_TRY(need_ptr(wts->pooler));
  MOE_TRY(need_ptr(wts->w13_codes));
  MOE_TRY(need_ptr(wts->w13_scales));
  MOE_TRY(need_ptr(wts->w2_codes));
  MOE_TRY(need_ptr(wts->w2_scales));
  MOE_TRY(need_ptr(wts->norm_gain));
  MOE_TRY(need_ptr(wts->unpooler));
  if (dims->expert_format == MOE_FMT_NVFP4) {
    MOE_TRY(need_ptr(wts->w13_global));
    MOE_TRY(need_ptr(wts->w2_global));
  }
  MOE_TRY(need_ptr(out));
  MOE_TRY(need_ptr(workspace));
  if (workspace_bytes < make_plan(dims, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

size_t moe_block_workspace_bytes(const moe_dims* dims, int32_t max_tokens) {
  if (check_dims(dims) != MOE_OK || check_tokens(dims, max_tokens) != MOE_OK) return 0;
  return make_plan(dims, max_tokens, true).total;
}

int moe_block_forward_validate(const moe_dims* dims, int32_t T, const uint16_t* resid,
                               const uint16_t* pre_gain, const uint16_t* post_gain, float block_eps,
                               const moe_weights* wts, const uint16_t* out, const void* workspace,
                               size_t workspace_bytes) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(dims, T));
  if (!(block_eps >= 0.0f) || !isfinite(block_eps)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  MOE_TRY(need_ptr(pre_gain));
  MOE_TRY(need_ptr(post_gain));
  // the layer's own checks, with the residual stream as its input
  MOE_TRY(moe_latent_forward_validate(dims, T, resid, wts, out, workspace, workspace_bytes));
  if (workspace_bytes < make_plan(dims, T, true).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

int moe_block_forward(const moe_dims* dims, int32_t T, const uint16_t* resid,
                      const uint16_t* pre_gain, const uint16_t* post_gain, float block_eps,
                      const moe_weights* wts, uint16_t* out, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(moe_block_forward_validate(dims, T, resid, pre_gain, post_gain, block_eps, wts, out,
                                     workspace, workspace_bytes));
  if (T == 0) return MOE_OK;
  const Block blk{resid, pre_gain, post_gain, static_cast<double>(block_eps)};
  return forward_impl(dims, T, resid, wts, out, workspace, hip_stream, nullptr, nullptr, nullptr,
                      &blk);
}

int moe_latent_forward_routed(const moe_dims* dims, int32_t T, const uint16_t* x,
                              const int32_t* topk_ids, const float* topk_w,
                              const moe_weights* wts, uint16_t* out, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(moe_latent_forward_routed_validate(dims, T, x, topk_ids, topk_w, wts, out, workspace,
                                             workspace_bytes));
  if (T == 0) return MOE_OK;
  return forward_impl(dims, T, x, wts, out, workspace, hip_stream, nullptr, topk_ids, topk_w);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (!p) return MOE_EHIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_latent_forward_noalloc(const moe_dims* dims, int32_t T, const uint16_t* x,
                               const moe_weights* wts, uint16_t* out, void* hip_stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(dims, T));
  if (T == 0) return MOE_OK;
  if (make_plan(dims, T).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  void* ws = nullptr;
  MOE_TRY(scratch_ptr(&ws));
  MOE_TRY(moe_latent_forward_validate(dims, T, x, wts, out, ws, MOE_NOALLOC_SCRATCH_BYTES));
  return forward_impl(dims, T, x, wts, out, ws, hip_stream, nullptr, nullptr, nullptr);
}

int moe_latent_forward_persistent(const moe_dims* dims, int32_t T, const uint16_t* x,
                                  const moe_weights* wts, uint16_t* out, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  MOE_TRY(moe_latent_forward_validate(dims, T, x, wts, out, workspace, workspace_bytes));
  if (T == 0) return MOE_OK;
  if (T > kPersistentMaxT || !route_in_router(dims, T) ||
      !moe::decode_layer_ok(T, dims->hidden, dims->latent, dims->inter, dims->n_experts, dims->top_k,
                            dims->expert_format == MOE_FMT_NVFP4, route_sum(dims, T)))
    return MOE_EUNSUPPORTED;
  const Plan p = make_plan(dims, T);
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  moe::DecodeLayer d{};
  d.T = T;
  d.H = dims->hidden;
  d.L = dims->latent;
  d.I = dims->inter;
  d.E = dims->n_experts;
  d.K = dims->top_k;
  d.nvfp4 = dims->expert_format == MOE_FMT_NVFP4;
  d.gain_per_expert = dims->gain_per_expert;
  d.eps = dims->norm_eps;
  d.x = x;
  d.router = wts->router;
  d.pooler = wts->pooler;
  d.w13_codes = wts->w13_codes;
  d.w13_scales = wts->w13_scales;
  d.w13_global = wts->w13_global;
  d.w2_codes = wts->w2_codes;
  d.w2_scales = wts->w2_scales;
  d.w2_global = wts->w2_global;
  d.gain = wts->norm_gain;
  d.unpooler = wts->unpooler;
  d.out = out;
  d.logits = static_cast<float*>(at(p.logits));
  d.tagged = static_cast<uint64_t*>(at(p.tagged));
  d.ids = static_cast<int32_t*>(at(p.ids));
  d.w = static_cast<float*>(at(p.w));
  d.offsets = static_cast<int32_t*>(at(p.offsets));
  d.sorted = static_cast<int32_t*>(at(p.sorted));
  d.active = static_cast<int32_t*>(at(p.active));
  d.counters = static_cast<int32_t*>(at(p.counters));
  d.tiles = static_cast<int32_t*>(at(p.tiles));
  d.lat = static_cast<uint16_t*>(at(p.lat));
  d.h = static_cast<uint16_t*>(at(p.h));
  d.rows = static_cast<float*>(at(p.rows));
  d.ssp = static_cast<float*>(at(p.ssp));
  d.y = static_cast<uint16_t*>(at(p.y));
  d.rows16 = route_sum(dims, T) ? static_cast<uint16_t*>(at(p.rows16)) : nullptr;  // (as moe_latent_forward)
  d.sync = static_cast<uint32_t*>(at(p.sync));
  d.slots = static_cast<uint32_t*>(at(p.pbar));
  d.grp = static_cast<uint32_t*>(at(p.pbar + 4 * moe::kDecodeMaxWorkers));
  d.rel = static_cast<uint32_t*>(at(p.pbar + 4 * moe::kDecodeMaxWorkers + 8 * 128));
  return hip_status(moe::launch_decode_layer(d, static_cast<hipStream_t>(hip_stream)));
}

int moe_workspace_view(const moe_dims* dims, int32_t T, int32_t which, size_t* offset,
                       size_t* bytes) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(dims, T));
  if (!offset || !bytes) return MOE_EINVAL;
  const Plan p = make_plan(dims, T);
  const size_t R = static_cast<size_t>(T) * dims->top_k;
  const size_t E = dims->n_experts, L = dims->latent, I = dims->inter, H = dims->hidden;
  switch (which) {
    case MOE_VIEW_LOGITS: *offset = p.logits; *bytes = 4 * T * E; break;
    case MOE_VIEW_IDS: *offset = p.ids; *bytes = 4 * R; break;
    case MOE_VIEW_WEIGHTS: *offset = p.w; *bytes = 4 * R; break;
    case MOE_VIEW_OFFSETS: *offset = p.offsets; *bytes = 4 * (E + 1); break;
    case MOE_VIEW_SORTED: *offset = p.sorted; *bytes = 4 * R; break;
    case MOE_VIEW_LATENT: *offset = p.lat; *bytes = 2 * T * L; break;
    case MOE_VIEW_H: *offset = p.h; *bytes = 2 * R * I; break;
    case MOE_VIEW_ROWS: *offset = p.rows; *bytes = 4 * R * L; break;
    case MOE_VIEW_Y: *offset = p.y; *bytes = 2 * T * L; break;
    case MOE_VIEW_NORM_F32: *offset = make_plan(dims, T, true).nf32; *bytes = 4 * T * H; break;
    case MOE_VIEW_NORM_BF16: *offset = make_plan(dims, T, true).nbf16; *bytes = 2 * T * H; break;
    case MOE_VIEW_LAYER_OUT: *offset = make_plan(dims, T, true).fout; *bytes = 2 * T * H; break;
    case MOE_VIEW_SYNC: *offset = p.sync; *bytes = 256; break;
    case MOE_VIEW_ROWS_BF16: *offset = p.rows16; *bytes = route_sum(dims, T) ? 2 * R * L : 0; break;
    default: return MOE_EINVAL;
  }
  return MOE_OK;
}

int moe_tile_map(int32_t kind, int32_t a, int32_t b, int32_t* out, int32_t capacity) {
  if (a <= 0 || b <= 0 || a > (1 << 20) || b > (1 << 16)) return MOE_EINVAL;
  if (kind == MOE_TILES_DENSE) {
    if (b % 256) return MOE_EINVAL;
    const int G = moe::dense_grid(a, b);
    if (out && capacity >= 2 * G)
      for (int i = 0; i < G; ++i) {
        const moe::TileRC t = moe::dense_tile_host(i, a, b);
        out[2 * i] = t.mt;
        out[2 * i + 1] = t.nt;
      }
    return G;
  }
  if (kind == MOE_TILES_EXPERT || kind == MOE_TILES_TILED) {
    const int chunk = (kind == MOE_TILES_EXPERT ? moe::expert_chunk_rows() : 1) * b;
    const int64_t n = static_cast<int64_t>(a) * b;
    if (n > (1 << 26)) return MOE_EINVAL;
    const int G = moe::xcd_grid(static_cast<int>(n), chunk);
    if (out && capacity >= 2 * G)
      for (int i = 0; i < G; ++i) {
        const int logical = moe::xcd_tile_of(i, chunk);
        out[2 * i] = logical / b;
        out[2 * i + 1] = logical % b;
      }
    return G;
  }
  return MOE_EINVAL;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, negative size, bad eps or flag)";
    case MOE_EUNSUPPORTED: return "unsupported dimensions";
    case MOE_EALIGN: return "pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
