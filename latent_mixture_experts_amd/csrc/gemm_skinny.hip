// gemm_skinny.hip -- projections for few rows per weight matrix (decode).
//
// C[rows][n] = sum_k A[row][k] * B[n][k] with A bf16 activations and B either
// a bf16 matrix (pooler, unpooler: steps A4, A8) or one expert's MXFP4 matrix
// (W13 and W2: steps A5, A6). With a handful of rows per weight matrix the
// work is bound by streaming B from HBM: every weight byte is read once, by
// one wavefront, which owns NF fragments of 16 B rows for its share of K and
// keeps U stages of weight loads in flight (software pipeline). All loads are
// raw buffer loads: a lane without a row gets zeros from an out-of-range
// offset, so the loop has no branches and the loads stay in flight.
//
// The A rows either stream through registers beside B, or (AL) are copied
// once per pass of 16 rows into LDS and read from there by every wavefront of
// the workgroup. A bf16 operand costs four times the registers of a 4-bit one
// (64 bytes per lane and 128-element chunk against 16), so staging A in LDS is
// what leaves room for several weight stages in flight: at one or two rows per
// expert the kernel is bound by how many weight bytes each compute unit keeps
// in flight against HBM latency.
//
// MXFP4 is decoded in registers: 16 code bytes per lane (32 elements, one
// E8M0 block) become four bf16x8 MFMA operands through the gfx950 scaled FP4
// conversion, so no bf16 copy of a weight ever reaches memory ("Muse Spark
// Open on Gaudi 2", section "What it taught about Gaudi", shows the cost of
// unpacking touched expert slices to bf16 in memory).
//
// Reduction order inside a 128-element chunk: lane group g = lane/16 owns
// elements [32g, 32g+32) (one E8M0 block); MFMA j takes elements 32g+8j .. +7
// from each group, for both operands, so A and B always pair the same k.
// The scale bytes of a row for two consecutive chunks are 8 contiguous bytes:
// each lane loads all 8 with one load and picks its own.
#include "device_common.h"
#include "kernels.h"
#include "route_small.h"
#include "router_gemv.h"
#include "stream_body.h"

#include <algorithm>

namespace moe {

namespace {

// The expert kernels keep two workgroups per CU (at most 128 VGPRs).
template <int BFMT, int EPI, int NF, int MB, int U, int KS, int SC, bool AL>
__global__ __launch_bounds__(64 * kWaves, is_fp4(BFMT) ? 4 : 1) void stream_kernel(SkinnyArgs p) {
  stream_body<BFMT, EPI, NF, MB, U, KS, SC, AL>(p, blockIdx.x, blockIdx.y);
}

// The router (T <= 16 tokens) and the pooler read only the layer input, so
// one launch runs both: workgroups 0 .. E-1 compute one expert's logits each
// (router_gemv.h, eight wavefronts), the rest are the pooler's streaming
// workgroups. The router's 8 MiB then streams beside the pooler's weights
// instead of in a launch of its own. The router reads the same bf16 input,
// or (xf set) the fp32 output of the block's pre-norm. For T <= 8 tokens the
// router workgroups also take the top K and group the routes (one of them,
// those that find all logits stored; route_small.h), under the pooler's
// stream, so routing needs no launch of its own either.
struct RouterArgs {
  const uint16_t* x;
  const float* xf;
  const float* wr;
  float* logits;
  int T, H, E;
  RouteFuse rf;  // rf.tagged set: the router workgroups also route (route_small.h)
  // the block's pre-norm folded in (XIN_PRENORM): x is the residual stream
  const uint16_t* pre_gain;
  double pre_eps;
  float* nf32_out;     // workgroup 0 stores the pre-norm's outputs (fp32, bf16)
  uint16_t* nbf16_out;
};

enum { XIN_BF16 = 0, XIN_F32 = 1, XIN_PRENORM = 2 };

template <int TMAX, int U, int KS, int SC, bool AL, int XIN>
__global__ __launch_bounds__(64 * kWaves) void pool_router_kernel(SkinnyArgs p, RouterArgs r) {
  __shared__ double part[kWaves][TMAX];
  if (static_cast<int>(blockIdx.x) < r.E) {
    const uint32_t gen =
        r.rf.tagged ? __hip_atomic_load(r.rf.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const uint32_t tag = route_tag(gen);
    if constexpr (XIN == XIN_PRENORM)
      router_prenorm_body<TMAX, kWaves>(r.x, r.pre_gain, r.pre_eps, r.wr, r.logits, r.T, r.H, r.E,
                                        blockIdx.x, part, r.rf.tagged, tag,
                                        blockIdx.x == 0 ? r.nf32_out : nullptr, r.nbf16_out);
    else if constexpr (XIN == XIN_F32)
      router_gemv_body<TMAX, kWaves, float>(r.xf, r.wr, r.logits, r.T, r.H, r.E, blockIdx.x, part,
                                            r.rf.tagged, tag);
    else
      router_gemv_body<TMAX, kWaves>(r.x, r.wr, r.logits, r.T, r.H, r.E, blockIdx.x, part,
                                     r.rf.tagged, tag);
    if (r.rf.tagged) route_when_complete<kWaves>(r.rf, gen, r.T, r.E);
    return;
  }
  stream_body<B_BF16, EPI_BF16, 1, 1, U, KS, SC, AL>(p, blockIdx.x - r.E, 0);
}

// Launch shape of one projection: A through LDS, and the number of
// wavefronts below which K is split. The weight stages in flight (at most
// UMAX) and the largest K split (KSMAX) are template parameters of the
// launchers, so only reachable kernel shapes are compiled.
constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr size_t kAlLdsBudget = 40 * 1024;

struct Tune {
  bool al;
  int split_waves = 8192;  // split K while fewer wavefronts than this stream the weights
  size_t lds_budget = kAlLdsBudget;  // AL: LDS for the staged rows of one pass
  bool token_rows = true;  // a gather may stage every token row once (a_tokens)
};

template <int TMAX, int U, int KS, int SC, bool AL>
hipError_t launch_fused(const SkinnyArgs& a, const RouterArgs& r, int gx, size_t lds, hipStream_t st) {
  if (r.pre_gain) {
    // (the pooler normalises its staged rows: A in LDS, one pass)
    if constexpr (AL)
      MOE_LAUNCH((pool_router_kernel<TMAX, U, KS, SC, AL, XIN_PRENORM>), dim3(gx + r.E),
                 dim3(64 * kWaves), lds, st, a, r);
    else
      return hipErrorInvalidValue;
  } else if (r.xf) {
    MOE_LAUNCH((pool_router_kernel<TMAX, U, KS, SC, AL, XIN_F32>), dim3(gx + r.E), dim3(64 * kWaves), lds,
               st, a, r);
  } else {
    MOE_LAUNCH((pool_router_kernel<TMAX, U, KS, SC, AL, XIN_BF16>), dim3(gx + r.E), dim3(64 * kWaves), lds,
               st, a, r);
  }
  return hipGetLastError();
}

template <int BFMT, int EPI, int NF, int MB, int U, int KS, int SC>
hipError_t launch_al(SkinnyArgs a, int ny, bool al, const RouterArgs* fuse, hipStream_t st) {
  const dim3 grid((a.n_groups + kWaves / KS - 1) / (kWaves / KS), ny);
  const dim3 block(64 * kWaves);
  const size_t lds = stream_lds_bytes(a, al, KS, MB, NF, few_rows(BFMT) ? 1 : 0);
  if constexpr (BFMT == B_BF16 && EPI == EPI_BF16 && NF == 1 && MB == 1) {
    if (fuse) {
      if (fuse->T <= 1)
        return al ? launch_fused<1, U, KS, SC, true>(a, *fuse, grid.x, lds, st)
                  : launch_fused<1, U, KS, SC, false>(a, *fuse, grid.x, lds, st);
      return al ? launch_fused<16, U, KS, SC, true>(a, *fuse, grid.x, lds, st)
                : launch_fused<16, U, KS, SC, false>(a, *fuse, grid.x, lds, st);
    }
  }
  if constexpr (few_rows(BFMT) > 0 || EPI == EPI_ROUTE_SUM) {  // (A in LDS only)
    if (!al) return hipErrorInvalidValue;
    MOE_LAUNCH((stream_kernel<BFMT, EPI, NF, MB, U, KS, SC, true>), grid, block, lds, st, a);
  } else if (al) {
    MOE_LAUNCH((stream_kernel<BFMT, EPI, NF, MB, U, KS, SC, true>), grid, block, lds, st, a);
  } else {
    MOE_LAUNCH((stream_kernel<BFMT, EPI, NF, MB, U, KS, SC, false>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}

template <int BFMT, int EPI, int NF, int MB, int UMAX, int KS, int SC>
hipError_t launch_ks(const SkinnyArgs& a, int ny, int sps, const Tune& t, const RouterArgs* fuse,
                     hipStream_t st) {
  static_assert(UMAX >= 1 && UMAX <= 2, "weight stages in flight");
  // the pipeline depth must divide the stages of a split
  if constexpr (UMAX == 2)
    if (sps % 2 == 0) return launch_al<BFMT, EPI, NF, MB, 2, KS, SC>(a, ny, t.al, fuse, st);
  return launch_al<BFMT, EPI, NF, MB, 1, KS, SC>(a, ny, t.al, fuse, st);
}

// Split K across the wavefronts of a workgroup when there are few output
// groups, so that about t.split_waves wavefronts stream the weights. a_rows bounds
// the rows of one pass (for the LDS size of A).
template <int BFMT, int EPI, int NF, int MB, int UMAX, int KSMAX>
hipError_t launch_u(SkinnyArgs a, int ny, Tune t, int a_rows, hipStream_t st,
                    const RouterArgs* fuse = nullptr, bool al_one_pass = false) {
  // AL: rows per pass such that the staged rows fit the LDS budget of a
  // workgroup (several workgroups per compute unit); an expert with more
  // rows streams its weights once per pass.
  constexpr int kFragRows = (few_rows(BFMT) ? few_rows(BFMT) : 16) * MB;  // rows of the MB fragments
  constexpr int kZeroRows = few_rows(BFMT) ? 1 : 0;
  const size_t row_bytes = 2 * static_cast<size_t>(a.K) + 16;
  a.pass_rows = static_cast<int>(std::min<size_t>(std::min(kFragRows, std::max(1, a_rows)),
                                                  std::max<size_t>(1, t.lds_budget / row_bytes)));
  if ((a.pass_rows + kZeroRows) * row_bytes + sizeof(float) * kWaves * MB * NF * 256 > kMaxLds) t.al = false;
  // (dense rows are few and the weights large: staging only pays when all
  // rows fit one pass)
  if (al_one_pass && a.pass_rows < std::min(kFragRows, std::max(1, a_rows))) t.al = false;
  if (!t.al) a.pass_rows = kFragRows;
  // a gather whose tokens all fit one pass stages every token row once
  a.a_tokens = (t.al && t.token_rows && a.a_gather && a_rows <= a.pass_rows) ? a_rows : 0;
  const int nchunks = a.K / 128;
  if (nchunks % 2) {  // odd chunk count (K = 128 * odd): one-chunk stages, no split
    return launch_ks<BFMT, EPI, NF, MB, UMAX, 1, 1>(a, ny, nchunks, t, fuse, st);
  }
  const int nstages = nchunks / 2;
  const int64_t groups = static_cast<int64_t>(a.n_groups) * ny;
  int ks = 1;
  while (ks < kWaves && ks < KSMAX && groups * ks < t.split_waves && nstages % (2 * ks) == 0) ks *= 2;
  const int sps = nstages / ks;
  if constexpr (KSMAX >= 8)
    if (ks == 8) return launch_ks<BFMT, EPI, NF, MB, UMAX, 8, 2>(a, ny, sps, t, fuse, st);
  if constexpr (KSMAX >= 4)
    if (ks == 4) return launch_ks<BFMT, EPI, NF, MB, UMAX, 4, 2>(a, ny, sps, t, fuse, st);
  if constexpr (KSMAX >= 2)
    if (ks == 2) return launch_ks<BFMT, EPI, NF, MB, UMAX, 2, 2>(a, ny, sps, t, fuse, st);
  return launch_ks<BFMT, EPI, NF, MB, UMAX, 1, 2>(a, ny, sps, t, fuse, st);
}

// Weight stages in flight of the dense projections with one 16-row fragment
// (A staged in LDS). One: 113 VGPRs, two workgroups per CU, every workgroup
// of the real-shape unpooler resident at once; two stages took 153 VGPRs,
// one workgroup per CU and two rounds (T = 1 unpooler 14.8 -> 13.6 us; the
// layer 0.5-1.0 us faster at every T from 1 to 16, same box).
constexpr int kDenseU = 1;
// The router + pooler launch keeps one weight stage in flight: at two its
// registers (163) allow one workgroup per CU, and the pooler's workgroups
// wait for the router's; at one (123) both share the CUs (T = 1 layer
// 91.4 -> 89.4 us).
constexpr int kPoolRouterU = 1;
// The expert projections: two weight stages in flight, K split at most four
// ways, A staged in LDS.
constexpr int kExpertU = 2;
constexpr int kExpertKs = 4;

}  // namespace

// The block's pre-norm folds into the router + pooler launch for one token
// whose row the pooler stages in LDS (the row it normalises); the router
// then runs its one-token body (125 VGPRs with the fold, two workgroups per
// CU; its 16-token body would take 243).
bool prenorm_fold_ok(int T, int H) {
  const size_t row_bytes = 2 * static_cast<size_t>(H) + 16;
  return T == 1 && row_bytes <= kAlLdsBudget && row_bytes + sizeof(float) * kWaves * 256 <= kMaxLds;
}

// Dense bf16 projection: out[m][n] = bf16(sum_k a[m][k] * b[n][k]).
hipError_t launch_dense_skinny(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N,
                               int K, hipStream_t st) {
  SkinnyArgs p{};
  p.a = a;
  p.b_bf16 = b;
  p.out = out;
  p.ldo = N;
  p.K = K;
  p.m_total = M;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(M) * K * 2);
  p.n_groups = N / 16;
  const int mb = M > 16 ? 2 : 1;
  const int ny = (M + 16 * mb - 1) / (16 * mb);
  // one 16-row fragment: A staged in LDS, kDenseU weight stages in flight;
  // two fragments: A in registers
  // (A in registers: one fragment of weight rows keeps two stages in flight,
  // T = 32 pooler 33.3 -> 30.9 us; two fragments keep one, two measured 66 us)
  const Tune t1{true}, t2{false};
  // two fragments of A rows against two of weight rows per wavefront halve
  // the A loads per weight byte; taken while that still leaves 256 groups
  // (T = 32 unpooler 31.1 -> 25.4 us; the pooler, 128 groups, slowed down)
  if (mb == 2 && N % 32 == 0 && N / 32 >= 256) {
    p.n_groups = N / 32;
    return launch_u<B_BF16, EPI_BF16, 2, 2, 1, kWaves>(p, ny, t2, M, st, nullptr, true);
  }
  return mb == 2 ? launch_u<B_BF16, EPI_BF16, 1, 2, 2, kWaves>(p, ny, t2, M, st, nullptr, true)
                 : launch_u<B_BF16, EPI_BF16, 1, 1, kDenseU, kWaves>(p, ny, t1, M, st, nullptr, true);
}

// Steps A7 and A8 in one launch (EPI_ROUTE_SUM). The post-norm scales c and
// the weighted sum are linear in the unpooler's input, so
// unpooler . (sum_k c_k g*row_k) = sum_k c_k (unpooler . g*row_k): the
// unpooler streams its weights once against the T*K gain-scaled route rows
// (one 16-row fragment holds them) and adds each token's K products with
// their scales in its epilogue, which replaces the combine's launch and its
// round trip of y (T = 1 layer 88.8 -> 86.9 us, same box). Taken while the
// rows fit one pass in kRouteSumLds of LDS (two workgroups per CU; 16 rows
// of 8 KiB at T = 2 need one workgroup per CU and measured 5 us slower).
constexpr size_t kRouteSumLds = 72 * 1024;

bool route_sum_ok(int T, int K, int L, int H) {
  const int64_t rows = static_cast<int64_t>(T) * K;
  return rows >= 1 && rows <= 16 && H % 16 == 0 && L % 128 == 0 &&
         rows * (2 * static_cast<int64_t>(L) + 16) <= static_cast<int64_t>(kRouteSumLds);
}

hipError_t launch_unpool_routes(const uint16_t* rows16, const float* ssp, const float* w, float eps, int T,
                                int K, int L, int H, const uint16_t* unpooler, uint16_t* out, hipStream_t st) {
  if (!route_sum_ok(T, K, L, H)) return hipErrorInvalidValue;
  SkinnyArgs p{};
  p.a = rows16;
  p.b_bf16 = unpooler;
  p.out = out;
  p.ldo = H;
  p.K = L;
  p.m_total = T * K;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(T) * K * L * 2);
  p.n_groups = H / 16;
  p.topk = K;
  p.ssp = const_cast<float*>(ssp);
  p.route_w = w;
  p.norm_eps = eps;
  Tune t{true};
  t.lds_budget = kRouteSumLds;
  return launch_u<B_BF16, EPI_ROUTE_SUM, 1, 1, kDenseU, kWaves>(p, 1, t, T * K, st, nullptr, true);
}

// The pooler (T <= 16 rows) with the router logits in the same launch; the
// router reads xf (fp32) when given, else x. With pre (the block's pre-norm
// folded in) x is the residual stream, and both the router and the pooler
// normalise it themselves.
hipError_t launch_pool_router(const uint16_t* x, const uint16_t* pooler, uint16_t* lat, int T, int L,
                              int H, const float* wr, float* logits, int E, hipStream_t st,
                              const float* xf, const RouteFuse* rf, const PreNormFold* pre) {
  SkinnyArgs p{};
  p.a = x;
  p.b_bf16 = pooler;
  p.out = lat;
  p.ldo = L;
  p.K = H;
  p.m_total = T;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(T) * H * 2);
  p.n_groups = L / 16;
  RouterArgs r{x, xf, wr, logits, T, H, E, RouteFuse{}, nullptr, 0.0, nullptr, nullptr};
  if (rf) {
    if (T > kWaves || T * rf->K > 64) return hipErrorInvalidValue;  // one wavefront per token, 64 routes
    r.rf = *rf;
  }
  if (pre) {
    if (!prenorm_fold_ok(T, H)) return hipErrorInvalidValue;
    r.pre_gain = pre->gain;
    r.pre_eps = pre->eps;
    r.nf32_out = pre->nf32_out;
    r.nbf16_out = pre->nbf16_out;
    p.pre_gain = pre->gain;
    p.pre_eps = pre->eps;
  }
  const Tune t{true};
  return launch_u<B_BF16, EPI_BF16, 1, 1, kPoolRouterU, kWaves>(p, 1, t, T, st, &r, true);
}

// NVFP4 expert projections take a few-rows form when a pass holds at most
// four rows (one row) anyway: then it changes nothing but how the block
// scales are applied (at K = 4096 the LDS budget of a pass is four rows of
// 8 KiB, so this holds at every token count of the decode regime). Returns
// the rows per pass, or 0 for the plain form.
static int nvfp4_few_rows(const SkinnyArgs& p, const Tune& t, int a_rows) {
  const size_t row_bytes = 2 * static_cast<size_t>(p.K) + 16;
  const size_t rows = std::min<size_t>(std::min<size_t>(16, std::max(1, a_rows)),
                                       std::max<size_t>(1, t.lds_budget / row_bytes));
  const bool ok = t.al && rows <= 4 && (rows + 1) * row_bytes + sizeof(float) * kWaves * 2 * 256 <= kMaxLds;
  return ok ? static_cast<int>(rows) : 0;
}

// The light experts' share of a split projection (ExpertGemm::split_rows):
// only work-list entries of at most `rows` rows, all of them staged in LDS
// in one pass (up to 16 rows of 8 KiB: one workgroup per CU), none of the
// gather's whole-token staging.
static void split_light(SkinnyArgs& p, Tune& t, int rows, int* a_rows) {
  p.max_rows = rows;
  t.lds_budget = static_cast<size_t>(rows) * (2 * static_cast<size_t>(p.K) + 16);
  t.token_rows = false;
  *a_rows = rows;
}

// Gate/up projection of every route row against its expert's W13 plus
// SwiGLU: h[i][n] = bf16(silu(g) * u) for sorted position i. An expert has
// at most one row per token.
hipError_t launch_gateup_skinny(const ExpertGemm& x, hipStream_t st) {
  SkinnyArgs p{};
  p.a = x.lat;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.latent * 2);
  p.a_gather = 1;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.active = x.active;
  p.b_codes = x.w13_codes;
  p.b_scales = x.w13_scales;
  p.b_rows_per_expert = 2 * x.inter;
  p.K = x.latent;
  p.inter = x.inter;
  p.out = x.h;
  p.ldo = x.inter;
  p.n_groups = x.inter / 16;
  p.b_global = x.w13_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  Tune t{true};
  int a_rows = x.tokens;
  if (x.split_rows > 0) split_light(p, t, x.split_rows, &a_rows);
  const int few = x.nvfp4 ? nvfp4_few_rows(p, t, a_rows) : 0;
  if (few == 1) return launch_u<B_NVFP4_ONE, EPI_SWIGLU, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
  if (few > 1) return launch_u<B_NVFP4_FEW, EPI_SWIGLU, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
  return x.nvfp4 ? launch_u<B_NVFP4, EPI_SWIGLU, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st)
                 : launch_u<B_MXFP4, EPI_SWIGLU, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
}

// (the scaled rows only in the MXFP4 and one-row NVFP4 forms: in the
// few-rows and plain NVFP4 forms the extra stores spilled 16-76 bytes per
// lane; down_scaled_ok tells the host which form a call takes)
template <int EPI>
static hipError_t down_skinny(const SkinnyArgs& p, const ExpertGemm& x, const Tune& t, int a_rows, int few,
                              hipStream_t st) {
  if (few == 1) return launch_u<B_NVFP4_ONE, EPI, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
  if constexpr (EPI == EPI_F32_SCATTER_SCALED) {
    if (x.nvfp4) return hipErrorInvalidValue;
    return launch_u<B_MXFP4, EPI, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
  } else {
    if (few > 1) return launch_u<B_NVFP4_FEW, EPI, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
    return x.nvfp4 ? launch_u<B_NVFP4, EPI, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st)
                   : launch_u<B_MXFP4, EPI, 2, 1, kExpertU, kExpertKs>(p, x.max_active, t, a_rows, st);
  }
}

// The down projection's Tune (launch_down_skinny) and whether it can store
// the gain-scaled rows for T tokens of inter-wide rows.
static Tune down_tune() { return Tune{true, 131072}; }

bool down_scaled_ok(int T, int I, bool nvfp4) {
  if (!nvfp4) return true;
  SkinnyArgs p{};
  p.K = I;
  return nvfp4_few_rows(p, down_tune(), T) == 1;
}

// Down projection of every route row: rows[r][n] (fp32, route-major), and
// with x.rows16 bf16(gain * row) too.
hipError_t launch_down_skinny(const ExpertGemm& x, hipStream_t st) {
  SkinnyArgs p{};
  p.a = x.h;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.topk * x.inter * 2);
  p.a_gather = 0;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.active = x.active;
  p.b_codes = x.w2_codes;
  p.b_scales = x.w2_scales;
  p.b_rows_per_expert = x.latent;
  p.K = x.inter;
  p.out = x.rows;
  p.ldo = x.latent;
  p.n_groups = x.latent / 32;
  p.ssp = x.ssp;
  p.out_scaled = x.rows16;
  p.gain = x.gain;
  p.gain_per_expert = x.gain_per_expert;
  p.b_global = x.w2_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  // (T = 32, about 163 touched experts: four K splits take the down
  // projection from 441 to 422 us in a harness, while gate/up is fastest
  // unsplit)
  Tune t = down_tune();
  int a_rows = x.tokens;
  if (x.split_rows > 0) split_light(p, t, x.split_rows, &a_rows);
  const int few = x.nvfp4 ? nvfp4_few_rows(p, t, a_rows) : 0;
  if (x.rows16) return down_skinny<EPI_F32_SCATTER_SCALED>(p, x, t, a_rows, few, st);
  return down_skinny<EPI_F32_SCATTER>(p, x, t, a_rows, few, st);
}

}  // namespace moe
