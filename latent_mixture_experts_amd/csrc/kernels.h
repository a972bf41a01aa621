// kernels.h -- launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"

namespace moe {

// Events that the next kernel launch records at its own start and end (for
// per-step timing); both null outside a timed call. Per host thread.
struct StageEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
StageEvents& stage_events();

#define MOE_LAUNCH(kern, grid, block, shmem, stream, ...)                                  \
  hipExtLaunchKernelGGL(kern, grid, block, shmem, stream, ::moe::stage_events().start,     \
                        ::moe::stage_events().stop, 0, __VA_ARGS__)

enum { B_BF16 = 0, B_MXFP4 = 1, B_NVFP4 = 2, B_NVFP4_FEW = 3, B_NVFP4_ONE = 4 };
// 4-bit expert formats: E2M1 codes with one E8M0 scale per 32 elements
// (MXFP4) or one E4M3 scale per 16 elements times a per-tensor fp32 scale
// (NVFP4). B_NVFP4_FEW and B_NVFP4_ONE are NVFP4 in the streaming kernels'
// few-rows form, for at most four rows (one row) per 16-row MFMA fragment:
// each row spreads over four MFMA rows, one per scale-block group, so the
// block scales multiply fp32 partial sums instead of every decoded weight
// (stream_body.h).
constexpr bool is_fp4(int f) { return f != B_BF16; }
constexpr bool is_nvfp4(int f) { return f == B_NVFP4 || f == B_NVFP4_FEW || f == B_NVFP4_ONE; }
// rows per fragment of the few-rows forms (0: not one)
constexpr int few_rows(int f) { return f == B_NVFP4_ONE ? 1 : f == B_NVFP4_FEW ? 4 : 0; }
constexpr int scale_block(int f) { return is_nvfp4(f) ? 16 : 32; }
// Epilogues of the streaming projections: bf16 rows; SwiGLU -> bf16 h;
// fp32 route rows scattered to route order (+ partial sums of squares; the
// _SCALED form also stores bf16(gain * row) to out_scaled, a kernel of its
// own so the plain one keeps its registers); route sum: dense bf16 weights
// whose A rows are a token's K gain-scaled route rows, the outputs summed
// over them with each row's post-norm scale (the weighted sum after the
// products).
enum { EPI_BF16 = 0, EPI_SWIGLU = 1, EPI_F32_SCATTER = 2, EPI_ROUTE_SUM = 3, EPI_F32_SCATTER_SCALED = 4 };
constexpr bool is_scatter(int e) { return e == EPI_F32_SCATTER || e == EPI_F32_SCATTER_SCALED; }

// The routing done inside the router + pooler launch (route_small.h): the
// router workgroups also store their logits tagged with the call's tag, and
// those that find all logits present take the top K and group the routes.
// tagged == nullptr: no routing in that launch.
struct RouteFuse {
  uint64_t* tagged;   // [T][E]: tag << 32 | logit bits
  uint32_t* gen;      // generation word, advanced by every call routed this way
  uint32_t* status;   // bit 0 set when a router workgroup gave up waiting (never in practice)
  int K;
  int32_t* ids;       // [T][K] expert ids (outputs, as the grouping kernels write them)
  float* w;           // [T][K] router weights
  int32_t* offsets;
  int32_t* sorted;
  int32_t* active;
  int32_t* counters;
  int32_t* tiles;
};

// Arguments of the decode-regime projection kernel.
struct SkinnyArgs {
  const uint16_t* a;         // bf16 A rows, K elements each
  uint32_t a_bytes;          // bytes of the A tensor (buffer range)
  int a_gather;              // 1: A row of sorted position i is token sorted[i] / topk
  const int32_t* sorted;     // sorted routes (gather of A, scatter of fp32 rows)
  int topk;
  int m_total;               // dense: number of rows
  const int32_t* active;     // MXFP4: [E][4] (expert, first row, end row, -) per touched expert
  const uint16_t* b_bf16;    // dense B [N][K]
  const uint8_t* b_codes;    // MXFP4 B codes [E][rows][K/2]
  const uint8_t* b_scales;   // MXFP4 B scales [E][rows][K/32]
  int b_rows_per_expert;
  int K;
  int inter;                 // SwiGLU: up rows start at row `inter`
  void* out;
  int ldo;
  int n_groups;              // output column groups (one wavefront each)
  float* ssp;                // F32 rows: partial sums of squares [row][group], or null
  int pass_rows;             // A staged in LDS: rows per pass over the weights
  int a_tokens;              // gather with every token row staged once (T rows), or 0
  const float* b_global;     // NVFP4: [E] per-tensor scale of B
  int n_experts;             // MXFP4/NVFP4: work-list entries outside [0, n_experts) or past
  int n_routes;              // n_routes rows are skipped (never an access outside the weights)
  const uint16_t* pre_gain;  // dense A staged in LDS in one pass: the block's pre-norm (gain [K],
  double pre_eps;            // eps) applied to the staged rows, or null
  uint32_t red_off;          // K split: byte offset of the partial-sum buffer in the dynamic LDS
  int max_rows;              // MXFP4/NVFP4: > 0: work-list entries with more rows are skipped
  uint16_t* out_scaled;      // EPI_F32_SCATTER_SCALED: also bf16(gain * row) here (route-major)
  const uint16_t* gain;      // its gain, [n] or [E][n] (gain_per_expert)
  int gain_per_expert;
  const float* route_w;      // EPI_ROUTE_SUM: router weight of each A row; ssp: their partial sums
  float norm_eps;            // of squares [row][K / 32]; the post-norm's eps
};

// Dynamic LDS of a streaming projection: the staged A rows (AL), then the
// K-split partial sums; sets a.red_off and returns the bytes.
// (B_NVFP4_FEW: one more row, of zeros, after the staged rows.)
inline size_t stream_lds_bytes(SkinnyArgs& a, bool al, int ks, int mb, int nf, int zero_rows = 0) {
  const size_t a_bytes =
      al ? static_cast<size_t>(a.pass_rows + zero_rows) * (2 * static_cast<size_t>(a.K) + 16) : 0;
  const size_t off = (a_bytes + 15) / 16 * 16;
  a.red_off = static_cast<uint32_t>(off);
  return off + (ks > 1 ? sizeof(float) * 8 * mb * nf * 256 : 0);
}

// Rows per tile of the prefill expert projections (an expert's rows are cut
// into consecutive tiles of this many rows, the last one shorter).
constexpr int kTileRows = 64;
// Rows per tile of the LDS-staged expert projections (gemm_expert.hip).
constexpr int kExpertTileRows = 128;

// Arguments of the prefill-regime (tiled) projection kernel.
struct TiledArgs {
  const uint16_t* a;         // bf16 A rows, K elements each
  uint32_t a_bytes;
  int a_gather;              // 1: A row of sorted position i is token sorted[i] / topk
  const int32_t* sorted;
  int topk;
  int grouped;               // 1: row tiles from the expert tile list
  int m_total;               // dense: number of rows
  const int32_t* offsets;
  const int32_t* counters;   // counters[1] = number of row tiles
  const int32_t* tiles;      // [n][2] (expert, first sorted row)
  const uint16_t* b_bf16;    // dense B [N][K]
  uint32_t b_bytes;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int b_rows_per_expert;
  int K;
  int inter;
  void* out;
  int ldo;
  int n_col_tiles;           // column tiles per row tile
  const float* b_global;     // NVFP4: [E] per-tensor scale of B
  int n_experts;             // grouped: tiles outside [0, n_experts) or past n_routes rows
  int n_routes;              // are skipped (never an access outside the weights)
  int min_rows;              // grouped: tiles of experts with at most this many rows are skipped
};

// Everything the expert projections need.
struct ExpertGemm {
  const uint16_t* lat;       // [T][L] bf16
  const int32_t* sorted;     // [T*K]
  const int32_t* offsets;    // [E+1]
  const int32_t* active;     // [E][4]: touched expert, its first and end sorted row; expert -1 after the last
  const int32_t* counters;   // [0] touched experts, [1] row tiles
  const int32_t* tiles;      // [n_tiles][2] (expert, first sorted row)
  const uint8_t* w13_codes;
  const uint8_t* w13_scales;
  const uint8_t* w2_codes;
  const uint8_t* w2_scales;
  uint16_t* h;               // [T*K][I] bf16, sorted order
  float* rows;               // [T*K][L] fp32, route-major
  float* ssp;                // [T*K][L/32] partial sums of squares of the rows, or null
  int tokens, topk, latent, inter;
  int n_experts;
  int max_active;            // grid bound: min(E, T*K)
  int max_tiles;             // grid bound on row tiles
  int nvfp4;                 // 1: NVFP4 weights (scales [rows][K/16] E4M3, per-tensor scales below)
  const float* w13_global;   // NVFP4: [E] per-tensor scale of W13
  const float* w2_global;    // NVFP4: [E] per-tensor scale of W2
  // > 0: the projection's experts with at most this many rows run on the
  // streaming kernels (the *_skinny launchers, all of an expert's rows in
  // one pass), the others on the row tiles (the *_expert / *_tiled
  // launchers skip the light experts' tiles); 0: every expert on one kernel
  int split_rows;
  // or null: the streaming down projection also writes bf16(gain * row) of
  // every route row here ([T*K][L], route-major), for the unpooler that
  // takes the weighted sum after its products (launch_unpool_routes)
  uint16_t* rows16;
  const uint16_t* gain;      // [L] or [E][L] bf16
  int gain_per_expert;
};
// Largest split_rows: one 16-row fragment per pass of the streaming kernel.
constexpr int kMaxSplitRows = 16;

hipError_t launch_router_logits(const uint16_t* x, const float* wr, double* partial, int T, int H,
                                int E, int splits, hipStream_t st);
// the same for an fp32 input (the block's pre-norm output)
hipError_t launch_router_logits(const float* x, const float* wr, double* partial, int T, int H,
                                int E, int splits, hipStream_t st);
// the block around the layer (block.hip)
hipError_t launch_pre_norm(const uint16_t* resid, const uint16_t* gain, double eps, int T, int H,
                           float* n_f32, uint16_t* n_bf16, hipStream_t st);
hipError_t launch_post_norm_residual(const uint16_t* resid, const uint16_t* f, const uint16_t* gain,
                                     double eps, int T, int H, uint16_t* out, hipStream_t st);
hipError_t launch_topk(const double* partial, int S, int T, int E, int K, float* logits,
                       int32_t* ids, float* w, hipStream_t st);
hipError_t launch_router_gemv(const uint16_t* x, const float* wr, float* logits, int T, int H,
                              int E, hipStream_t st);
// The persistent decode layer (decode_layer.hip): the whole layer for one
// or two tokens in one launch.
constexpr int kDecodeMaxWorkers = 1024;  // arrival slots in the workspace (8 groups of 128)
struct DecodeLayer {
  int T, H, L, I, E, K;
  int nvfp4, gain_per_expert;
  float eps;
  const uint16_t* x;
  const float* router;
  const uint16_t* pooler;
  const uint8_t* w13_codes;
  const uint8_t* w13_scales;
  const float* w13_global;
  const uint8_t* w2_codes;
  const uint8_t* w2_scales;
  const float* w2_global;
  const uint16_t* gain;
  const uint16_t* unpooler;
  uint16_t* out;
  // workspace
  float* logits;
  uint64_t* tagged;
  int32_t* ids;
  float* w;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* active;
  int32_t* counters;
  int32_t* tiles;
  uint16_t* lat;
  uint16_t* h;
  float* rows;
  float* ssp;
  uint16_t* y;
  uint16_t* rows16; // or null: the post-norm and weighted sum in the unpooler's phase (launch_unpool_routes)
  uint32_t* sync;   // [0] generation word, [1] status, [2] routing flag
  uint32_t* slots;  // [kDecodeMaxWorkers]
  uint32_t* grp;    // 8 group words, 128 bytes apart
  uint32_t* rel;    // 8 release words, 128 bytes apart
};
// route_sum: the call takes the post-norm and weighted sum in the unpooler's
// phase (as moe_latent_forward does for the same T and shape)
bool decode_layer_ok(int T, int H, int L, int I, int E, int K, bool nvfp4, bool route_sum);
hipError_t launch_decode_layer(const DecodeLayer& d, hipStream_t st);
hipError_t launch_route_small(const float* logits, int T, int E, int K, int32_t* ids, float* w,
                              int32_t* offsets, int32_t* sorted_routes, int32_t* active,
                              int32_t* counters, int32_t* tiles, int tile_m, hipStream_t st);
// ids_copy: null, or where to write the ids clamped into [0, E);
// chunk_counts: permute_chunks(R) * E ints of workspace (R > 6144: the
// grouping over several workgroups), or null (one workgroup)
int permute_chunks(int R);
hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* offsets, int32_t* sorted_routes,
                          int32_t* active, int32_t* counters, int32_t* tiles, int tile_m,
                          hipStream_t st, int32_t* ids_copy = nullptr, int32_t* chunk_counts = nullptr);
hipError_t launch_dense_skinny(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N,
                               int K, hipStream_t st);
// The block's pre-norm folded into the router + pooler launch
struct PreNormFold {
  const uint16_t* gain;  // [H] bf16
  double eps;
  float* nf32_out;       // [T][H]: the pre-norm's fp32 output (the router's input), stored
  uint16_t* nbf16_out;   // [T][H]: its bf16 output (the pooler's input), stored
};
bool prenorm_fold_ok(int T, int H);
hipError_t launch_pool_router(const uint16_t* x, const uint16_t* pooler, uint16_t* lat, int T, int L,
                              int H, const float* wr, float* logits, int E, hipStream_t st,
                              const float* xf = nullptr, const RouteFuse* rf = nullptr,
                              const PreNormFold* pre = nullptr);
bool expert_lds_ok(int latent, int inter, bool nvfp4);
hipError_t launch_gateup_expert(const ExpertGemm& x, hipStream_t st);
hipError_t launch_down_expert(const ExpertGemm& x, hipStream_t st);
hipError_t launch_gateup_skinny(const ExpertGemm& x, hipStream_t st);
bool dense_lds_ok(int M, int N, int K);
// host evaluation of the prefill kernels' tile orders (tile_map export)
int dense_grid(int M, int N);
TileRC dense_tile_host(int block, int M, int N);
int expert_chunk_rows();  // row tiles dealt to one XCD together by the LDS-staged expert kernel
int dense_splits(int M, int N, int K);
hipError_t launch_dense_lds(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N, int K,
                            hipStream_t st, float* part = nullptr);
hipError_t launch_dense_tiled(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N,
                              int K, hipStream_t st, float* part = nullptr);
hipError_t launch_gateup_tiled(const ExpertGemm& x, hipStream_t st);
hipError_t launch_down_tiled(const ExpertGemm& x, hipStream_t st);
hipError_t launch_down_skinny(const ExpertGemm& x, hipStream_t st);
// Steps A7 and A8 in one launch for few route rows (gemm_skinny.hip): the
// unpooler's A rows are the T*K gain-scaled route rows (rows16), each
// workgroup takes every row's post-norm scale c = w / sqrt(ss / L + eps)
// from the partial sums of squares, and out[t] = bf16(sum over the token's
// routes of c * (unpooler . row)). route_sum_ok: T*K <= 16 and the rows fit
// one pass in LDS.
bool route_sum_ok(int T, int K, int L, int H);
// whether the streaming down projection of T tokens (inter-wide rows) takes
// a form that also stores the gain-scaled rows (MXFP4, or NVFP4 one row per pass)
bool down_scaled_ok(int T, int I, bool nvfp4);
hipError_t launch_unpool_routes(const uint16_t* rows16, const float* ssp, const float* w, float eps, int T,
                                int K, int L, int H, const uint16_t* unpooler, uint16_t* out, hipStream_t st);
hipError_t launch_combine_cols(const float* rows, const float* ssp, const float* w,
                               const int32_t* ids, const uint16_t* gain, int gain_per_expert,
                               float eps, int T, int K, int L, uint16_t* y, hipStream_t st);
hipError_t launch_combine(const float* rows, const float* w, const int32_t* ids,
                          const uint16_t* gain, int gain_per_expert, float eps, int T, int K,
                          int L, uint16_t* y, hipStream_t st);

}  // namespace moe
