/*
 * moe.h -- C ABI of the latent mixture-of-experts layer on AMD MI355X (gfx950).
 *
 * The layer (one MoE layer of the 816B-A42B "Muse Spark Open" model):
 *   1. an fp32 router scores every expert for each token and keeps the top K
 *      ("Muse Spark Open on Gaudi 2", section "What was built": fp32 router,
 *      256 experts, top 8);
 *   2. the routes are grouped by expert;
 *   3. one pooler shared by all experts projects each token from the hidden
 *      width H to the latent width L ("Soporte de dia 0 para Muse Spark Open
 *      en vLLM", section "Arquitectura del modelo", paragraph "MoE latente");
 *   4. every (token, route) pair is its own row through its expert's MXFP4
 *      SwiGLU FFN, W4A16: 4-bit E2M1 weights with E8M0 block scales, bf16
 *      activations ("Muse Spark Open on Gaudi 2", sections "What was built"
 *      and "The latent MoE: A' with a per-expert norm");
 *   5. each route row gets the post-expert RMS norm, then the rows are
 *      multiplied by the router weights and summed in fp32 (same section);
 *   6. the shared unpooler projects the sum from L back to H (same section).
 *
 * Conventions for every entry point:
 *  - Device pointers unless stated otherwise; bf16 values are passed as their
 *    16-bit patterns (uint16_t). All matrices are row-major.
 *  - Ownership: the caller allocates and owns every buffer and the stream.
 *    The library allocates no memory, keeps no state between calls (apart
 *    from the thread-local last HIP error) and never synchronises the host:
 *    work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream),
 *    so calls can be captured into a HIP graph.
 *  - Errors: every entry point returns an int status, MOE_OK (0) or a
 *    negative MOE_E* code. Invalid arguments are reported before anything is
 *    enqueued, and outputs are left untouched. MOE_EHIP means a launch
 *    failed; moe_last_hip_error() returns the HIP error code.
 *  - Inputs, outputs and the workspace must not overlap. T == 0 is a no-op
 *    returning MOE_OK. Outputs are fully overwritten.
 *  - Routing and the permutation are deterministic (bit-identical across
 *    runs); the output does not depend on the workspace contents. (For
 *    T <= 8 the first 256 bytes of the workspace hold a generation word that
 *    each call advances on the device, so that a call, or a replay of a
 *    captured graph, recognises its own router logits among stale words;
 *    any initial contents work, and calls sharing a workspace must not
 *    overlap, as for every other buffer of it.)
 *
 * Supported shapes (else MOE_EUNSUPPORTED): hidden, latent and inter are
 * multiples of 128, at least 128, latent <= 8192, hidden and inter <= 65536;
 * 1 <= n_experts <= 256; 1 <= top_k <= min(8, n_experts);
 * T * top_k < 2^28. Pointers must be 16-byte aligned (MOE_EALIGN).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null pointer, negative size, bad eps or flag   */
#define MOE_EUNSUPPORTED (-2) /* dims outside the supported shapes above        */
#define MOE_EALIGN (-3)       /* a pointer is not 16-byte aligned               */
#define MOE_EWORKSPACE (-4)   /* workspace smaller than moe_workspace_bytes()   */
#define MOE_EHIP (-5)         /* a HIP launch failed (see moe_last_hip_error)   */

typedef struct {
  int32_t hidden;          /* H: width of the layer input and output (8192)          */
  int32_t latent;          /* L: width after the pooler, the experts' width (4096)    */
  int32_t inter;           /* I: SwiGLU intermediate width of each expert (4096)      */
  int32_t n_experts;       /* E: routed experts (256)                                  */
  int32_t top_k;           /* K: experts per token (8)                                 */
  float norm_eps;          /* eps inside the post-expert RMS norm's square root (1e-6) */
  int32_t gain_per_expert; /* 0: one norm gain [L] for all experts; 1: gain [E][L]     */
  int32_t expert_format;   /* MOE_FMT_MXFP4 or MOE_FMT_NVFP4                           */
  int32_t expert_split_rows; /* the expert projections' two loops (below); 0: default */
} moe_dims;

/* expert_split_rows: how the expert projections treat experts with few
 * routes when the routes average at least 16 per expert (otherwise every
 * expert already runs on the streaming kernels). "RadixArk team serves
 * Meta's Muse Spark Open on one TPU host", section "Changes to attention
 * and expert processing": many-request decode steps under random routing
 * ran faster once the expert work was split into two loops; the page does
 * not say which, and here the two loops are the experts' two row regimes:
 *   n in 1..16: experts with at most n routes stream their weights once for
 *      all their rows (HBM-bound kernels), the others run on MFMA row tiles
 *      (a second launch per projection);
 *   -1: one loop, every expert on the row tiles;
 *   0: the library's choice.
 * Other values return MOE_EINVAL. Results are within the same bounds either
 * way (the two kernels sum in different orders, so the bits may differ). */

/* Expert weight formats. Both store E2M1 codes as below. MXFP4: one E8M0
 * scale byte per 32 elements ([rows][K/32]). NVFP4 (public NVIDIA format;
 * "Soporte de día 0 para Muse Spark Open en vLLM", section "Aspectos
 * destacados": the model ships in NVFP4): one OCP E4M3 scale byte per 16
 * elements ([rows][K/16]) times one fp32 scale per stored tensor and expert
 * (w13_global, w2_global). */
#define MOE_FMT_MXFP4 0
#define MOE_FMT_NVFP4 1

/* Layer weights, as stored (no repacking step). 4-bit expert tensors: byte j
 * of a code row holds element 2j in bits 0..3 and element 2j+1 in bits 4..7
 * (E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit). MXFP4: one E8M0
 * scale byte (value 2^(b-127)) covers 32 consecutive elements of a row along
 * the reduction dimension. NVFP4: one E4M3 scale byte covers 16, and the
 * tensor's fp32 scale multiplies every element. */
typedef struct {
  const float *router;          /* [E][H] fp32                                     */
  const uint16_t *pooler;       /* [L][H] bf16: lat = x . pooler^T                 */
  const uint8_t *w13_codes;     /* [E][2I][L/2]: rows 0..I-1 gate, I..2I-1 up      */
  const uint8_t *w13_scales;    /* [E][2I][L/32] (NVFP4: [E][2I][L/16])            */
  const uint8_t *w2_codes;      /* [E][L][I/2]: down projection                    */
  const uint8_t *w2_scales;     /* [E][L][I/32] (NVFP4: [E][L][I/16])              */
  const uint16_t *norm_gain;    /* [L] or [E][L] bf16 (see gain_per_expert)        */
  const uint16_t *unpooler;     /* [H][L] bf16: out = y . unpooler^T               */
  const float *w13_global;      /* NVFP4: [E] fp32 scale of each expert's W13      */
  const float *w2_global;       /* NVFP4: [E] fp32 scale of each expert's W2       */
} moe_weights;

/* Token counts: T * H * 2, T * latent * 2 and T * top_k * inter * 2 bytes
 * must each be below 2^31 (T <= 32767 at H 8192, L 4096, K 8, I 4096);
 * larger T returns MOE_EUNSUPPORTED (split the batch).
 *
 * Bytes of device workspace needed by moe_route and moe_latent_forward for
 * any T <= max_tokens. Returns 0 if the dims are invalid or unsupported. */
size_t moe_workspace_bytes(const moe_dims *dims, int32_t max_tokens);

/*
 * moe_route -- steps 1 and 2 for T tokens (router logits, top-K with router
 * weights, grouping of the routes by expert).
 *   x              [T][H] bf16      layer input (the router reads the full
 *                                   H-wide input, converted exactly to fp32)
 *   router         [E][H] fp32
 *   topk_ids       [T][K] int32     out: experts in rank order: larger logit
 *                                   first, equal logits (-0 == +0) by lower
 *                                   id, NaN after every number
 *   topk_w         [T][K] fp32      out: softmax over the K selected logits
 *   expert_offsets [E+1]  int32     out: exclusive prefix sum of the number
 *                                   of routes per expert; [E] = T*K
 *   sorted_routes  [T*K]  int32     out: route ids r = t*K + k grouped by
 *                                   expert, ascending r within an expert
 *   logits_out     [T][E] fp32      out, optional (NULL): the router logits,
 *                                   each the fp32 rounding of the exact sum
 *                                   (accumulated in fp64)
 */
int moe_route(const moe_dims *dims, int32_t T, const uint16_t *x,
              const float *router, int32_t *topk_ids, float *topk_w,
              int32_t *expert_offsets, int32_t *sorted_routes,
              float *logits_out, void *workspace, size_t workspace_bytes,
              void *hip_stream);

/*
 * moe_latent_forward -- the whole layer for T tokens:
 *   out[t] = bf16( unpooler . bf16( sum_k w[t][k] * rmsnorm_e(row[t][k]) ) )
 *   row[t][k] = W2_e . bf16( silu(W13gate_e . lat[t]) * (W13up_e . lat[t]) )
 *   lat[t] = bf16( pooler . x[t] ),   e = topk_ids[t][k]
 * with rmsnorm_e(v) = v / sqrt(mean(v^2) + eps) * gain (gain[e] if per expert).
 *   x   [T][H] bf16,   out [T][H] bf16 (out)
 * Intermediates (router logits, routes, lat, h, route rows, y) live in the
 * workspace; moe_workspace_view() locates them.
 */
int moe_latent_forward(const moe_dims *dims, int32_t T, const uint16_t *x,
                       const moe_weights *weights, uint16_t *out,
                       void *workspace, size_t workspace_bytes,
                       void *hip_stream);

/*
 * moe_latent_forward_routed -- the same layer with the routing given by the
 * caller (routing replay: "Soporte de día 0 para Muse Spark Open en vLLM",
 * section "Aprendizaje por refuerzo en vLLM", where the trainer reuses the
 * rollout's MoE routing). Steps 1 and 2 are skipped; steps 3 to 8 run as in
 * moe_latent_forward with:
 *   topk_ids [T][K] int32  device: the experts of each token, each in [0, E).
 *                          A token may list an expert more than once (each
 *                          listing is its own route row). Ids outside
 *                          [0, E) are not reported: they are clamped into
 *                          range, so the result is unspecified but no
 *                          access leaves the weights.
 *   topk_w   [T][K] fp32   device: router weights, used as given (no
 *                          renormalisation).
 * weights->router is not read (may be NULL). The grouping and the clamped
 * ids are left in the workspace as for moe_latent_forward (views OFFSETS,
 * SORTED, IDS); the weights view is not written. Same errors as
 * moe_latent_forward.
 */
int moe_latent_forward_routed(const moe_dims *dims, int32_t T, const uint16_t *x,
                              const int32_t *topk_ids, const float *topk_w,
                              const moe_weights *weights, uint16_t *out,
                              void *workspace, size_t workspace_bytes,
                              void *hip_stream);

/*
 * moe_block_forward -- the layer inside its block: the sandwich norms and the
 * residual ("Soporte de día 0 para Muse Spark Open en vLLM", section
 * "Arquitectura del modelo": out = x + post_norm(F(norm(x))); section
 * "Nvidia": the router is fed by the norm's fp32 output):
 *   n      = resid[t] / sqrt(mean(resid[t]^2) + block_eps) * pre_gain
 *            (fp64; the router reads fp32(n), the pooler bf16(n))
 *   f[t]   = the layer of moe_latent_forward on that input
 *   out[t] = bf16( resid[t] + f[t] / sqrt(mean(f[t]^2) + block_eps) * post_gain )
 *   resid     [T][H] bf16   the residual stream (the block's input)
 *   pre_gain  [H]    bf16   gain of the norm before the layer
 *   post_gain [H]    bf16   gain of the norm after the layer
 *   block_eps        fp32   eps inside both square roots (>= 0)
 *   out       [T][H] bf16   out; may be the same buffer as resid
 * The workspace must hold moe_block_workspace_bytes(dims, T) bytes; it also
 * holds the layer's intermediates (moe_workspace_view, including the views
 * NORM_F32, NORM_BF16 and LAYER_OUT). Same errors as moe_latent_forward, and
 * MOE_EINVAL for a null gain or a negative or non-finite block_eps.
 */
size_t moe_block_workspace_bytes(const moe_dims *dims, int32_t max_tokens);
int moe_block_forward(const moe_dims *dims, int32_t T, const uint16_t *resid,
                      const uint16_t *pre_gain, const uint16_t *post_gain,
                      float block_eps, const moe_weights *weights, uint16_t *out,
                      void *workspace, size_t workspace_bytes, void *hip_stream);

/* Same as moe_latent_forward, and additionally times each step with HIP
 * events recorded by the step's kernel launch itself (hipExtLaunchKernel),
 * so nothing else is added to the stream. stage_events: NULL, or an array of
 * 2 * MOE_N_STAGES hipEvent_t created by the caller: events 2i and 2i+1 mark
 * the start and end of step i; NULL entries are skipped. A step that needs
 * no kernel for the given T records its two events back to back. For
 * T <= 16 the router and the pooler share one launch, timed as step 0
 * (step 3 then has no kernel), and top-k and grouping share one launch,
 * timed as step 1. */
#define MOE_N_STAGES 8 /* router, top-k, permute, pool, gate/up, down, combine, unpool */
int moe_latent_forward_timed(const moe_dims *dims, int32_t T,
                             const uint16_t *x, const moe_weights *weights,
                             uint16_t *out, void *workspace,
                             size_t workspace_bytes, void *hip_stream,
                             void *const *stage_events);

/* Argument checks of moe_route / moe_latent_forward without enqueuing
 * anything (callable without a GPU). Same arguments and return codes. */
int moe_route_validate(const moe_dims *dims, int32_t T, const uint16_t *x,
                       const float *router, const int32_t *topk_ids,
                       const float *topk_w, const int32_t *expert_offsets,
                       const int32_t *sorted_routes, const float *logits_out,
                       const void *workspace, size_t workspace_bytes);
int moe_latent_forward_routed_validate(const moe_dims *dims, int32_t T,
                                       const uint16_t *x, const int32_t *topk_ids,
                                       const float *topk_w, const moe_weights *weights,
                                       const uint16_t *out, const void *workspace,
                                       size_t workspace_bytes);
int moe_block_forward_validate(const moe_dims *dims, int32_t T, const uint16_t *resid,
                               const uint16_t *pre_gain, const uint16_t *post_gain,
                               float block_eps, const moe_weights *weights,
                               const uint16_t *out, const void *workspace,
                               size_t workspace_bytes);
int moe_latent_forward_validate(const moe_dims *dims, int32_t T,
                                const uint16_t *x, const moe_weights *weights,
                                const uint16_t *out, const void *workspace,
                                size_t workspace_bytes);

/* Location of an intermediate inside the workspace after moe_latent_forward
 * for T tokens: byte offset and size. Returns MOE_EINVAL for an unknown id.
 *   MOE_VIEW_LOGITS  [T][E] fp32       MOE_VIEW_IDS    [T][K] int32
 *   MOE_VIEW_WEIGHTS [T][K] fp32       MOE_VIEW_OFFSETS [E+1] int32
 *   MOE_VIEW_SORTED  [T*K] int32       MOE_VIEW_LATENT [T][L] bf16
 *   MOE_VIEW_H       [T*K][I] bf16, row i belongs to route sorted_routes[i]
 *   MOE_VIEW_ROWS    [T*K][L] fp32, route-major (r = t*K + k)
 *   MOE_VIEW_Y       [T][L] bf16 (normed, weighted sum); not written when
 *                    MOE_VIEW_ROWS_BF16 has a nonzero size
 *   MOE_VIEW_ROWS_BF16 [T*K][L] bf16, route-major: bf16(gain * row), the
 *                    unpooler's input when few route rows (T*K <= 16 whose
 *                    latent rows fit 72 KiB, on the streaming expert path;
 *                    with NVFP4 experts one token only) let one launch
 *                    take the post-norm, the weighted sum and the
 *                    unpooler: out[t] = bf16(sum over the token's
 *                    routes of w / sqrt(mean(row^2) + eps) * (unpooler .
 *                    bf16(gain * row))), the weighted sum after the
 *                    products ("Muse Spark Open on Gaudi 2", section "The
 *                    latent MoE: A' with a per-expert norm"; both are
 *                    linear); 0 bytes otherwise (the same for
 *                    moe_latent_forward_persistent). */
#define MOE_VIEW_LOGITS 0
#define MOE_VIEW_IDS 1
#define MOE_VIEW_WEIGHTS 2
#define MOE_VIEW_OFFSETS 3
#define MOE_VIEW_SORTED 4
#define MOE_VIEW_LATENT 5
#define MOE_VIEW_H 6
#define MOE_VIEW_ROWS 7
#define MOE_VIEW_Y 8
#define MOE_VIEW_NORM_F32 9   /* moe_block_forward: [T][H] fp32 pre-norm output */
#define MOE_VIEW_NORM_BF16 10 /* moe_block_forward: [T][H] bf16 pre-norm output */
#define MOE_VIEW_LAYER_OUT 11 /* moe_block_forward: [T][H] bf16 layer output    */
/* The words that carry over between calls (256 bytes at offset 0 whatever
 * T): uint32 [0] the generation word of the routing done inside the router
 * launch (T <= 8) and of the persistent decode layer, advanced by exactly
 * one per such call; [1] status bits, bit 0 set if a router workgroup ever
 * gave up its bounded wait for that routing, bit 1 if a wait of the
 * persistent decode layer gave up (the call's output is then not valid; not
 * expected to happen; bits 2-4 name the wait: routing flag, release, tagged
 * logits); [2] the persistent
 * layer's routing flag; [3] its workgroup count; [8]-[12] and [16]-[21] its
 * last call's clock stamps (the 100 MHz constant clock, low 32 bits):
 * routing done and barriers 1-4 released; workgroup 0's start and the end
 * of its five phases (with few route rows, see MOE_VIEW_ROWS_BF16: barriers
 * 1-3, and the start and end of the unpooler's phase, which also takes the
 * post-norm and the weighted sum, in place of phases 4 and 5). */
#define MOE_VIEW_SYNC 12
#define MOE_VIEW_ROWS_BF16 13
int moe_workspace_view(const moe_dims *dims, int32_t T, int32_t which,
                       size_t *offset, size_t *bytes);

/* The same layer for one or two tokens in a single launch: the persistent
 * decode layer ("RadixArk team serves Meta's Muse Spark Open on one TPU
 * host", section "A single program for a serving step"). One grid, sized to
 * what the device holds at once, runs the router and pooler, the routing,
 * gate/up, down, the post-norm and weighted sum, and the unpooler as phases
 * separated by barriers between its workgroups (with few route rows the
 * post-norm and the weighted sum run in the unpooler's phase, as in
 * moe_latent_forward); every workgroup issues its next weights before it
 * waits. Same arguments, workspace and results as moe_latent_forward (the
 * workspace views hold the same intermediates).
 *  - T > 2, T * top_k > 64, or shapes outside what its phases are compiled
 *    for (hidden and latent multiples of 4096 with inter a multiple of
 *    2048, as the real shape is) return MOE_EUNSUPPORTED before anything is
 *    enqueued.
 *  - It assumes every workgroup of its grid is scheduled while the others
 *    wait: other kernels running on the device at the same time (another
 *    stream, another process) can keep part of the grid out; the bounded
 *    waits then give up, bit 1 of the MOE_VIEW_SYNC status word is set and
 *    the output is not valid. */
int moe_latent_forward_persistent(const moe_dims *dims, int32_t T, const uint16_t *x,
                                  const moe_weights *weights, uint16_t *out, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/* moe_latent_forward for callers that cannot allocate device memory (code
 * under HIP graph capture that must not allocate, tight serving loops,
 * harnesses that forbid hipMalloc): the same layer and the same kernels,
 * with the workspace taken from a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends. The caller still passes the inputs, the weights and
 * `out`. Allocates nothing: on the first call on a device (the current one)
 * the array's device address is looked up once (hipGetSymbolAddress) and
 * kept for that device.
 *  - T with moe_workspace_bytes(dims, T) > MOE_NOALLOC_SCRATCH_BYTES returns
 *    MOE_EWORKSPACE before anything is enqueued (at the real shape,
 *    H 8192, L 4096, E 256, K 8, I 4096: T <= 55, decode and verify).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (the layer needs no cleared workspace): calls that
 *    overlap on one GPU (several streams or host threads) race, and the
 *    caller must order them.
 *  - A device index beyond 63 returns MOE_EUNSUPPORTED; other errors as
 *    moe_latent_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_latent_forward_noalloc(const moe_dims *dims, int32_t T, const uint16_t *x,
                               const moe_weights *weights, uint16_t *out, void *hip_stream);

/* Host-side evaluation of the tile orders of the prefill kernels (tests
 * check them over many shapes; no device work). For launch `kind`:
 *  MOE_TILES_DENSE  (0): the dense projection of an a x b output (pooler,
 *                         unpooler at prefill; b a multiple of its 256-column
 *                         tiles);
 *  MOE_TILES_EXPERT (1): the LDS-staged expert kernel over a row tiles (the
 *                         grid's bound) of b column tiles each;
 *  MOE_TILES_TILED  (2): the register-staged expert kernel, likewise.
 * Returns the launch's workgroup count G (or MOE_EINVAL for a bad kind or
 * size), and when out holds 2 * G ints writes (row tile, column tile) per
 * workgroup: (-1, -1) for a dense padding workgroup; row tiles of the expert
 * kernels beyond the tiles a call lists are skipped by the kernel itself. */
#define MOE_TILES_DENSE 0
#define MOE_TILES_EXPERT 1
#define MOE_TILES_TILED 2
int moe_tile_map(int32_t kind, int32_t a, int32_t b, int32_t *out, int32_t capacity);

/* Text of a status code (static storage). */
const char *moe_status_string(int status);

/* HIP error code of the last MOE_EHIP on the calling thread (0 if none). */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
