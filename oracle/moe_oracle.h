/*
 * moe_oracle.h -- plain CPU oracle for the latent mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may call this library. The GPU product path
 * never links, loads or calls it, and it shares no code, header, table or
 * constant with the GPU library.
 *
 * Every pointer is a host pointer. bf16 values are passed as their 16-bit
 * patterns (uint16_t). Arithmetic is IEEE double with round-to-nearest-even;
 * values are rounded only where the layer's stored types demand it (see the
 * per-function comments). Nothing here is blocked, fused or reordered.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats --------------------------------------------------- */

/* Value of a 4-bit FP4 E2M1 code (bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa), from the OCP Microscaling (MX) v1.0 element format. */
double moe_ref_e2m1_value(unsigned code);

/* Value of an E8M0 scale byte: 2^(b-127); the byte 0xFF is NaN (OCP MX v1.0). */
double moe_ref_e8m0_value(unsigned byte);

/* Value of an OCP FP8 E4M3 byte ("fn": bias 7, no infinities, S.1111.111 is
 * NaN, exponent 0 subnormal), the NVFP4 block scale. */
double moe_ref_e4m3_value(unsigned byte);

/* bf16 bit pattern -> exact double. */
double moe_ref_bf16_value(uint16_t bits);

/* double -> bf16 bit pattern, one round-to-nearest-even step (no detour
 * through float), subnormals kept, overflow to infinity, NaN quieted. */
uint16_t moe_ref_round_bf16(double v);

/* ---- the layer, step by step ------------------------------------------- */

/* Router logits: logits[t][e] = fp32( sum_h x[t][h] * router[e][h] ).
 * x: [T][H] bf16, router: [E][H] fp32, logits: [T][E] fp32.
 * The sum is taken in double in ascending h and rounded once to fp32. */
void moe_ref_router_logits(int T, int H, int E, const uint16_t *x,
                           const float *router, float *logits);

/* The same router logits for an fp32 input x [T][H] (the sandwich
 * pre-norm's output; every product of two fp32 values is exact in double). */
void moe_ref_router_logits_f32(int T, int H, int E, const float *x,
                               const float *router, float *logits);

/* Top-K selection and router weights for T tokens.
 * Order: larger logit first; equal logits (-0 == +0) by lower expert id;
 * NaN ranks below every number (and among NaNs, lower id first).
 * ids[t][k] is the k-th expert in that order; w[t][k] is the softmax of the
 * K selected logits, computed in double and rounded to fp32. */
void moe_ref_topk(int T, int E, int K, const float *logits, int32_t *ids,
                  float *w);

/* Route permutation. Route r = t*K + k. counts[e] = routes with ids[r]==e,
 * offsets[0..E] = exclusive prefix sum of counts (offsets[E] = T*K), and
 * sorted_routes lists the routes of expert 0, then expert 1, ..., each group
 * in ascending r. */
void moe_ref_permute(int T, int K, int E, const int32_t *ids,
                     int32_t *offsets, int32_t *sorted_routes);

/* Dense projection y[t][n] = bf16( sum_k x[t][k] * w[n][k] ).
 * x: [T][Kd] bf16, w: [N][Kd] bf16 (output-major), y: [T][N] bf16.
 * Used for the pooler (Kd=hidden, N=latent) and unpooler (Kd=latent,
 * N=hidden). The sum is taken in double and rounded once to bf16. */
void moe_ref_linear_bf16(int T, int N, int Kd, const uint16_t *x,
                         const uint16_t *w, uint16_t *y);

/* Value of element (n, k) of an MXFP4 matrix with `cols` columns:
 * codes [rows][cols/2], byte j holds column 2j in bits 0..3 and column 2j+1
 * in bits 4..7; scales [rows][cols/32], one E8M0 byte per 32 consecutive
 * columns. Exact in double. */
double moe_ref_mxfp4_value(const uint8_t *codes, const uint8_t *scales,
                           int cols, int n, int k);

/* Value of element (n, k) of an NVFP4 matrix: E2M1 codes as for MXFP4,
 * scales [rows][cols/16] one E4M3 byte per 16 consecutive columns, times the
 * tensor's fp32 global scale. Exact in double. */
double moe_ref_nvfp4_value(const uint8_t *codes, const uint8_t *scales, float global,
                           int cols, int n, int k);

/* Expert weight formats */
#define MOE_REF_MXFP4 0 /* E2M1 + E8M0 per 32 */
#define MOE_REF_NVFP4 1 /* E2M1 + E4M3 per 16, times a per-tensor fp32 scale */

/* One route row through one expert (W4A16 SwiGLU FFN).
 * lat_row [L] bf16; expert tensors of this expert only:
 *   w13_codes [2I][L/2], w13_scales [2I][L/32]: rows 0..I-1 gate, I..2I-1 up
 *   w2_codes  [L][I/2],  w2_scales  [L][I/32]
 * g[n] = sum_l lat[l]*W13[n][l], u[n] = sum_l lat[l]*W13[I+n][l] (double),
 * h[n] = bf16( silu(g[n]) * u[n] ), silu(z) = z / (1 + exp(-z)),
 * row[m] = fp32( sum_n h[n]*W2[m][n] ).
 * h_out [I] (may be NULL), row_out [L]. */
void moe_ref_expert_row(int L, int I, const uint16_t *lat_row,
                        const uint8_t *w13_codes, const uint8_t *w13_scales,
                        const uint8_t *w2_codes, const uint8_t *w2_scales,
                        uint16_t *h_out, float *row_out);

/* The same in either format: for NVFP4 the scales are [2I][L/16] and
 * [L][I/16] E4M3 bytes and w13_global / w2_global the tensors' fp32 scales
 * (ignored for MXFP4). */
void moe_ref_expert_row_fmt(int fmt, int L, int I, const uint16_t *lat_row,
                            const uint8_t *w13_codes, const uint8_t *w13_scales, float w13_global,
                            const uint8_t *w2_codes, const uint8_t *w2_scales, float w2_global,
                            uint16_t *h_out, float *row_out);

/* RMS norm of one route row: nrm[m] = row[m] / sqrt(mean(row^2) + eps) * gain[m]
 * (double, gain given as bf16). */
void moe_ref_rmsnorm_row(int L, const float *row, const uint16_t *gain,
                         double eps, double *nrm);

/* Post-expert norm and router-weighted sum for one token:
 * y[m] = sum_{k ascending} w[k] * rmsnorm(rows[k])[m], ybf = bf16(y).
 * rows [K][L] fp32; gain is [L] (gain_per_expert == 0) or [E][L] indexed by
 * ids[k] (gain_per_expert != 0). */
void moe_ref_combine(int K, int L, const float *rows, const float *w,
                     const int32_t *ids, const uint16_t *gain,
                     int gain_per_expert, double eps, uint16_t *ybf);

/* The same with the post-expert norm selectable: identity != 0 replaces the
 * norm by the identity (nrm = row, no gain), the form in which the
 * per-route expansion must equal a fused weighted top-K sum of the expert
 * FFNs ("Muse Spark Open on Gaudi 2", sections "Why it needed a port" and
 * "The latent MoE: A' with a per-expert norm": the stock fused op returns
 * only that weighted sum, which is why the port expands routes into rows). */
void moe_ref_combine_norm(int K, int L, const float *rows, const float *w,
                          const int32_t *ids, const uint16_t *gain,
                          int gain_per_expert, double eps, int identity,
                          uint16_t *ybf);

/* Whole layer for T tokens with full expert tensors
 * (w13_* [E][2I][...], w2_* [E][L][...]). out [T][H] bf16.
 * Optional intermediates (each may be NULL): logits [T][E], ids [T][K],
 * w [T][K], lat [T][L], h [T*K][I] and rows [T*K][L] indexed by route
 * r = t*K + k, ybf [T][L]. Returns 0, or -1 if scratch allocation fails. */
typedef struct {
  int hidden, latent, inter, n_experts, top_k;
  double norm_eps;
  int gain_per_expert;
  int expert_format;         /* MOE_REF_MXFP4 or MOE_REF_NVFP4 */
  const float *w13_global;   /* NVFP4: [E] per-tensor scales of W13 (NULL: 1) */
  const float *w2_global;    /* NVFP4: [E] per-tensor scales of W2 (NULL: 1) */
  int post_norm_identity;    /* 1: the post-expert norm replaced by the identity
                                (see moe_ref_combine_norm); 0: the RMS norm */
} moe_ref_dims;

int moe_ref_latent_forward(const moe_ref_dims *d, int T, const uint16_t *x,
                           const float *router, const uint16_t *pooler,
                           const uint8_t *w13_codes, const uint8_t *w13_scales,
                           const uint8_t *w2_codes, const uint8_t *w2_scales,
                           const uint16_t *gain, const uint16_t *unpooler,
                           uint16_t *out, float *logits, int32_t *ids,
                           float *w, uint16_t *lat, uint16_t *h, float *rows,
                           uint16_t *ybf);

/* Steps A4 to A8 with the routing given (routing replay): the same layer as
 * moe_ref_latent_forward with ids [T][K] (each in [0, E); a token may list an
 * expert more than once, each listing being its own route row) and w [T][K]
 * taken as they are, in place of the router's choice. The router weights are
 * used as given (no renormalisation). Optional intermediates as above.
 * Returns 0, -1 if scratch allocation fails, -2 for an id outside [0, E). */
int moe_ref_latent_forward_routed(const moe_ref_dims *d, int T, const uint16_t *x,
                                  const int32_t *ids, const float *w,
                                  const uint16_t *pooler, const uint8_t *w13_codes,
                                  const uint8_t *w13_scales, const uint8_t *w2_codes,
                                  const uint8_t *w2_scales, const uint16_t *gain,
                                  const uint16_t *unpooler, uint16_t *out,
                                  uint16_t *lat, uint16_t *h, float *rows,
                                  uint16_t *ybf);

/* ---- the block around the layer ---------------------------------------
 * "Soporte de día 0 para Muse Spark Open en vLLM", section "Arquitectura del
 * modelo", paragraph on the sandwich norm: a norm before and another after
 * the block, out = x + post_norm(F(norm(x))); section "Nvidia": the router
 * GEMM is fed by the norm's fp32 output. Both norms are RMS norms over the
 * H-wide row with a bf16 gain [H] and the block's eps. */

/* Pre-norm of T rows of the residual stream resid [T][H] bf16:
 * n = v / sqrt(mean(v^2) + eps) * gain in double (sum of squares in
 * ascending h), rounded once to fp32 (n_f32, the router's input) and once to
 * bf16 (n_bf16, the pooler's input). Either output may be NULL. */
void moe_ref_pre_norm(int T, int H, const uint16_t *resid, const uint16_t *gain,
                      double eps, float *n_f32, uint16_t *n_bf16);

/* Post-norm of the layer's bf16 output f [T][H] plus the residual:
 * out = bf16( resid + f / sqrt(mean(f^2) + eps) * gain ), in double with one
 * rounding. */
void moe_ref_post_norm_residual(int T, int H, const uint16_t *resid, const uint16_t *f,
                                const uint16_t *gain, double eps, uint16_t *out);

/* The block: out = resid + post_norm(layer(pre_norm(resid))), where the
 * layer's router reads the fp32 pre-norm output and its pooler the bf16 one.
 * Optional intermediates: n_f32 [T][H], n_bf16 [T][H], logits [T][E],
 * ids [T][K], w [T][K], f [T][H] (the layer's output). Returns 0 or -1. */
int moe_ref_block_forward(const moe_ref_dims *d, int T, const uint16_t *resid,
                          const uint16_t *pre_gain, const uint16_t *post_gain,
                          double block_eps, const float *router, const uint16_t *pooler,
                          const uint8_t *w13_codes, const uint8_t *w13_scales,
                          const uint8_t *w2_codes, const uint8_t *w2_scales,
                          const uint16_t *gain, const uint16_t *unpooler, uint16_t *out,
                          float *n_f32, uint16_t *n_bf16, float *logits, int32_t *ids,
                          float *w, uint16_t *f);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
