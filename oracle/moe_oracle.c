/*
 * moe_oracle.c -- plain CPU oracle for the latent mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may call this library; the GPU product path
 * never links, loads or calls it and shares no code with it.
 *
 * What it computes, and where that is stated:
 *  - "Muse Spark Open on Gaudi 2", section "What was built": the router is an
 *    fp32 router over 256 experts choosing 8; experts run W4A16 (4-bit MXFP4
 *    weights, bf16 activations), and the CPU reference follows the same rule.
 *  - same page, section "The latent MoE: A' with a per-expert norm": every
 *    (token, route) pair is its own row; post_expert_norm is applied to each
 *    row, the rows are multiplied by the router weights and summed in fp32,
 *    and the unpooler takes 4096 back to 8192.
 *  - same page, section "Correctness": the CPU reference keeps bf16 values,
 *    accumulates at least in fp32 and dequantizes MXFP4 exactly.
 *  - same page, section "Why it needed a port": the norm is applied to each
 *    expert's output before the weighted sum.
 *  - "Soporte de dia 0 para Muse Spark Open en vLLM", section "Arquitectura
 *    del modelo", paragraph "MoE latente": one pooler (8192x4096) and one
 *    unpooler shared by all 256 experts of the layer; the experts work at
 *    width 4096.
 *
 * Readings where the pages are silent: the router reads the 8192-wide layer
 * input; the weights are a softmax over the K selected logits; ties in the
 * top-K go to the lower expert id; the expert FFN is SwiGLU
 * (silu(gate) * up, then down); the post-expert norm is an RMS norm with a
 * bf16 gain, eps inside the square root. All accumulation is done in double
 * (at least as precise as the fp32 the pages require) and values are rounded
 * once where the stored type is bf16 (latent, h, y, out) or fp32 (logits,
 * router weights, per-route rows).
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- number formats ---------------------------------------------------- */

double moe_ref_e2m1_value(unsigned code) {
  /* E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa. Exponent 0 is the
   * subnormal range: value = mantissa * 0.5. */
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

double moe_ref_e8m0_value(unsigned byte) {
  byte &= 0xFFu;
  if (byte == 0xFFu) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

double moe_ref_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

uint16_t moe_ref_round_bf16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(v);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  /* bf16 keeps 8 significant bits. a = f * 2^ex with f in [0.5, 1), so the
   * leading bit is 2^(ex-1) and the last kept bit is 2^(ex-8); below the
   * normal range the spacing stays at the subnormal quantum 2^-133. */
  int ex;
  (void)frexp(a, &ex);
  int q = ex - 8;
  if (q < -133) q = -133;
  double r = nearbyint(ldexp(a, -q)); /* default mode: nearest, ties to even */
  double res = ldexp(r, q);
  if (res > 0x1.FEp127) return (uint16_t)(sign | 0x7F80u); /* above max finite */
  float f = (float)res; /* exact: res has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* ---- A1: router logits --------------------------------------------------- */

void moe_ref_router_logits(int T, int H, int E, const uint16_t *x,
                           const float *router, float *logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += moe_ref_bf16_value(x[(size_t)t * H + h]) * (double)router[(size_t)e * H + h];
      logits[(size_t)t * E + e] = (float)acc;
    }
}

/* Router logits for an fp32 input (the sandwich pre-norm's output): every
 * product of two fp32 values is exact in double; the same sum and rounding. */
void moe_ref_router_logits_f32(int T, int H, int E, const float *x,
                               const float *router, float *logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += (double)x[(size_t)t * H + h] * (double)router[(size_t)e * H + h];
      logits[(size_t)t * E + e] = (float)acc;
    }
}

/* ---- A2: top-K and router weights ---------------------------------------- */

/* 1 if (a, ia) ranks before (b, ib): larger value first, NaN last, equal
 * values (including -0 and +0) by lower id. */
static int ranks_before(float a, int ia, float b, int ib) {
  int an = isnan(a), bn = isnan(b);
  if (an || bn) {
    if (an && bn) return ia < ib;
    return bn;
  }
  if (a > b) return 1;
  if (a < b) return 0;
  return ia < ib;
}

void moe_ref_topk(int T, int E, int K, const float *logits, int32_t *ids,
                  float *w) {
  char *taken = (char *)calloc((size_t)E, 1);
  double *a = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    /* selection: the k-th pick is the best expert not yet picked */
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      ids[(size_t)t * K + k] = best;
    }
    /* softmax over the K selected logits, shifted by the largest one */
    double m = (double)l[ids[(size_t)t * K]];
    double sum = 0.0;
    for (int k = 0; k < K; ++k) {
      a[k] = exp((double)l[ids[(size_t)t * K + k]] - m);
      sum += a[k];
    }
    for (int k = 0; k < K; ++k) w[(size_t)t * K + k] = (float)(a[k] / sum);
  }
  free(a);
  free(taken);
}

/* ---- A3: route permutation ---------------------------------------------- */

void moe_ref_permute(int T, int K, int E, const int32_t *ids,
                     int32_t *offsets, int32_t *sorted_routes) {
  int R = T * K;
  int32_t *fill = (int32_t *)calloc((size_t)E + 1, sizeof(int32_t));
  for (int e = 0; e <= E; ++e) offsets[e] = 0;
  for (int r = 0; r < R; ++r) offsets[ids[r] + 1] += 1; /* counts, shifted */
  for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  for (int r = 0; r < R; ++r) {
    int e = ids[r];
    sorted_routes[offsets[e] + fill[e]] = r;
    fill[e] += 1;
  }
  free(fill);
}

/* ---- A4 / A8: dense bf16 projections --------------------------------------- */

void moe_ref_linear_bf16(int T, int N, int Kd, const uint16_t *x,
                         const uint16_t *w, uint16_t *y) {
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < Kd; ++k)
        acc += moe_ref_bf16_value(x[(size_t)t * Kd + k]) *
               moe_ref_bf16_value(w[(size_t)n * Kd + k]);
      y[(size_t)t * N + n] = moe_ref_round_bf16(acc);
    }
}

/* OCP FP8 E4M3 (the "fn" variant): bit 7 sign, bits 6..3 exponent with bias
 * 7, bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); exponent 15
 * with mantissa 7 is NaN (no infinities). */
double moe_ref_e4m3_value(unsigned byte) {
  const int sign = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* ---- A5 / A6: one route row through one MXFP4 expert ---------------------- */

double moe_ref_mxfp4_value(const uint8_t *codes, const uint8_t *scales,
                           int cols, int n, int k) {
  uint8_t byte = codes[(size_t)n * (cols / 2) + k / 2];
  unsigned code = (k & 1) ? (byte >> 4) : (byte & 0x0Fu);
  return moe_ref_e2m1_value(code) *
         moe_ref_e8m0_value(scales[(size_t)n * (cols / 32) + k / 32]);
}

double moe_ref_nvfp4_value(const uint8_t *codes, const uint8_t *scales, float global,
                           int cols, int n, int k) {
  uint8_t byte = codes[(size_t)n * (cols / 2) + k / 2];
  unsigned code = (k & 1) ? (byte >> 4) : (byte & 0x0Fu);
  return moe_ref_e2m1_value(code) *
         moe_ref_e4m3_value(scales[(size_t)n * (cols / 16) + k / 16]) * (double)global;
}

/* Decode row n of a 4-bit matrix into doubles, through the 16 E2M1 values
 * and the 256 values of the scale bytes (E8M0 per 32 elements, or E4M3 per
 * 16 elements times the tensor's global scale; filled from the definitions
 * above). */
static void dequant_row(const uint8_t *codes, const uint8_t *scales, int cols,
                        int n, const double *e2m1, const double *sval, int block,
                        double global, double *out) {
  for (int k = 0; k < cols; ++k) {
    uint8_t byte = codes[(size_t)n * (cols / 2) + k / 2];
    unsigned code = (k & 1) ? (byte >> 4) : (byte & 0x0Fu);
    out[k] = e2m1[code] * sval[scales[(size_t)n * (cols / block) + k / block]] * global;
  }
}

void moe_ref_expert_row(int L, int I, const uint16_t *lat_row,
                        const uint8_t *w13_codes, const uint8_t *w13_scales,
                        const uint8_t *w2_codes, const uint8_t *w2_scales,
                        uint16_t *h_out, float *row_out) {
  moe_ref_expert_row_fmt(MOE_REF_MXFP4, L, I, lat_row, w13_codes, w13_scales, 1.0f, w2_codes,
                         w2_scales, 1.0f, h_out, row_out);
}

void moe_ref_expert_row_fmt(int fmt, int L, int I, const uint16_t *lat_row,
                            const uint8_t *w13_codes, const uint8_t *w13_scales, float w13_global,
                            const uint8_t *w2_codes, const uint8_t *w2_scales, float w2_global,
                            uint16_t *h_out, float *row_out) {
  double e2m1[16], sval[256];
  const int block = fmt == MOE_REF_NVFP4 ? 16 : 32;
  const double g13 = fmt == MOE_REF_NVFP4 ? (double)w13_global : 1.0;
  const double g2 = fmt == MOE_REF_NVFP4 ? (double)w2_global : 1.0;
  for (unsigned c = 0; c < 16; ++c) e2m1[c] = moe_ref_e2m1_value(c);
  for (unsigned b = 0; b < 256; ++b)
    sval[b] = fmt == MOE_REF_NVFP4 ? moe_ref_e4m3_value(b) : moe_ref_e8m0_value(b);
  double *a = (double *)malloc(sizeof(double) * (size_t)L);
  double *wg = (double *)malloc(sizeof(double) * (size_t)(L > I ? L : I));
  double *wu = (double *)malloc(sizeof(double) * (size_t)L);
  double *h = (double *)malloc(sizeof(double) * (size_t)I);
  for (int l = 0; l < L; ++l) a[l] = moe_ref_bf16_value(lat_row[l]);
  /* gate row n and up row I+n of W13, then SwiGLU, rounded to bf16 */
  for (int n = 0; n < I; ++n) {
    dequant_row(w13_codes, w13_scales, L, n, e2m1, sval, block, g13, wg);
    dequant_row(w13_codes, w13_scales, L, I + n, e2m1, sval, block, g13, wu);
    double g = 0.0, u = 0.0;
    for (int l = 0; l < L; ++l) {
      g += a[l] * wg[l];
      u += a[l] * wu[l];
    }
    double silu = g / (1.0 + exp(-g));
    uint16_t hb = moe_ref_round_bf16(silu * u);
    if (h_out) h_out[n] = hb;
    h[n] = moe_ref_bf16_value(hb);
  }
  /* down projection: row m of W2 against h, rounded to fp32 */
  for (int m = 0; m < L; ++m) {
    dequant_row(w2_codes, w2_scales, I, m, e2m1, sval, block, g2, wg);
    double acc = 0.0;
    for (int n = 0; n < I; ++n) acc += h[n] * wg[n];
    row_out[m] = (float)acc;
  }
  free(h);
  free(wu);
  free(wg);
  free(a);
}

/* ---- A7: post-expert norm and router-weighted sum ------------------------ */

void moe_ref_rmsnorm_row(int L, const float *row, const uint16_t *gain,
                         double eps, double *nrm) {
  double ss = 0.0;
  for (int m = 0; m < L; ++m) ss += (double)row[m] * (double)row[m];
  double s = 1.0 / sqrt(ss / (double)L + eps);
  for (int m = 0; m < L; ++m)
    nrm[m] = (double)row[m] * s * moe_ref_bf16_value(gain[m]);
}

void moe_ref_combine_norm(int K, int L, const float *rows, const float *w,
                          const int32_t *ids, const uint16_t *gain,
                          int gain_per_expert, double eps, int identity,
                          uint16_t *ybf) {
  double *y = (double *)calloc((size_t)L, sizeof(double));
  double *nrm = (double *)malloc(sizeof(double) * (size_t)L);
  for (int k = 0; k < K; ++k) {
    const uint16_t *g = gain_per_expert ? gain + (size_t)ids[k] * L : gain;
    if (identity) {
      for (int m = 0; m < L; ++m) nrm[m] = (double)rows[(size_t)k * L + m];
    } else {
      moe_ref_rmsnorm_row(L, rows + (size_t)k * L, g, eps, nrm);
    }
    for (int m = 0; m < L; ++m) y[m] += (double)w[k] * nrm[m];
  }
  for (int m = 0; m < L; ++m) ybf[m] = moe_ref_round_bf16(y[m]);
  free(nrm);
  free(y);
}

void moe_ref_combine(int K, int L, const float *rows, const float *w,
                     const int32_t *ids, const uint16_t *gain,
                     int gain_per_expert, double eps, uint16_t *ybf) {
  moe_ref_combine_norm(K, L, rows, w, ids, gain, gain_per_expert, eps, 0, ybf);
}

/* ---- the whole layer -------------------------------------------------------- */

/* Steps A4 to A8 for token t, given its K routes (ids, w). Scratch: lat [L],
 * h [I], rows [K][L]. Writes out[t] and the optional intermediates. */
static void token_after_routing(const moe_ref_dims *d, int t, const uint16_t *xt,
                                const int32_t *ids, const float *w,
                                const uint16_t *pooler, const uint8_t *w13_codes,
                                const uint8_t *w13_scales, const uint8_t *w2_codes,
                                const uint8_t *w2_scales, const uint16_t *gain,
                                const uint16_t *unpooler, uint16_t *lat, uint16_t *h,
                                float *rows, uint16_t *ybf, uint16_t *out,
                                uint16_t *lat_o, uint16_t *h_o, float *rows_o,
                                uint16_t *ybf_o) {
  const int H = d->hidden, L = d->latent, I = d->inter, K = d->top_k;
  const int block = d->expert_format == MOE_REF_NVFP4 ? 16 : 32;  /* elements per scale byte */
  const size_t w13c = (size_t)2 * I * (L / 2), w13s = (size_t)2 * I * (L / block);
  const size_t w2c = (size_t)L * (I / 2), w2s = (size_t)L * (I / block);
  moe_ref_linear_bf16(1, L, H, xt, pooler, lat);           /* A4 */
  for (int k = 0; k < K; ++k) {                            /* A5, A6 */
    const size_t e = (size_t)ids[k];
    moe_ref_expert_row_fmt(d->expert_format, L, I, lat, w13_codes + e * w13c,
                           w13_scales + e * w13s, d->w13_global ? d->w13_global[e] : 1.0f,
                           w2_codes + e * w2c, w2_scales + e * w2s,
                           d->w2_global ? d->w2_global[e] : 1.0f, h, rows + (size_t)k * L);
    if (h_o) memcpy(h_o + ((size_t)t * K + k) * I, h, sizeof(uint16_t) * (size_t)I);
  }
  moe_ref_combine_norm(K, L, rows, w, ids, gain, d->gain_per_expert, d->norm_eps,
                       d->post_norm_identity, ybf);        /* A7 */
  moe_ref_linear_bf16(1, H, L, ybf, unpooler, out + (size_t)t * H); /* A8 */
  if (lat_o) memcpy(lat_o + (size_t)t * L, lat, sizeof(uint16_t) * (size_t)L);
  if (rows_o) memcpy(rows_o + (size_t)t * K * L, rows, sizeof(float) * (size_t)K * L);
  if (ybf_o) memcpy(ybf_o + (size_t)t * L, ybf, sizeof(uint16_t) * (size_t)L);
}

int moe_ref_latent_forward(const moe_ref_dims *d, int T, const uint16_t *x,
                           const float *router, const uint16_t *pooler,
                           const uint8_t *w13_codes, const uint8_t *w13_scales,
                           const uint8_t *w2_codes, const uint8_t *w2_scales,
                           const uint16_t *gain, const uint16_t *unpooler,
                           uint16_t *out, float *logits_o, int32_t *ids_o,
                           float *w_o, uint16_t *lat_o, uint16_t *h_o,
                           float *rows_o, uint16_t *ybf_o) {
  const int H = d->hidden, L = d->latent, I = d->inter, E = d->n_experts,
            K = d->top_k;
  float *logits = (float *)malloc(sizeof(float) * (size_t)E);
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
  float *w = (float *)malloc(sizeof(float) * (size_t)K);
  uint16_t *lat = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
  uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
  float *rows = (float *)malloc(sizeof(float) * (size_t)K * L);
  uint16_t *ybf = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
  int rc = 0;
  if (!logits || !ids || !w || !lat || !h || !rows || !ybf) {
    rc = -1;
    goto done;
  }
  for (int t = 0; t < T; ++t) {
    const uint16_t *xt = x + (size_t)t * H;
    moe_ref_router_logits(1, H, E, xt, router, logits);     /* A1 */
    moe_ref_topk(1, E, K, logits, ids, w);                   /* A2 */
    token_after_routing(d, t, xt, ids, w, pooler, w13_codes, w13_scales, w2_codes,
                        w2_scales, gain, unpooler, lat, h, rows, ybf, out, lat_o,
                        h_o, rows_o, ybf_o);
    if (logits_o) memcpy(logits_o + (size_t)t * E, logits, sizeof(float) * (size_t)E);
    if (ids_o) memcpy(ids_o + (size_t)t * K, ids, sizeof(int32_t) * (size_t)K);
    if (w_o) memcpy(w_o + (size_t)t * K, w, sizeof(float) * (size_t)K);
  }
done:
  free(logits); free(ids); free(w); free(lat); free(h); free(rows); free(ybf);
  return rc;
}

int moe_ref_latent_forward_routed(const moe_ref_dims *d, int T, const uint16_t *x,
                                  const int32_t *ids, const float *w,
                                  const uint16_t *pooler, const uint8_t *w13_codes,
                                  const uint8_t *w13_scales, const uint8_t *w2_codes,
                                  const uint8_t *w2_scales, const uint16_t *gain,
                                  const uint16_t *unpooler, uint16_t *out,
                                  uint16_t *lat_o, uint16_t *h_o, float *rows_o,
                                  uint16_t *ybf_o) {
  const int H = d->hidden, L = d->latent, I = d->inter, E = d->n_experts,
            K = d->top_k;
  for (size_t r = 0; r < (size_t)T * K; ++r)
    if (ids[r] < 0 || ids[r] >= E) return -2;
  uint16_t *lat = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
  uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
  float *rows = (float *)malloc(sizeof(float) * (size_t)K * L);
  uint16_t *ybf = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
  int rc = 0;
  if (!lat || !h || !rows || !ybf) {
    rc = -1;
  } else {
    for (int t = 0; t < T; ++t)
      token_after_routing(d, t, x + (size_t)t * H, ids + (size_t)t * K, w + (size_t)t * K,
                          pooler, w13_codes, w13_scales, w2_codes, w2_scales, gain,
                          unpooler, lat, h, rows, ybf, out, lat_o, h_o, rows_o, ybf_o);
  }
  free(lat); free(h); free(rows); free(ybf);
  return rc;
}


/* ---- the block around the layer: sandwich norms and residual ------------- */

void moe_ref_pre_norm(int T, int H, const uint16_t *resid, const uint16_t *gain,
                      double eps, float *n_f32, uint16_t *n_bf16) {
  for (int t = 0; t < T; ++t) {
    const uint16_t *r = resid + (size_t)t * H;
    double ss = 0.0;
    for (int h = 0; h < H; ++h) ss += moe_ref_bf16_value(r[h]) * moe_ref_bf16_value(r[h]);
    const double s = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; ++h) {
      const double n = moe_ref_bf16_value(r[h]) * s * moe_ref_bf16_value(gain[h]);
      if (n_f32) n_f32[(size_t)t * H + h] = (float)n;
      if (n_bf16) n_bf16[(size_t)t * H + h] = moe_ref_round_bf16(n);
    }
  }
}

void moe_ref_post_norm_residual(int T, int H, const uint16_t *resid, const uint16_t *f,
                                const uint16_t *gain, double eps, uint16_t *out) {
  for (int t = 0; t < T; ++t) {
    const uint16_t *ft = f + (size_t)t * H;
    double ss = 0.0;
    for (int h = 0; h < H; ++h) ss += moe_ref_bf16_value(ft[h]) * moe_ref_bf16_value(ft[h]);
    const double s = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; ++h) {
      const double v = moe_ref_bf16_value(resid[(size_t)t * H + h]) +
                       moe_ref_bf16_value(ft[h]) * s * moe_ref_bf16_value(gain[h]);
      out[(size_t)t * H + h] = moe_ref_round_bf16(v);
    }
  }
}

int moe_ref_block_forward(const moe_ref_dims *d, int T, const uint16_t *resid,
                          const uint16_t *pre_gain, const uint16_t *post_gain,
                          double block_eps, const float *router, const uint16_t *pooler,
                          const uint8_t *w13_codes, const uint8_t *w13_scales,
                          const uint8_t *w2_codes, const uint8_t *w2_scales,
                          const uint16_t *gain, const uint16_t *unpooler, uint16_t *out,
                          float *n_f32_o, uint16_t *n_bf16_o, float *logits_o,
                          int32_t *ids_o, float *w_o, uint16_t *f_o) {
  const int H = d->hidden, L = d->latent, I = d->inter, E = d->n_experts,
            K = d->top_k;
  float *nf = (float *)malloc(sizeof(float) * (size_t)H);
  uint16_t *nb = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H);
  float *logits = (float *)malloc(sizeof(float) * (size_t)E);
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
  float *w = (float *)malloc(sizeof(float) * (size_t)K);
  uint16_t *lat = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
  uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
  float *rows = (float *)malloc(sizeof(float) * (size_t)K * L);
  uint16_t *ybf = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
  uint16_t *f = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
  int rc = 0;
  if (!nf || !nb || !logits || !ids || !w || !lat || !h || !rows || !ybf || !f) {
    rc = -1;
    goto done;
  }
  for (int t = 0; t < T; ++t) {
    const uint16_t *rt = resid + (size_t)t * H;
    moe_ref_pre_norm(1, H, rt, pre_gain, block_eps, nf, nb);     /* norm(x) */
    moe_ref_router_logits_f32(1, H, E, nf, router, logits);      /* A1 on the fp32 norm */
    moe_ref_topk(1, E, K, logits, ids, w);                       /* A2 */
    token_after_routing(d, t, nb, ids, w, pooler, w13_codes, w13_scales, w2_codes,
                        w2_scales, gain, unpooler, lat, h, rows, ybf, f, NULL, NULL,
                        NULL, NULL);                             /* A4-A8: F(norm(x)) */
    if (n_f32_o) memcpy(n_f32_o + (size_t)t * H, nf, sizeof(float) * (size_t)H);
    if (n_bf16_o) memcpy(n_bf16_o + (size_t)t * H, nb, sizeof(uint16_t) * (size_t)H);
    if (logits_o) memcpy(logits_o + (size_t)t * E, logits, sizeof(float) * (size_t)E);
    if (ids_o) memcpy(ids_o + (size_t)t * K, ids, sizeof(int32_t) * (size_t)K);
    if (w_o) memcpy(w_o + (size_t)t * K, w, sizeof(float) * (size_t)K);
  }
  moe_ref_post_norm_residual(T, H, resid, f, post_gain, block_eps, out); /* x + post_norm(F) */
  if (f_o) memcpy(f_o, f, sizeof(uint16_t) * (size_t)T * H);
done:
  free(nf); free(nb); free(logits); free(ids); free(w); free(lat); free(h); free(rows);
  free(ybf); free(f);
  return rc;
}
