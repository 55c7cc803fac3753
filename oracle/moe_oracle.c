/*
 * moe_oracle.c -- plain, slow, double-precision reference of the sparse Mixture-of-Experts layer
 * forward pass (Nemotron 3 MoE layer and its LatentMoE variant).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. The HIP library never includes, links or calls it, and the two
 * share no code: formats are decoded here from their definitions, independently of the kernels.
 *
 * Every function is a direct transcription of the layer's definition: single-threaded loops in
 * double precision, inputs read exactly (fp32, bf16 and e4m3 x fp32-scale values are all exact
 * doubles), no blocking, no reordering, no BLAS.
 *
 * Sources (page title, section):
 *  [MTP]  MarkTechPost article "NVIDIA AI发布了Nemotron 3：一款混合Mamba Transformer MoE堆栈",
 *         section "混合Mamba Transformer MoE架构": the MoE layer replaces the FFN; a learned router
 *         picks a small subset of routable experts per token (6 of 128 in Nano).
 *  [N3N]  "Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer 智能體推理模型", section 2.2,
 *         training hyper-parameters: DeepSeek's aux-loss-free load balancing; section 4:
 *         selective-precision FP8 post-training quantisation.
 *  [N3A]  "Nemotron 3 Nano: Open, Efficient Mixture-of-Experts Hybrid Mamba-Transformer Model for
 *         Agentic Reasoning", section "技术框架": router -> selected experts -> weighted combination.
 *  [N3W]  "NVIDIA Nemotron 3: Efficient and Open Intelligence", section 2.2 (LatentMoE, Figure 3b,
 *         Table 1) and the speed-read equation E' = E*H/l, k' = k*H/l; section 2.4 (latent
 *         projections kept in BF16; NVFP4 micro-block scaling with E2M1 elements, whose native
 *         gfx950 counterpart, the OCP microscaling formats MXFP4 / MXFP8, is what the block-scaled
 *         expert weights here use).
 * Where the pages leave a step open, the reading taken is stated at the function.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_F64 = 3, ORC_MXFP4 = 4, ORC_MXFP8 = 5 };
enum { ORC_OK = 0, ORC_EINVAL = -1 };

/* A row-major matrix view [rows][cols] in its storage format (cols counts elements).
 *   e4m3:   value (r, c) = e4m3(code[r][c]) * scale[r], one fp32 scale per row (output channel);
 *   MXFP8:  value (r, c) = e4m3(code[r][c]) * e8m0(scale[r][c / 32]), uint8 block scales;
 *   MXFP4:  value (r, c) = e2m1(nibble c of row r) * e8m0(scale[r][c / 32]); a row holds cols / 2
 *           bytes, element 2i in the low nibble of byte i and element 2i + 1 in the high one. */
typedef struct {
  const void *data;
  const void *scale;
  int32_t dtype;
  int32_t pad_;
  int64_t cols;
} orc_mat;

/* One layer call. Expert stacks are viewed as 2-D: W_up is [E*I][D], W_down is [E*D][I]. */
typedef struct {
  int32_t T, H, E, k, I, I_shared, latent, fp8_emulate;
  orc_mat x, W_r;
  const float *b;
  orc_mat W_up, W_down, Ws_up, Ws_down, W_in, W_out;
} orc_layer;

/* ------------------------------------------------------------------ storage formats */

/* bf16 is the upper half of an IEEE binary32 pattern. */
double orc_bf16_to_f64(uint16_t u) {
  uint32_t w = (uint32_t)u << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* OCP 8-bit E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 holds
 * subnormals m/8 * 2^-6; there are no infinities and S.1111.111 is NaN; largest finite is 448. */
double orc_e4m3_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest e4m3 code (ties to even), saturating to +-448. v must not be NaN. */
uint8_t orc_f64_to_e4m3(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  int ex;
  frexp(a, &ex);               /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;              /* a in [2^e, 2^(e+1)) */
  if (e < -6) e = -6;          /* below 2^-6 the quantum stays 2^-9 (subnormals) */
  double q = nearbyint(ldexp(a, 3 - e)); /* mantissa steps of 2^(e-3); default mode: ties even */
  double val = ldexp(q, e - 3);
  if (val >= 448.0) return sign | 0x7E;
  if (val == 0.0) return sign;
  if (val < ldexp(1.0, -6)) return sign | (uint8_t)nearbyint(ldexp(val, 9)); /* subnormal */
  frexp(val, &ex);
  e = ex - 1;
  int mant = (int)nearbyint(ldexp(val, 3 - e)) - 8;
  return sign | (uint8_t)(((e + 7) << 3) | mant);
}

/* OCP E2M1 (MX spec, FP4): 1 sign, 2 exponent (bias 1) and 1 mantissa bit; exponent field 0
 * holds the subnormal m * 0.5; no infinities or NaN; largest magnitude 6. */
double orc_e2m1_to_f64(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* OCP E8M0 block scale: 2^(code - 127); code 255 is NaN. */
double orc_e8m0_to_f64(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

static double at(const orc_mat *m, int64_t r, int64_t c) {
  int64_t i = r * m->cols + c;
  switch (m->dtype) {
    case ORC_F32: return (double)((const float *)m->data)[i];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)m->data)[i]);
    case ORC_E4M3:
      return orc_e4m3_to_f64(((const uint8_t *)m->data)[i]) * (double)((const float *)m->scale)[r];
    case ORC_MXFP8:
      return orc_e4m3_to_f64(((const uint8_t *)m->data)[i]) *
             orc_e8m0_to_f64(((const uint8_t *)m->scale)[r * (m->cols / 32) + c / 32]);
    case ORC_MXFP4: {
      const uint8_t byte = ((const uint8_t *)m->data)[r * (m->cols / 2) + c / 2];
      return orc_e2m1_to_f64((uint8_t)(c % 2 ? byte >> 4 : byte & 15)) *
             orc_e8m0_to_f64(((const uint8_t *)m->scale)[r * (m->cols / 32) + c / 32]);
    }
    default: return ((const double *)m->data)[i];
  }
}

/* ------------------------------------------------------------------ router */

/* Router logits z[t][e] = sum_h x[t][h] * W_r[e][h] for the listed tokens (all T if tokens is
 * NULL). The gating network reads the H-wide token, also in LatentMoE [N3W 2.2]. */
int orc_logits(const orc_layer *L, const int32_t *tokens, int32_t n, double *z) {
  if (!L || !z) return ORC_EINVAL;
  int32_t cnt = tokens ? n : L->T;
  for (int32_t a = 0; a < cnt; ++a) {
    int32_t t = tokens ? tokens[a] : a;
    for (int32_t e = 0; e < L->E; ++e) {
      double acc = 0.0;
      for (int32_t h = 0; h < L->H; ++h) acc += at(&L->x, t, h) * at(&L->W_r, e, h);
      z[(int64_t)a * L->E + e] = acc;
    }
  }
  return ORC_OK;
}

/* Top-k by selection: k rounds, each taking the largest remaining key, the lowest expert index
 * among equal keys. idx is therefore in descending key order. margin = k-th key minus the best
 * unselected key (+inf when k == E). Gates are the selected *unbiased* scores divided by their sum:
 * the bias steers which experts are chosen, never how they are weighted (aux-loss-free balancing,
 * [N3N 2.2]; sigmoid scores and renormalisation are the reading taken for the score function,
 * which the pages do not spell out). */
static void select_topk(const double *key, const double *s, int32_t E, int32_t k,
                        int32_t *idx, double *gates, double *margin, unsigned char *taken) {
  memset(taken, 0, (size_t)E);
  double last = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e; /* strict '>' keeps the lower index on ties */
    }
    taken[best] = 1;
    idx[j] = best;
    last = key[best];
  }
  if (margin) {
    if (k == E) {
      *margin = INFINITY;
    } else {
      int32_t nxt = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!taken[e] && (nxt < 0 || key[e] > key[nxt])) nxt = e;
      *margin = last - key[nxt];
    }
  }
  double sum = 0.0;
  for (int32_t j = 0; j < k; ++j) sum += s[idx[j]];
  for (int32_t j = 0; j < k; ++j) gates[j] = s[idx[j]] / sum;
}

#define ORC_EMAX 4096

/* Routing from double logits: s = 1 / (1 + exp(-z)), key = s + b, all in double. */
int orc_route(const double *z, const float *b, int32_t T, int32_t E, int32_t k, int32_t *idx,
              double *gates, double *margin) {
  if (!z || !b || !idx || !gates || E < 1 || E > ORC_EMAX || k < 1 || k > E) return ORC_EINVAL;
  double s[ORC_EMAX], key[ORC_EMAX];
  unsigned char taken[ORC_EMAX];
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      s[e] = 1.0 / (1.0 + exp(-z[(int64_t)t * E + e]));
      key[e] = s[e] + (double)b[e];
    }
    select_topk(key, s, E, k, idx + (int64_t)t * k, gates + (int64_t)t * k,
                margin ? margin + t : NULL, taken);
  }
  return ORC_OK;
}

/* Routing from fp32 logits with every value that decides the selection rounded to fp32, the
 * precision the GPU takes the decision in: s = fp32(1 / (1 + exp(-z))) evaluated in double, then
 * key = fp32(s + b) as one binary32 addition. Gates are formed in double from those fp32 s. */
int orc_route_f32(const float *z, const float *b, int32_t T, int32_t E, int32_t k, int32_t *idx,
                  double *gates, double *margin) {
  if (!z || !b || !idx || !gates || E < 1 || E > ORC_EMAX || k < 1 || k > E) return ORC_EINVAL;
  double s[ORC_EMAX], key[ORC_EMAX];
  unsigned char taken[ORC_EMAX];
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float sf = (float)(1.0 / (1.0 + exp(-(double)z[(int64_t)t * E + e])));
      volatile float kf = sf + b[e]; /* binary32 add, not contracted or widened */
      s[e] = (double)sf;
      key[e] = (double)kf;
    }
    select_topk(key, s, E, k, idx + (int64_t)t * k, gates + (int64_t)t * k,
                margin ? margin + t : NULL, taken);
  }
  return ORC_OK;
}

/* Gates of a given selection (the gate step alone): g_j = s[idx_j] / sum_j s[idx_j] with
 * s = 1 / (1 + exp(-z)) in double. Used when a selection inside the near-tie band is taken from
 * elsewhere and the layer output is recomputed for it. */
int orc_gates_for(const double *z, const int32_t *idx, int32_t T, int32_t E, int32_t k,
                  double *gates) {
  if (!z || !idx || !gates || E < 1 || k < 1 || k > E) return ORC_EINVAL;
  for (int32_t t = 0; t < T; ++t) {
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = idx[(int64_t)t * k + j];
      if (e < 0 || e >= E) return ORC_EINVAL;
      sum += 1.0 / (1.0 + exp(-z[(int64_t)t * E + e]));
    }
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = idx[(int64_t)t * k + j];
      gates[(int64_t)t * k + j] = (1.0 / (1.0 + exp(-z[(int64_t)t * E + e]))) / sum;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ dispatch */

/* Group the T*k (token, slot) pairs by expert, tokens ascending inside an expert:
 * counts[e] = number of pairs on e; offsets = exclusive prefix sum (offsets[E] = T*k);
 * perm[r] = token of the r-th pair in that order; pos[t][j] = r of pair (t, j). */
int orc_dispatch(const int32_t *idx, int32_t T, int32_t E, int32_t k, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *pos) {
  if (!idx || !counts || !offsets || !perm || !pos || E < 1 || k < 1) return ORC_EINVAL;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < (int64_t)T * k; ++p) {
    if (idx[p] < 0 || idx[p] >= E) return ORC_EINVAL;
    counts[idx[p]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t r = 0;
  for (int32_t e = 0; e < E; ++e)
    for (int32_t t = 0; t < T; ++t)
      for (int32_t j = 0; j < k; ++j)
        if (idx[(int64_t)t * k + j] == e) {
          perm[r] = t;
          pos[(int64_t)t * k + j] = r;
          ++r;
        }
  return ORC_OK;
}

/* ------------------------------------------------------------------ fp8 activation emulation */

/* Per-row e4m3 quantisation of an activation row as the fp8 path performs it: the row's scale is
 * fp32(amax / 448) (1 for an all-zero row); codes are e4m3(fp32(v * fp32(448 / amax))), i.e. the
 * row is multiplied by the rounded reciprocal of the scale; value = code * scale. Replaces v in
 * place with the dequantised value. Used only in the emulation mode. */
static void quant_row_e4m3(double *v, int64_t n) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf((float)v[i]);
    if (a > amax) amax = a;
  }
  volatile float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  volatile float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
  for (int64_t i = 0; i < n; ++i) {
    volatile float q = (float)v[i] * inv;
    v[i] = orc_e4m3_to_f64(orc_f64_to_e4m3((double)q)) * (double)scale;
  }
}

static double round_bf16(double v) {
  float f = (float)v;
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  w = (w + 0x7FFFu + ((w >> 16) & 1u)) & 0xFFFF0000u;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------ layer forward */

static double sqrelu(double a) { return a > 0.0 ? a * a : 0.0; }

/* y[a][:] for the listed tokens (all T if tokens is NULL), given their routing idx/gates (one row
 * of k per listed token).
 *   u      = W_in x_t (LatentMoE: routed experts live in the latent width l [N3W 2.2]) or x_t;
 *   acc    = sum_j g_j * W_down[e_j] relu(W_up[e_j] u)^2   (non-gated squared-ReLU experts);
 *   y_t    = W_out acc (LatentMoE) or acc;
 *   y_t   += Ws_down relu(Ws_up x_t)^2 when a shared expert is present; it is always on, outside
 *            the gate normalisation, and reads the H-wide token [N3W 2.2].
 * With fp8_emulate (8-bit or block-scaled expert weights only: e4m3, MXFP8, MXFP4) u and each h
 * row are quantised per row to e4m3 first, h after rounding to bf16, which is where those paths
 * store it; so is the LatentMoE projection u of a bf16 layer. */
int orc_forward_tokens(const orc_layer *L, const int32_t *tokens, int32_t n, const int32_t *idx,
                       const double *gates, double *y, double *work) {
  if (!L || !idx || !gates || !y || !work) return ORC_EINVAL;
  const int32_t H = L->H, I = L->I, Is = L->I_shared, Lw = L->latent;
  const int32_t D = Lw ? Lw : H;
  const int emulate = L->fp8_emulate && (L->W_up.dtype == ORC_E4M3 ||
                                         L->W_up.dtype == ORC_MXFP8 || L->W_up.dtype == ORC_MXFP4);
  /* work holds u[D], acc[D], h[max(I, I_s)] */
  double *u = work, *acc = work + D, *h = work + 2 * (int64_t)D;
  int32_t cnt = tokens ? n : L->T;
  for (int32_t a = 0; a < cnt; ++a) {
    int32_t t = tokens ? tokens[a] : a;
    double *yt = y + (int64_t)a * H;
    for (int32_t d = 0; d < D; ++d) {
      if (Lw) {
        double s = 0.0;
        for (int32_t c = 0; c < H; ++c) s += at(&L->W_in, d, c) * at(&L->x, t, c);
        u[d] = s;
      } else {
        u[d] = at(&L->x, t, d);
      }
      acc[d] = 0.0;
    }
    if (emulate) {
      if (Lw && L->x.dtype == ORC_BF16)
        for (int32_t d = 0; d < D; ++d) u[d] = round_bf16(u[d]);
      quant_row_e4m3(u, D);
    }
    for (int32_t j = 0; j < L->k; ++j) {
      int32_t e = idx[(int64_t)a * L->k + j];
      double g = gates[(int64_t)a * L->k + j];
      if (e < 0 || e >= L->E) return ORC_EINVAL;
      for (int32_t i = 0; i < I; ++i) {
        double s = 0.0;
        for (int32_t d = 0; d < D; ++d) s += at(&L->W_up, (int64_t)e * I + i, d) * u[d];
        h[i] = sqrelu(s);
      }
      if (emulate) {
        for (int32_t i = 0; i < I; ++i) h[i] = round_bf16(h[i]);
        quant_row_e4m3(h, I);
      }
      for (int32_t d = 0; d < D; ++d) {
        double s = 0.0;
        for (int32_t i = 0; i < I; ++i) s += at(&L->W_down, (int64_t)e * D + d, i) * h[i];
        acc[d] += g * s;
      }
    }
    for (int32_t c = 0; c < H; ++c) {
      if (Lw) {
        double s = 0.0;
        for (int32_t d = 0; d < D; ++d) s += at(&L->W_out, c, d) * acc[d];
        yt[c] = s;
      } else {
        yt[c] = acc[c];
      }
    }
    if (Is) {
      for (int32_t i = 0; i < Is; ++i) {
        double s = 0.0;
        for (int32_t c = 0; c < H; ++c) s += at(&L->Ws_up, i, c) * at(&L->x, t, c);
        h[i] = sqrelu(s);
      }
      for (int32_t c = 0; c < H; ++c) {
        double s = 0.0;
        for (int32_t i = 0; i < Is; ++i) s += at(&L->Ws_down, c, i) * h[i];
        yt[c] += s;
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ aux-loss-free bias update */

/* One step of aux-loss-free balancing [N3N 2.2]: an expert loaded below its target gets its
 * selection bias raised by gamma, one above it lowered by gamma, one on target left alone.
 * (The pages name the strategy only; this sign rule toward a per-expert target is the reading
 * taken. With a uniform target it is the usual rule toward the mean load.) */
int orc_bias_update(double *b, const int32_t *counts, const double *target, int32_t E,
                    double gamma) {
  if (!b || !counts || !target) return ORC_EINVAL;
  for (int32_t e = 0; e < E; ++e) {
    double d = target[e] - (double)counts[e];
    b[e] += gamma * (double)((d > 0.0) - (d < 0.0));
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ layer backward */

/* Gradient accumulators of the backward pass, all in double; any pointer may be NULL (that
 * gradient is skipped). With expert >= 0 the routed weight gradients dW_up / dW_down hold that
 * one expert only ([I][D] and [D][I]); with expert < 0 they hold the whole stacks ([E*I][D],
 * [E*D][I]). dW_r is [E][H]; dWs_up [I_s][H]; dWs_down [H][I_s]. */
typedef struct {
  double *dW_r, *dW_up, *dW_down, *dWs_up, *dWs_down;
  int32_t expert;
  int32_t pad_;
  double *dW_in, *dW_out; /* LatentMoE: [l][H] and [H][l] */
} orc_grads;

/* Backward pass of the MoE layer for the listed tokens (all T if tokens is NULL), given the
 * selection idx the forward made (one row of k per listed token) and the gradient dy of a scalar
 * loss with respect to y (one row of H per listed token).
 *
 * The selection is piecewise constant in the inputs, so it is held fixed and the gradient flows
 * through the gate weights only: with s_j = sigmoid(z_{e_j}), Z = sum_j s_j and g_j = s_j / Z
 * (the renormalised unbiased scores; the bias steers the choice and gets no gradient, as in
 * aux-loss-free balancing [N3N 2.2]), the chain rule of the forward written out step by step:
 *   a = W_up[e] x,  r = max(a, 0),  h = r^2,  Y_j = W_down[e] h,  y += g_j Y_j;
 *   dY_j = g_j dy,  dg_j = <dy, Y_j>,  dh = W_down[e]^T dY_j,  da = 2 r (.) dh,
 *   dx += W_up[e]^T da,  dW_down[e] += dY_j h^T,  dW_up[e] += da x^T;
 *   ds_j = (dg_j - sum_m g_m dg_m) / Z,  dz_{e_j} = ds_j s_j (1 - s_j)  (0 for other experts),
 *   dx += sum_j dz_{e_j} W_r[e_j],  dW_r[e_j] += dz_{e_j} x;
 *   shared expert (weight 1): a_s = Ws_up x, r_s = max(a_s, 0), dh_s = Ws_down^T dy,
 *   da_s = 2 r_s (.) dh_s, dx += Ws_up^T da_s, dWs_down += dy h_s^T, dWs_up += da_s x^T.
 * LatentMoE [N3W 2.2]: the routed experts read u = W_in x and their gated sum acc (width l)
 * leaves through y = W_out acc, so the experts see dacc = W_out^T dy in place of dy and u in place
 * of x; dW_out += dy acc^T; their input gradient du reaches x through dx += W_in^T du, and
 * dW_in += du x^T. The router and the shared expert read x in H as in the plain layer.
 * The derivative of the squared ReLU is taken as 2 max(a, 0), which is 0 at a = 0.
 * dx is [n][H] and dz [n][E] per listed token (either may be NULL). */
int orc_backward_tokens(const orc_layer *L, const int32_t *tokens, int32_t n, const int32_t *idx,
                        const double *dy, double *dx, double *dz, const orc_grads *G) {
  if (!L || !idx || !dy || L->k < 1 || L->k > ORC_EMAX) return ORC_EINVAL;
  const int32_t H = L->H, I = L->I, Is = L->I_shared, E = L->E, k = L->k, Lw = L->latent;
  const int32_t D = Lw ? Lw : H;
  const int32_t Imax = I > Is ? I : Is;
  double *r = (double *)malloc(sizeof(double) * (size_t)Imax);
  double *dh = (double *)malloc(sizeof(double) * (size_t)Imax);
  double *Y = (double *)malloc(sizeof(double) * (size_t)D);
  double *gx = (double *)malloc(sizeof(double) * (size_t)H);
  double *u = (double *)malloc(sizeof(double) * (size_t)D);    /* expert input (x or W_in x) */
  double *ge = (double *)malloc(sizeof(double) * (size_t)D);   /* gradient reaching the experts */
  double *gu = (double *)malloc(sizeof(double) * (size_t)D);   /* gradient of u */
  double *acc = (double *)malloc(sizeof(double) * (size_t)D);  /* latent: gated expert sum */
  double s[ORC_EMAX], g[ORC_EMAX], dg[ORC_EMAX];
  int rc = ORC_OK;
  if (!r || !dh || !Y || !gx || !u || !ge || !gu || !acc) { rc = ORC_EINVAL; goto done; }
  int32_t cnt = tokens ? n : L->T;
  for (int32_t a = 0; a < cnt; ++a) {
    const int32_t t = tokens ? tokens[a] : a;
    const int32_t *it = idx + (int64_t)a * k;
    const double *dyt = dy + (int64_t)a * H;
    for (int32_t c = 0; c < H; ++c) gx[c] = 0.0;
    /* gates of the given selection */
    double Z = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      if (it[j] < 0 || it[j] >= E) { rc = ORC_EINVAL; goto done; }
      double z = 0.0;
      for (int32_t c = 0; c < H; ++c) z += at(&L->x, t, c) * at(&L->W_r, it[j], c);
      s[j] = 1.0 / (1.0 + exp(-z));
      Z += s[j];
    }
    for (int32_t j = 0; j < k; ++j) g[j] = s[j] / Z;
    /* expert input u and the gradient reaching the experts' gated sum */
    for (int32_t d = 0; d < D; ++d) {
      double a = 0.0;
      if (Lw)
        for (int32_t c = 0; c < H; ++c) a += at(&L->W_in, d, c) * at(&L->x, t, c);
      else
        a = at(&L->x, t, d);
      u[d] = a;
      gu[d] = 0.0;
      acc[d] = 0.0;
      double e = 0.0;
      if (Lw)
        for (int32_t c = 0; c < H; ++c) e += at(&L->W_out, c, d) * dyt[c];
      else
        e = dyt[d];
      ge[d] = e;
    }
    /* routed experts */
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = it[j];
      const int want_w = G && (G->expert < 0 || G->expert == e);
      const int64_t ew = G && G->expert >= 0 ? 0 : e; /* row block of e in the dW arrays */
      for (int32_t i = 0; i < I; ++i) {
        double a = 0.0;
        for (int32_t d = 0; d < D; ++d) a += at(&L->W_up, (int64_t)e * I + i, d) * u[d];
        r[i] = a > 0.0 ? a : 0.0;
      }
      dg[j] = 0.0;
      for (int32_t d = 0; d < D; ++d) {
        double a = 0.0;
        for (int32_t i = 0; i < I; ++i) a += at(&L->W_down, (int64_t)e * D + d, i) * (r[i] * r[i]);
        Y[d] = a;
        acc[d] += g[j] * a;
        dg[j] += ge[d] * a;
      }
      for (int32_t i = 0; i < I; ++i) {
        double a = 0.0;
        for (int32_t d = 0; d < D; ++d) a += at(&L->W_down, (int64_t)e * D + d, i) * (g[j] * ge[d]);
        dh[i] = 2.0 * r[i] * a; /* da */
      }
      for (int32_t d = 0; d < D; ++d) {
        double a = 0.0;
        for (int32_t i = 0; i < I; ++i) a += at(&L->W_up, (int64_t)e * I + i, d) * dh[i];
        gu[d] += a;
      }
      if (want_w && G->dW_down)
        for (int32_t d = 0; d < D; ++d)
          for (int32_t i = 0; i < I; ++i)
            G->dW_down[(ew * D + d) * I + i] += g[j] * ge[d] * (r[i] * r[i]);
      if (want_w && G->dW_up)
        for (int32_t i = 0; i < I; ++i)
          for (int32_t d = 0; d < D; ++d)
            G->dW_up[(ew * I + i) * D + d] += dh[i] * u[d];
    }
    /* back to x: directly, or through the latent projections */
    if (Lw) {
      for (int32_t c = 0; c < H; ++c) {
        double a = 0.0;
        for (int32_t d = 0; d < D; ++d) a += at(&L->W_in, d, c) * gu[d];
        gx[c] += a;
      }
      if (G && G->dW_in)
        for (int32_t d = 0; d < D; ++d)
          for (int32_t c = 0; c < H; ++c) G->dW_in[(int64_t)d * H + c] += gu[d] * at(&L->x, t, c);
      if (G && G->dW_out)
        for (int32_t c = 0; c < H; ++c)
          for (int32_t d = 0; d < D; ++d) G->dW_out[(int64_t)c * D + d] += dyt[c] * acc[d];
    } else {
      for (int32_t c = 0; c < H; ++c) gx[c] += gu[c];
    }
    /* router: through the renormalised gates and the sigmoid */
    double gdg = 0.0;
    for (int32_t j = 0; j < k; ++j) gdg += g[j] * dg[j];
    if (dz)
      for (int32_t e = 0; e < E; ++e) dz[(int64_t)a * E + e] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const double dzj = (dg[j] - gdg) / Z * s[j] * (1.0 - s[j]);
      if (dz) dz[(int64_t)a * E + it[j]] = dzj;
      for (int32_t c = 0; c < H; ++c) gx[c] += dzj * at(&L->W_r, it[j], c);
      if (G && G->dW_r)
        for (int32_t c = 0; c < H; ++c) G->dW_r[(int64_t)it[j] * H + c] += dzj * at(&L->x, t, c);
    }
    /* shared expert */
    if (Is) {
      for (int32_t i = 0; i < Is; ++i) {
        double acc = 0.0;
        for (int32_t c = 0; c < H; ++c) acc += at(&L->Ws_up, i, c) * at(&L->x, t, c);
        r[i] = acc > 0.0 ? acc : 0.0;
        double d = 0.0;
        for (int32_t c = 0; c < H; ++c) d += at(&L->Ws_down, c, i) * dyt[c];
        dh[i] = 2.0 * r[i] * d; /* da_s */
      }
      for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t i = 0; i < Is; ++i) acc += at(&L->Ws_up, i, c) * dh[i];
        gx[c] += acc;
      }
      if (G && G->dWs_down)
        for (int32_t c = 0; c < H; ++c)
          for (int32_t i = 0; i < Is; ++i) G->dWs_down[(int64_t)c * Is + i] += dyt[c] * (r[i] * r[i]);
      if (G && G->dWs_up)
        for (int32_t i = 0; i < Is; ++i)
          for (int32_t c = 0; c < H; ++c) G->dWs_up[(int64_t)i * H + c] += dh[i] * at(&L->x, t, c);
    }
    if (dx)
      for (int32_t c = 0; c < H; ++c) dx[(int64_t)a * H + c] = gx[c];
  }
done:
  free(r); free(dh); free(Y); free(gx); free(u); free(ge); free(gu); free(acc);
  return rc;
}
