/* CPU oracle of one transformer decode step (test infrastructure only).
 *
 * This file is the plain, slow, obviously-correct definition that the HIP
 * library is checked against.  Only the test suite, the package's smoke check
 * and the benchmark's CPU-baseline leg load it; the library never does.  It
 * shares no code with the library.
 *
 * What it computes follows the operator chain that the CMU 15-779 lecture 7
 * notes list for Llama-family decode (section 2, "the cost of small-batch
 * decoding": RMSNorm, QKV, attention, output projection, RMSNorm, gate/up,
 * down, final RMSNorm and LM head; section 5.1 lists the same chain as the
 * HazyResearch megakernel's seven fused instruction types, with RoPE fused
 * after QKV), and the MegaRTP article, section 1 (RMSNorm, GEMMs, RoPE,
 * KV-cache write).  Where the pages leave a step open the plainest reading is
 * taken:
 *   - RMSNorm: y_i = x_i / sqrt(mean(x^2) + eps) * w_i.
 *   - RoPE: rotate-half pairs (i, i + d/2), angle = pos * theta^(-2i/d).
 *   - The new token's K (after RoPE) and V are rounded to bf16 (RNE), stored at
 *     row kv_len[b] of the cache and then attended together with the kv_len[b]
 *     prior rows (write, then read).  ``round_new_kv = 0`` attends to the
 *     unrounded values instead (the cache still receives the bf16 row); that
 *     variant exists so the oracle can be compared with a library model.
 *   - Attention: softmax(q.K^T / sqrt(d)) V over positions 0..kv_len[b],
 *     query head h uses kv head h / (n_q / n_kv).
 *   - Qwen3 shape: per-head RMSNorm of q and k (same eps) before RoPE.
 *   - FFN: (silu(y Wg^T) * (y Wu^T)) Wd^T, silu(z) = z / (1 + exp(-z)).
 *   - Logits from the final-RMSNorm'd state times the LM head (the embedding
 *     when tied); next token = argmax, lowest index on ties.
 * Arithmetic is in ``real`` (double unless built with -DORACLE_REAL=float),
 * sums run in natural index order, bf16 inputs are widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_REAL
#define ORACLE_REAL double
#endif
typedef ORACLE_REAL real;

#define SLOT_ATTN_NORM 0
#define SLOT_WQ 1
#define SLOT_WK 2
#define SLOT_WV 3
#define SLOT_Q_NORM 4
#define SLOT_K_NORM 5
#define SLOT_WO 6
#define SLOT_FFN_NORM 7
#define SLOT_W_GATE 8
#define SLOT_W_UP 9
#define SLOT_W_DOWN 10
#define N_SLOTS 11

typedef struct {
  int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int tied, qk_norm;
  int kv_capacity;   /* rows per (layer, K|V, seq, kv head) in the cache */
  double rms_eps, rope_theta;
  int round_new_kv;  /* 1: attend the bf16-rounded new row (default reading) */
} oracle_model;

int oracle_real_bytes(void) { return (int)sizeof(real); }

/* ---- bf16 <-> real ---------------------------------------------------- */
static real from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (real)f;
}

/* Round a real number to the nearest bf16 (ties to even), one rounding. */
uint16_t oracle_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  double a = fabs(v);
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  if (a < 0x1.0p-126) {                 /* subnormal range: spacing 2^-133 */
    double q = nearbyint(a * 0x1.0p133);  /* default mode: ties to even */
    return (uint16_t)(sign | (uint16_t)q); /* q <= 128 carries into the exponent field */
  }
  int e;
  double m = frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) */
  double q = nearbyint(m * 256.0);      /* 8 significant bits */
  double r = ldexp(q, e - 8);
  if (r >= 0x1.0p128) return (uint16_t)(sign | 0x7F80); /* rounds past the largest bf16 */
  float f = (float)r;                   /* exact: 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* ---- per-op definitions (exported for the pin tests) --------------------- */

/* y = x / sqrt(mean(x^2) + eps) * w */
void oracle_rmsnorm(int n, const real* x, const uint16_t* w, double eps, real* y) {
  real ss = 0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  real inv = (real)1 / sqrt(ss / (real)n + (real)eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * inv * from_bf16(w[i]);
}

/* out[r] = sum_c W[r][c] * x[c], W bf16 row-major [rows][cols] */
void oracle_matvec(int rows, int cols, const uint16_t* W, const real* x, real* out) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint16_t* wr = W + (size_t)r * cols;
    real acc = 0;
    for (int c = 0; c < cols; ++c) acc += from_bf16(wr[c]) * x[c];
    out[r] = acc;
  }
}

/* Rotate-half RoPE of one head vector v[d] at position pos. */
void oracle_rope(int d, int pos, double theta, real* v) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
    real c = (real)cos(ang), s = (real)sin(ang);
    real a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

real oracle_silu(real z) { return z / ((real)1 + exp(-z)); }

/* Single-query attention over n cache rows K[j], V[j] (bf16, row stride d),
 * except that row ``special`` (if >= 0) is taken from knew/vnew (real). */
void oracle_attend(int d, int n, const real* q, const uint16_t* K, const uint16_t* Vc, int special,
                   const real* knew, const real* vnew, real* out) {
  real* s = (real*)malloc(sizeof(real) * (size_t)(n > 0 ? n : 1));
  real scale = (real)1 / sqrt((real)d);
  real m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    real acc = 0;
    for (int i = 0; i < d; ++i)
      acc += q[i] * (j == special ? knew[i] : from_bf16(K[(size_t)j * d + i]));
    s[j] = acc * scale;
    if (s[j] > m) m = s[j];
  }
  real z = 0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - m);
    z += s[j];
  }
  for (int i = 0; i < d; ++i) out[i] = 0;
  for (int j = 0; j < n; ++j)
    for (int i = 0; i < d; ++i)
      out[i] += s[j] * (j == special ? vnew[i] : from_bf16(Vc[(size_t)j * d + i]));
  for (int i = 0; i < d; ++i) out[i] /= z;
  free(s);
}

int oracle_argmax(int n, const real* v) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* ---- the decode step ------------------------------------------------------
 * weights: pointer table, layer l slot s at [l * N_SLOTS + s] (NULL for q/k
 * norm without qk_norm), then embed, final_norm, lm_head at
 * [n_layers * N_SLOTS + 0/1/2] (lm_head may be NULL when tied).
 * kv_cache: bf16 [L][2][B][n_kv][kv_capacity][head_dim]; row kv_len[b] of
 * every (layer, K|V, b, head) is written.  logits: [B][vocab].
 * Optional intermediates (NULL to skip): hidden_out [L][2][B][hidden], the
 * residual stream after each layer's attention block and after its FFN block;
 * qkv_out [L][B][(n_q + 2 n_kv) head_dim], each layer's q, k, v projections
 * (q heads, then k heads, then v heads) before the q/k norm and RoPE.
 * Returns 0, or -1 on an invalid argument. */
int oracle_decode_step_ex(const oracle_model* m, const uint16_t* const* weights, int batch,
                          const int32_t* kv_len, const int32_t* tokens, uint16_t* kv_cache,
                          real* logits, int32_t* next_tokens, real* hidden_out, real* qkv_out) {
  const int H = m->hidden, nq = m->n_q_heads, nkv = m->n_kv_heads, d = m->head_dim, F = m->ffn;
  const int V = m->vocab, L = m->n_layers, cap = m->kv_capacity;
  if (nkv <= 0 || nq % nkv || d % 2 || batch <= 0) return -1;
  for (int b = 0; b < batch; ++b)
    if (kv_len[b] < 0 || kv_len[b] >= cap || tokens[b] < 0 || tokens[b] >= V) return -1;
  const int hpg = nq / nkv;
  const uint16_t* embed = weights[L * N_SLOTS + 0];
  const uint16_t* final_norm = weights[L * N_SLOTS + 1];
  const uint16_t* lm = m->tied ? embed : weights[L * N_SLOTS + 2];
  if (!lm) return -1;

  real* x = (real*)malloc(sizeof(real) * H);
  real* y = (real*)malloc(sizeof(real) * H);
  real* q = (real*)malloc(sizeof(real) * nq * d);
  real* k = (real*)malloc(sizeof(real) * nkv * d);
  real* v = (real*)malloc(sizeof(real) * nkv * d);
  real* kr = (real*)malloc(sizeof(real) * nkv * d);
  real* vr = (real*)malloc(sizeof(real) * nkv * d);
  real* o = (real*)malloc(sizeof(real) * nq * d);
  real* t = (real*)malloc(sizeof(real) * (H > nq * d ? H : nq * d));
  real* g = (real*)malloc(sizeof(real) * F);
  real* u = (real*)malloc(sizeof(real) * F);

  for (int b = 0; b < batch; ++b) {
    const int pos = kv_len[b];
    for (int i = 0; i < H; ++i) x[i] = from_bf16(embed[(size_t)tokens[b] * H + i]);
    for (int l = 0; l < L; ++l) {
      const uint16_t* const* W = weights + (size_t)l * N_SLOTS;
      /* attention block */
      oracle_rmsnorm(H, x, W[SLOT_ATTN_NORM], m->rms_eps, y);
      oracle_matvec(nq * d, H, W[SLOT_WQ], y, q);
      oracle_matvec(nkv * d, H, W[SLOT_WK], y, k);
      oracle_matvec(nkv * d, H, W[SLOT_WV], y, v);
      if (qkv_out) {
        real* dst = qkv_out + ((size_t)l * batch + b) * (size_t)(nq + 2 * nkv) * d;
        memcpy(dst, q, sizeof(real) * nq * d);
        memcpy(dst + (size_t)nq * d, k, sizeof(real) * nkv * d);
        memcpy(dst + (size_t)(nq + nkv) * d, v, sizeof(real) * nkv * d);
      }
      if (m->qk_norm) {
        for (int h = 0; h < nq; ++h) {
          oracle_rmsnorm(d, q + h * d, W[SLOT_Q_NORM], m->rms_eps, t);
          memcpy(q + h * d, t, sizeof(real) * d);
        }
        for (int h = 0; h < nkv; ++h) {
          oracle_rmsnorm(d, k + h * d, W[SLOT_K_NORM], m->rms_eps, t);
          memcpy(k + h * d, t, sizeof(real) * d);
        }
      }
      for (int h = 0; h < nq; ++h) oracle_rope(d, pos, m->rope_theta, q + h * d);
      for (int h = 0; h < nkv; ++h) oracle_rope(d, pos, m->rope_theta, k + h * d);
      for (int h = 0; h < nkv; ++h) {
        uint16_t* Kc = kv_cache + ((((size_t)l * 2 + 0) * batch + b) * nkv + h) * (size_t)cap * d;
        uint16_t* Vc = kv_cache + ((((size_t)l * 2 + 1) * batch + b) * nkv + h) * (size_t)cap * d;
        for (int i = 0; i < d; ++i) {
          Kc[(size_t)pos * d + i] = oracle_to_bf16((double)k[h * d + i]);
          Vc[(size_t)pos * d + i] = oracle_to_bf16((double)v[h * d + i]);
          kr[h * d + i] = m->round_new_kv ? from_bf16(Kc[(size_t)pos * d + i]) : k[h * d + i];
          vr[h * d + i] = m->round_new_kv ? from_bf16(Vc[(size_t)pos * d + i]) : v[h * d + i];
        }
      }
      for (int h = 0; h < nq; ++h) {
        int kvh = h / hpg;
        const uint16_t* Kc = kv_cache + ((((size_t)l * 2 + 0) * batch + b) * nkv + kvh) * (size_t)cap * d;
        const uint16_t* Vc = kv_cache + ((((size_t)l * 2 + 1) * batch + b) * nkv + kvh) * (size_t)cap * d;
        oracle_attend(d, pos + 1, q + h * d, Kc, Vc, pos, kr + kvh * d, vr + kvh * d, o + h * d);
      }
      oracle_matvec(H, nq * d, W[SLOT_WO], o, t);
      for (int i = 0; i < H; ++i) x[i] += t[i];
      if (hidden_out) memcpy(hidden_out + (((size_t)l * 2 + 0) * batch + b) * H, x, sizeof(real) * H);
      /* feed-forward block */
      oracle_rmsnorm(H, x, W[SLOT_FFN_NORM], m->rms_eps, y);
      oracle_matvec(F, H, W[SLOT_W_GATE], y, g);
      oracle_matvec(F, H, W[SLOT_W_UP], y, u);
      for (int i = 0; i < F; ++i) g[i] = oracle_silu(g[i]) * u[i];
      oracle_matvec(H, F, W[SLOT_W_DOWN], g, t);
      for (int i = 0; i < H; ++i) x[i] += t[i];
      if (hidden_out) memcpy(hidden_out + (((size_t)l * 2 + 1) * batch + b) * H, x, sizeof(real) * H);
    }
    oracle_rmsnorm(H, x, final_norm, m->rms_eps, y);
    oracle_matvec(V, H, lm, y, logits + (size_t)b * V);
    next_tokens[b] = oracle_argmax(V, logits + (size_t)b * V);
  }
  free(x); free(y); free(q); free(k); free(v); free(kr); free(vr); free(o); free(t); free(g); free(u);
  return 0;
}

int oracle_decode_step(const oracle_model* m, const uint16_t* const* weights, int batch,
                       const int32_t* kv_len, const int32_t* tokens, uint16_t* kv_cache,
                       real* logits, int32_t* next_tokens) {
  return oracle_decode_step_ex(m, weights, batch, kv_len, tokens, kv_cache, logits, next_tokens, NULL, NULL);
}
