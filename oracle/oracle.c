/*
 * CPU oracle of the Dual-AR per-frame decode step.  TEST INFRASTRUCTURE ONLY:
 * see oracle.h for who may use it, its precision rules and its pins.
 *
 * What it computes, and where each step comes from:
 *  - Dual-AR frame: a Slow AR along time predicts the semantic code, then a
 *    4-layer Fast AR fills the 9 residual codes in 9 greedy steps, conditioned
 *    on the Slow hidden state ("SGLang Day-0 Support for FishAudio S2",
 *    Architecture, Stage 2; "s2pro-native", What happens to a sentence;
 *    "Fish Audio Abre Codigo do S2", Arquitetura Dual-AR).
 *  - VQ injection: at a masked position the input embedding is the sum of the
 *    ten codebook embeddings of that frame (S2 page, Architecture, Stage 2).
 *  - Constrained decoding of the semantic code: the Slow argmax runs over the
 *    semantic-code ids only (S2 page, Background and Motivation).
 *  - Layers are Qwen3-style: RMSNorm, GQA with per-head q/k RMSNorm and
 *    rotate-half RoPE, SwiGLU MLP; the RoPE table is rounded to bf16 (S2 page,
 *    Engineering Appendix).
 * Readings where the pages are silent (which hidden feeds the Fast AR, which
 * embedding table a Fast input uses, norm placement, epsilon, GQA grouping)
 * are stated at the function that takes them.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ weights */

typedef struct {
  const void* p;
  int bf16;
} wt;

static inline double wget(wt w, int64_t i) {
  if (w.bf16) {
    union { uint32_t u; float f; } v;
    v.u = ((uint32_t)((const uint16_t*)w.p)[i]) << 16;
    return (double)v.f;
  }
  return (double)((const float*)w.p)[i];
}

typedef struct {
  wt attn_norm, wq, wk, wv, q_norm, k_norm, wo, mlp_norm, w_gate, w_up, w_down;
} layer_w;

struct orc_model {
  orc_config c;
  wt embed, slow_final, slow_head, codebook, fast_final, fast_head;
  layer_w* slow;
  layer_w* fast;
  double* rope_cos_slow; /* [max_context][D/2] */
  double* rope_sin_slow;
  double* rope_cos_fast; /* [n_codebooks-1][D/2] */
  double* rope_sin_fast;
};

struct orc_state {
  int32_t pos;
  double* k_cache; /* [slow layers][max_context][Hkv*D] */
  double* v_cache;
};

static int64_t g_counters[4];

void orc_get_counters(int64_t* out4) { memcpy(out4, g_counters, sizeof(g_counters)); }
void orc_reset_counters(void) { memset(g_counters, 0, sizeof(g_counters)); }
void orc_set_threads(int32_t n) {
#ifdef _OPENMP
  omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t orc_n_tensors(const orc_config* c) {
  return 1 + 11 * c->slow.n_layers + 3 + 11 * c->fast.n_layers + 2;
}

/* --------------------------------------------------------------- primitives */

double orc_bf16_round(double v) {
  union { float f; uint32_t u; } x;
  x.f = (float)v;
  uint32_t lsb = (x.u >> 16) & 1u;
  x.u = (x.u + 0x7fffu + lsb) & 0xffff0000u;
  return (double)x.f;
}

static float bf16_bits_f32(uint16_t b) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)b << 16;
  return x.f;
}

void orc_quantize_rows_i8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float m = 0.0f;
    for (int64_t k = 0; k < cols; ++k) {
      const float a = fabsf(bf16_bits_f32(w[r * cols + k]));
      if (a > m) m = a;
    }
    const float sc = m / 127.0f;
    s[r] = sc;
    for (int64_t k = 0; k < cols; ++k) {
      float v = sc > 0.0f ? rintf(bf16_bits_f32(w[r * cols + k]) / sc) : 0.0f;
      if (v > 127.0f) v = 127.0f;
      if (v < -127.0f) v = -127.0f;
      q[r * cols + k] = (int8_t)v;
    }
  }
}

void orc_dequantize_rows_i8(const int8_t* q, const float* s, int64_t rows, int64_t cols, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < cols; ++k) out[r * cols + k] = (float)q[r * cols + k] * s[r];
}

/* Value of an OCP FP8 E4M3 ("e4m3fn") byte: sign in bit 7, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN (never produced here).
 * Normal values are (8 + m) * 2^(e - 10). */
double orc_f8_value(uint8_t b) {
  const int e = (b >> 3) & 15, m = b & 7;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  if ((b & 0x7f) == 0x7f) v = NAN;
  return (b & 0x80) ? -v : v;
}

/* Nearest E4M3 magnitude code (0x00..0x7e) to an a in [0, 448]: the finite magnitudes increase with
 * the code, so a bisection of the table of their values finds the neighbours below and above a; a
 * tie between the two goes to the even code (even last mantissa bit). */
static uint8_t f8_nearest_code(const double* tab, double a) {
  int lo = 0, hi = 0x7e; /* invariant: tab[lo] <= a, and a <= tab[hi] once a <= 448 */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (tab[mid] <= a) lo = mid;
    else hi = mid;
  }
  const double dl = a - tab[lo], dh = tab[hi] - a;
  if (dl < dh) return (uint8_t)lo;
  if (dh < dl) return (uint8_t)hi;
  return (uint8_t)((lo & 1) == 0 ? lo : hi);
}

void orc_quantize_rows_f8(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* q, float* s) {
  double tab[0x7f]; /* every finite magnitude, indexed by its code */
  for (int c = 0; c < 0x7f; ++c) tab[c] = orc_f8_value((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float m = 0.0f;
    for (int64_t k = 0; k < cols; ++k) {
      const float a = fabsf(bf16_bits_f32(w[r * cols + k]));
      if (a > m) m = a;
    }
    const float sc = m / 448.0f;
    s[r] = sc;
    for (int64_t k = 0; k < cols; ++k) {
      float v = sc > 0.0f ? bf16_bits_f32(w[r * cols + k]) / sc : 0.0f;
      if (v > 448.0f) v = 448.0f;
      if (v < -448.0f) v = -448.0f;
      q[r * cols + k] = (uint8_t)(f8_nearest_code(tab, fabs((double)v)) | (v < 0.0f ? 0x80 : 0x00));
    }
  }
}

void orc_dequantize_rows_f8(const uint8_t* q, const float* s, int64_t rows, int64_t cols, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < cols; ++k) out[r * cols + k] = (float)orc_f8_value(q[r * cols + k]) * s[r];
}

/* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g  (epsilon inside the root). */
void orc_rmsnorm(const double* x, const double* g, int32_t n, double eps, double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = sqrt(ss / (double)n + eps);
  for (int32_t i = 0; i < n; ++i) y[i] = x[i] / r * g[i];
}

static void rmsnorm_w(const double* x, wt g, int64_t goff, int32_t n, double eps, double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = sqrt(ss / (double)n + eps);
  for (int32_t i = 0; i < n; ++i) y[i] = x[i] / r * wget(g, goff + i);
}

/* RoPE angles: inv_freq_i = theta^(-2i/D), angle = pos * inv_freq_i. */
void orc_rope_row(double theta, int32_t D, int32_t pos, int32_t bf16, double* c, double* s) {
  for (int32_t i = 0; i < D / 2; ++i) {
    double inv = pow(theta, -2.0 * (double)i / (double)D);
    double a = (double)pos * inv;
    c[i] = cos(a);
    s[i] = sin(a);
    if (bf16) {
      c[i] = orc_bf16_round(c[i]);
      s[i] = orc_bf16_round(s[i]);
    }
  }
}

/* Rotate-half RoPE: element i pairs with element i + D/2. */
void orc_rope_apply(double* v, int32_t D, const double* c, const double* s) {
  int32_t h = D / 2;
  for (int32_t i = 0; i < h; ++i) {
    double a = v[i], b = v[i + h];
    v[i] = a * c[i] - b * s[i];
    v[i + h] = b * c[i] + a * s[i];
  }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Greedy pick over [lo, hi): the largest value, ties to the lowest index.
 * margin = best minus the runner-up (0 on a tie). Returns the absolute index. */
int32_t orc_argmax(const double* v, int32_t lo, int32_t hi, double* margin) {
  int32_t best = lo;
  for (int32_t i = lo + 1; i < hi; ++i)
    if (v[i] > v[best]) best = i;
  if (margin) {
    double second = -INFINITY;
    for (int32_t i = lo; i < hi; ++i)
      if (i != best && v[i] > second) second = v[i];
    *margin = (hi - lo > 1) ? v[best] - second : INFINITY;
  }
  return best;
}

/* y[p][n] = sum_k w[n][k] * x[p][k], k ascending, one thread per row n. */
static void matvec(wt w, int64_t woff, int32_t N, int32_t K, const double* x, int32_t P, double* y) {
  if (P == 1) {
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n) {
      double acc = 0.0;
      int64_t base = woff + (int64_t)n * K;
      for (int32_t k = 0; k < K; ++k) acc += wget(w, base + k) * x[k];
      y[n] = acc;
    }
    return;
  }
  /* several vectors: the same per-element sums, with x transposed so that the
   * vectors can share each weight read */
  double* xt = (double*)malloc(sizeof(double) * (size_t)K * (size_t)P);
  for (int32_t p = 0; p < P; ++p)
    for (int32_t k = 0; k < K; ++k) xt[(size_t)k * P + p] = x[(size_t)p * K + k];
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)P);
#pragma omp for schedule(static)
    for (int32_t n = 0; n < N; ++n) {
      for (int32_t p = 0; p < P; ++p) acc[p] = 0.0;
      int64_t base = woff + (int64_t)n * K;
      for (int32_t k = 0; k < K; ++k) {
        double wv = wget(w, base + k);
        const double* xr = xt + (size_t)k * P;
        for (int32_t p = 0; p < P; ++p) acc[p] += wv * xr[p];
      }
      for (int32_t p = 0; p < P; ++p) y[(size_t)p * N + n] = acc[p];
    }
    free(acc);
  }
  free(xt);
}

void orc_matvec_f32(const float* w, int32_t N, int32_t K, const double* x, int32_t P, double* y) {
  wt ww = {w, 0};
  matvec(ww, 0, N, K, x, P, y);
}

/* Scaled dot-product attention of one query position over ctx cached keys.
 * Query head h reads KV head floor(h / (Hq/Hkv)) (contiguous GQA groups).
 * Scores are q.k / sqrt(D); the softmax subtracts the row maximum and sums in
 * fp64.  k_cache/v_cache: [ctx][Hkv*D].  probs (optional): [Hq][ctx]. */
void orc_attention(const double* q, const double* kc, const double* vc, int32_t Hq, int32_t Hkv,
                   int32_t D, int32_t ctx, double* o, double* probs) {
  int32_t group = Hq / Hkv;
  double scale = 1.0 / sqrt((double)D);
  double* p = (double*)malloc(sizeof(double) * (size_t)ctx);
  for (int32_t h = 0; h < Hq; ++h) {
    int32_t g = h / group;
    const double* qh = q + (size_t)h * D;
    double mx = -INFINITY;
    for (int32_t j = 0; j < ctx; ++j) {
      const double* kj = kc + (size_t)j * Hkv * D + (size_t)g * D;
      double s = 0.0;
      for (int32_t d = 0; d < D; ++d) s += qh[d] * kj[d];
      p[j] = s * scale;
      if (p[j] > mx) mx = p[j];
    }
    double l = 0.0;
    for (int32_t j = 0; j < ctx; ++j) {
      p[j] = exp(p[j] - mx);
      l += p[j];
    }
    for (int32_t j = 0; j < ctx; ++j) p[j] /= l;
    double* oh = o + (size_t)h * D;
    for (int32_t d = 0; d < D; ++d) oh[d] = 0.0;
    for (int32_t j = 0; j < ctx; ++j) {
      const double* vj = vc + (size_t)j * Hkv * D + (size_t)g * D;
      for (int32_t d = 0; d < D; ++d) oh[d] += p[j] * vj[d];
    }
    if (probs) memcpy(probs + (size_t)h * ctx, p, sizeof(double) * (size_t)ctx);
  }
  free(p);
}

/* ------------------------------------------------------------------- model */

static void gains_to_f64(wt g, int32_t n, double* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = wget(g, i);
}

orc_model* orc_model_new(const orc_config* cfg, const void* const* t, int32_t n_tensors) {
  if (n_tensors != orc_n_tensors(cfg)) return NULL;
  if (cfg->slow.hidden != cfg->fast.hidden) return NULL; /* h feeds the Fast AR unprojected */
  if (cfg->eos_id < -1 || cfg->eos_id >= cfg->vocab_text) return NULL; /* a text id, or none */
  if (cfg->slow.n_q_heads % cfg->slow.n_kv_heads || cfg->fast.n_q_heads % cfg->fast.n_kv_heads) return NULL;
  if (cfg->slow.head_dim % 2 || cfg->fast.head_dim % 2 || cfg->n_codebooks < 2) return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  m->c = *cfg;
  int bf = cfg->weight_dtype == 1;
  int i = 0;
#define NEXT() ((wt){t[i++], bf})
  m->embed = NEXT();
  m->slow = (layer_w*)calloc((size_t)cfg->slow.n_layers, sizeof(layer_w));
  m->fast = (layer_w*)calloc((size_t)cfg->fast.n_layers, sizeof(layer_w));
  for (int l = 0; l < cfg->slow.n_layers; ++l) {
    layer_w* L = &m->slow[l];
    L->attn_norm = NEXT(); L->wq = NEXT(); L->wk = NEXT(); L->wv = NEXT(); L->q_norm = NEXT();
    L->k_norm = NEXT(); L->wo = NEXT(); L->mlp_norm = NEXT(); L->w_gate = NEXT(); L->w_up = NEXT();
    L->w_down = NEXT();
  }
  m->slow_final = NEXT();
  m->slow_head = NEXT();
  m->codebook = NEXT();
  for (int l = 0; l < cfg->fast.n_layers; ++l) {
    layer_w* L = &m->fast[l];
    L->attn_norm = NEXT(); L->wq = NEXT(); L->wk = NEXT(); L->wv = NEXT(); L->q_norm = NEXT();
    L->k_norm = NEXT(); L->wo = NEXT(); L->mlp_norm = NEXT(); L->w_gate = NEXT(); L->w_up = NEXT();
    L->w_down = NEXT();
  }
  m->fast_final = NEXT();
  m->fast_head = NEXT();
#undef NEXT
  int32_t hs = cfg->slow.head_dim / 2, hf = cfg->fast.head_dim / 2;
  m->rope_cos_slow = (double*)malloc(sizeof(double) * (size_t)cfg->max_context * hs);
  m->rope_sin_slow = (double*)malloc(sizeof(double) * (size_t)cfg->max_context * hs);
  for (int32_t p = 0; p < cfg->max_context; ++p)
    orc_rope_row(cfg->rope_theta, cfg->slow.head_dim, p, cfg->rope_bf16, m->rope_cos_slow + (size_t)p * hs,
                 m->rope_sin_slow + (size_t)p * hs);
  int32_t nf = cfg->n_codebooks - 1;
  m->rope_cos_fast = (double*)malloc(sizeof(double) * (size_t)nf * hf);
  m->rope_sin_fast = (double*)malloc(sizeof(double) * (size_t)nf * hf);
  for (int32_t p = 0; p < nf; ++p)
    orc_rope_row(cfg->rope_theta, cfg->fast.head_dim, p, cfg->rope_bf16, m->rope_cos_fast + (size_t)p * hf,
                 m->rope_sin_fast + (size_t)p * hf);
  return m;
}

void orc_model_free(orc_model* m) {
  if (!m) return;
  free(m->slow); free(m->fast);
  free(m->rope_cos_slow); free(m->rope_sin_slow); free(m->rope_cos_fast); free(m->rope_sin_fast);
  free(m);
}

orc_state* orc_state_new(const orc_model* m) {
  orc_state* s = (orc_state*)calloc(1, sizeof(orc_state));
  size_t n = (size_t)m->c.slow.n_layers * m->c.max_context * m->c.slow.n_kv_heads * m->c.slow.head_dim;
  s->k_cache = (double*)calloc(n, sizeof(double));
  s->v_cache = (double*)calloc(n, sizeof(double));
  return s;
}

void orc_state_free(orc_state* s) {
  if (!s) return;
  free(s->k_cache); free(s->v_cache); free(s);
}

int32_t orc_state_pos(const orc_state* s) { return s->pos; }

/* Text position: row `token` of the Slow embedding (text ids and semantic ids
 * share one table of vocab_text + codebook_size rows). */
int orc_embed_token(const orc_model* m, int32_t token, double* x) {
  int32_t H = m->c.slow.hidden;
  if (token < 0 || token >= m->c.vocab_text + m->c.codebook_size) return -1;
  for (int32_t i = 0; i < H; ++i) x[i] = wget(m->embed, (int64_t)token * H + i);
  return 0;
}

/* VQ position: sum over codebooks k = 0..9 of E_cb[k][code_k] (replaces the
 * token embedding). */
int orc_embed_codes(const orc_model* m, const int32_t* codes, double* x) {
  int32_t H = m->c.slow.hidden, K = m->c.codebook_size;
  for (int32_t i = 0; i < H; ++i) x[i] = 0.0;
  for (int32_t k = 0; k < m->c.n_codebooks; ++k) {
    if (codes[k] < 0 || codes[k] >= K) return -1;
    int64_t base = ((int64_t)k * K + codes[k]) * H;
    for (int32_t i = 0; i < H; ++i) x[i] += wget(m->codebook, base + i);
  }
  return 0;
}

/* Run a stack of layers over n new positions pos0..pos0+n-1 whose inputs are
 * the rows of X ([n][H], updated in place).  Keys/values are appended to the
 * cache ([layers][cache_cap][Hkv*D]) at their positions; position i attends to
 * cache entries 0..pos0+i.  resid_tap (optional): [layers][n][H]. */
static void stack_forward(const orc_model* m, const orc_stack* s, const layer_w* lw, const double* rcos,
                          const double* rsin, double* X, int32_t n, int32_t pos0, double* kcache,
                          double* vcache, int32_t cache_cap, double* resid_tap) {
  int32_t H = s->hidden, Hq = s->n_q_heads, Hkv = s->n_kv_heads, D = s->head_dim, F = s->ffn;
  int32_t qd = Hq * D, kd = Hkv * D, hd = D / 2;
  double eps = m->c.rms_eps;
  double* xn = (double*)malloc(sizeof(double) * (size_t)n * H);
  double* q = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* k = (double*)malloc(sizeof(double) * (size_t)n * kd);
  double* v = (double*)malloc(sizeof(double) * (size_t)n * kd);
  double* o = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* t = (double*)malloc(sizeof(double) * (size_t)n * (F > qd ? F : qd));
  double* g = (double*)malloc(sizeof(double) * (size_t)n * F);
  double* u = (double*)malloc(sizeof(double) * (size_t)n * F);
  double* gq = (double*)malloc(sizeof(double) * (size_t)D);
  double* gk = (double*)malloc(sizeof(double) * (size_t)D);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  for (int32_t l = 0; l < s->n_layers; ++l) {
    const layer_w* L = &lw[l];
    double* kc = kcache + (size_t)l * cache_cap * kd;
    double* vc = vcache + (size_t)l * cache_cap * kd;
    /* attention block */
    for (int32_t i = 0; i < n; ++i) rmsnorm_w(X + (size_t)i * H, L->attn_norm, 0, H, eps, xn + (size_t)i * H);
    matvec(L->wq, 0, qd, H, xn, n, q);
    matvec(L->wk, 0, kd, H, xn, n, k);
    matvec(L->wv, 0, kd, H, xn, n, v);
    gains_to_f64(L->q_norm, D, gq);
    gains_to_f64(L->k_norm, D, gk);
    for (int32_t i = 0; i < n; ++i) {
      int32_t pos = pos0 + i;
      const double* c = rcos + (size_t)pos * hd;
      const double* sn = rsin + (size_t)pos * hd;
      for (int32_t h = 0; h < Hq; ++h) { /* per-head q RMSNorm, then RoPE */
        double* qh = q + (size_t)i * qd + (size_t)h * D;
        orc_rmsnorm(qh, gq, D, eps, tmp);
        memcpy(qh, tmp, sizeof(double) * D);
        orc_rope_apply(qh, D, c, sn);
      }
      for (int32_t h = 0; h < Hkv; ++h) {
        double* kh = k + (size_t)i * kd + (size_t)h * D;
        orc_rmsnorm(kh, gk, D, eps, tmp);
        memcpy(kh, tmp, sizeof(double) * D);
        orc_rope_apply(kh, D, c, sn);
      }
      memcpy(kc + (size_t)pos * kd, k + (size_t)i * kd, sizeof(double) * kd);
      memcpy(vc + (size_t)pos * kd, v + (size_t)i * kd, sizeof(double) * kd);
    }
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < n; ++i)
      orc_attention(q + (size_t)i * qd, kc, vc, Hq, Hkv, D, pos0 + i + 1, o + (size_t)i * qd, NULL);
    matvec(L->wo, 0, H, qd, o, n, t);
    for (size_t e = 0; e < (size_t)n * H; ++e) X[e] += t[e];
    /* SwiGLU MLP block */
    for (int32_t i = 0; i < n; ++i) rmsnorm_w(X + (size_t)i * H, L->mlp_norm, 0, H, eps, xn + (size_t)i * H);
    matvec(L->w_gate, 0, F, H, xn, n, g);
    matvec(L->w_up, 0, F, H, xn, n, u);
    for (size_t e = 0; e < (size_t)n * F; ++e) g[e] = orc_silu(g[e]) * u[e];
    matvec(L->w_down, 0, H, F, g, n, t);
    for (size_t e = 0; e < (size_t)n * H; ++e) X[e] += t[e];
    if (resid_tap) memcpy(resid_tap + (size_t)l * n * H, X, sizeof(double) * (size_t)n * H);
  }
  free(xn); free(q); free(k); free(v); free(o); free(t); free(g); free(u); free(gq); free(gk); free(tmp);
}

int32_t orc_slow_pick(const double* logits, int32_t vocab_text, int32_t codebook_size, int32_t eos_id,
                      double* margin) {
  /* candidate ids in increasing order: the EOS id (if any), then the semantic ids */
  const int32_t n = codebook_size + (eos_id >= 0 ? 1 : 0);
  int32_t best = -2;
  double bv = -INFINITY, second = -INFINITY;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = eos_id >= 0 ? (i == 0 ? eos_id : vocab_text + i - 1) : vocab_text + i;
    const double v = logits[id];
    if (best == -2 || v > bv) {
      if (best != -2) second = bv;
      best = id;
      bv = v;
    } else if (v > second) {
      second = v;
    }
  }
  if (margin) *margin = n > 1 ? bv - second : INFINITY;
  return best == eos_id ? -1 : best - vocab_text;
}

/* Final norm and Slow head on the residual x, then the Slow pick (semantic ids, plus the EOS id
 * when the model has one). */
static void slow_head(const orc_model* m, const double* x, double* h, double* logits, int32_t* c0,
                      double* margin) {
  int32_t H = m->c.slow.hidden, V = m->c.vocab_text + m->c.codebook_size;
  rmsnorm_w(x, m->slow_final, 0, H, m->c.rms_eps, h);
  matvec(m->slow_head, 0, V, H, h, 1, logits);
  *c0 = orc_slow_pick(logits, m->c.vocab_text, m->c.codebook_size, m->c.eos_id, margin);
}

int orc_prefill(const orc_model* m, orc_state* st, const int32_t* tokens, const uint8_t* mask,
                const int32_t* codes, int32_t n, double* h_out, double* logits_out, int32_t* c0_out,
                double* margin_out) {
  int32_t H = m->c.slow.hidden, V = m->c.vocab_text + m->c.codebook_size;
  if (n < 1 || st->pos + n > m->c.max_context) return -1;
  double* X = (double*)malloc(sizeof(double) * (size_t)n * H);
  for (int32_t i = 0; i < n; ++i) {
    int rc = (mask && mask[i]) ? orc_embed_codes(m, codes + (size_t)i * m->c.n_codebooks, X + (size_t)i * H)
                               : orc_embed_token(m, tokens[i], X + (size_t)i * H);
    if (rc) { free(X); return -2; }
  }
  stack_forward(m, &m->c.slow, m->slow, m->rope_cos_slow, m->rope_sin_slow, X, n, st->pos, st->k_cache,
                st->v_cache, m->c.max_context, NULL);
  st->pos += n;
  g_counters[0] += n;
  double* h = (double*)malloc(sizeof(double) * H);
  double* lg = (double*)malloc(sizeof(double) * V);
  int32_t c0;
  double mg;
  slow_head(m, X + (size_t)(n - 1) * H, h, lg, &c0, &mg);
  if (h_out) memcpy(h_out, h, sizeof(double) * H);
  if (logits_out) memcpy(logits_out, lg, sizeof(double) * V);
  if (c0_out) *c0_out = c0;
  if (margin_out) *margin_out = mg;
  free(h); free(lg); free(X);
  return 0;
}

int orc_slow_step_codes(const orc_model* m, orc_state* st, const int32_t* codes, double* resid_tap,
                        double* h_out, double* logits_out, int32_t* c0_out, double* margin_out) {
  int32_t H = m->c.slow.hidden, V = m->c.vocab_text + m->c.codebook_size;
  if (st->pos + 1 > m->c.max_context) return -1;
  double* x = (double*)malloc(sizeof(double) * H);
  if (orc_embed_codes(m, codes, x)) { free(x); return -2; }
  stack_forward(m, &m->c.slow, m->slow, m->rope_cos_slow, m->rope_sin_slow, x, 1, st->pos, st->k_cache,
                st->v_cache, m->c.max_context, resid_tap);
  st->pos += 1;
  g_counters[0] += 1;
  double* h = (double*)malloc(sizeof(double) * H);
  double* lg = (double*)malloc(sizeof(double) * V);
  int32_t c0;
  double mg;
  slow_head(m, x, h, lg, &c0, &mg);
  if (h_out) memcpy(h_out, h, sizeof(double) * H);
  if (logits_out) memcpy(logits_out, lg, sizeof(double) * V);
  if (c0_out) *c0_out = c0;
  if (margin_out) *margin_out = mg;
  free(h); free(lg); free(x);
  return 0;
}

/* Fast AR loop.  Readings: its first input is the Slow hidden after the final
 * RMSNorm (the vector the Slow head sees), fed without projection; the input of
 * step j >= 2 is codebook table j-1's row for code c_{j-1} (no separate Fast
 * embedding); the semantic code c0 is not fed; one head [K][H] serves all nine
 * steps; the cache is fresh per frame, at Fast positions 0..8. */
int orc_fast_loop(const orc_model* m, const double* h, const int32_t* forced, int32_t* codes_out,
                  double* margins, double* resid_tap, double* z_tap, double* logits_tap) {
  const orc_stack* s = &m->c.fast;
  int32_t H = s->hidden, K = m->c.codebook_size, nsteps = m->c.n_codebooks - 1;
  int32_t kd = s->n_kv_heads * s->head_dim;
  if (forced)
    for (int32_t j = 0; j < nsteps; ++j)
      if (forced[j] < 0 || forced[j] >= K) return -2;
  double* kc = (double*)calloc((size_t)s->n_layers * nsteps * kd, sizeof(double));
  double* vc = (double*)calloc((size_t)s->n_layers * nsteps * kd, sizeof(double));
  double* x = (double*)malloc(sizeof(double) * H);
  double* z = (double*)malloc(sizeof(double) * H);
  double* fl = (double*)malloc(sizeof(double) * K);
  double* rt = resid_tap ? (double*)malloc(sizeof(double) * (size_t)s->n_layers * H) : NULL;
  int32_t in_code = -1;
  for (int32_t j = 1; j <= nsteps; ++j) {
    if (j == 1) {
      memcpy(x, h, sizeof(double) * H);
    } else {
      int64_t base = ((int64_t)(j - 1) * K + in_code) * H;
      for (int32_t i = 0; i < H; ++i) x[i] = wget(m->codebook, base + i);
    }
    stack_forward(m, s, m->fast, m->rope_cos_fast, m->rope_sin_fast, x, 1, j - 1, kc, vc, nsteps, rt);
    g_counters[1] += 1;
    g_counters[2] += s->n_layers;
    rmsnorm_w(x, m->fast_final, 0, H, m->c.rms_eps, z);
    matvec(m->fast_head, 0, K, H, z, 1, fl);
    double mg;
    int32_t c = orc_argmax(fl, 0, K, &mg);
    codes_out[j - 1] = c;
    if (margins) margins[j - 1] = mg;
    if (resid_tap) memcpy(resid_tap + (size_t)(j - 1) * s->n_layers * H, rt, sizeof(double) * (size_t)s->n_layers * H);
    if (z_tap) memcpy(z_tap + (size_t)(j - 1) * H, z, sizeof(double) * H);
    if (logits_tap) memcpy(logits_tap + (size_t)(j - 1) * K, fl, sizeof(double) * K);
    in_code = forced ? forced[j - 1] : c;
  }
  free(kc); free(vc); free(x); free(z); free(fl); free(rt);
  return 0;
}

int orc_generate(const orc_model* m, orc_state* st, const double* h0, int32_t c0, int32_t n_frames,
                 int32_t* codes_out) {
  int32_t H = m->c.slow.hidden, NC = m->c.n_codebooks;
  double* h = (double*)malloc(sizeof(double) * H);
  memcpy(h, h0, sizeof(double) * H);
  int rc = 0;
  for (int32_t t = 0; t < n_frames; ++t) {
    int32_t* fr = codes_out + (size_t)t * NC;
    if (t > 0) {
      rc = orc_slow_step_codes(m, st, codes_out + (size_t)(t - 1) * NC, NULL, h, NULL, &c0, NULL);
      if (rc) break;
    }
    if (c0 < 0) { /* EOS: the stream has ended */
      for (size_t e = (size_t)t * NC; e < (size_t)n_frames * NC; ++e) codes_out[e] = -1;
      break;
    }
    fr[0] = c0;
    orc_fast_loop(m, h, NULL, fr + 1, NULL, NULL, NULL, NULL);
    g_counters[3] += NC;
  }
  free(h);
  return rc;
}

/* Matrix form with no cache: for every layer the n x n score matrix of each
 * head is formed in full and positions j > i are masked out before the
 * softmax. */
int orc_full_recompute(const orc_model* m, const int32_t* tokens, const uint8_t* mask, const int32_t* codes,
                       int32_t n, double* h_out) {
  const orc_stack* s = &m->c.slow;
  int32_t H = s->hidden, Hq = s->n_q_heads, Hkv = s->n_kv_heads, D = s->head_dim, F = s->ffn;
  int32_t qd = Hq * D, kd = Hkv * D, hd = D / 2, group = Hq / Hkv;
  double eps = m->c.rms_eps, scale = 1.0 / sqrt((double)D);
  if (n < 1 || n > m->c.max_context || D > 1024) return -1;
  double* X = (double*)malloc(sizeof(double) * (size_t)n * H);
  for (int32_t i = 0; i < n; ++i) {
    int rc = (mask && mask[i]) ? orc_embed_codes(m, codes + (size_t)i * m->c.n_codebooks, X + (size_t)i * H)
                               : orc_embed_token(m, tokens[i], X + (size_t)i * H);
    if (rc) { free(X); return -2; }
  }
  double* xn = (double*)malloc(sizeof(double) * (size_t)n * H);
  double* Q = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* Kx = (double*)malloc(sizeof(double) * (size_t)n * kd);
  double* Vx = (double*)malloc(sizeof(double) * (size_t)n * kd);
  double* O = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* T = (double*)malloc(sizeof(double) * (size_t)n * (F > qd ? F : qd));
  double* G = (double*)malloc(sizeof(double) * (size_t)n * F);
  double* U = (double*)malloc(sizeof(double) * (size_t)n * F);
  double* S = (double*)malloc(sizeof(double) * (size_t)n * n);
  double gq[1024], gk[1024], tmp[1024];
  for (int32_t l = 0; l < s->n_layers; ++l) {
    const layer_w* L = &m->slow[l];
    for (int32_t i = 0; i < n; ++i) rmsnorm_w(X + (size_t)i * H, L->attn_norm, 0, H, eps, xn + (size_t)i * H);
    matvec(L->wq, 0, qd, H, xn, n, Q);
    matvec(L->wk, 0, kd, H, xn, n, Kx);
    matvec(L->wv, 0, kd, H, xn, n, Vx);
    gains_to_f64(L->q_norm, D, gq);
    gains_to_f64(L->k_norm, D, gk);
    for (int32_t i = 0; i < n; ++i) {
      const double* c = m->rope_cos_slow + (size_t)i * hd;
      const double* sn = m->rope_sin_slow + (size_t)i * hd;
      for (int32_t h = 0; h < Hq; ++h) {
        double* qh = Q + (size_t)i * qd + (size_t)h * D;
        orc_rmsnorm(qh, gq, D, eps, tmp);
        for (int32_t d = 0; d < D; ++d) qh[d] = tmp[d];
        orc_rope_apply(qh, D, c, sn);
      }
      for (int32_t h = 0; h < Hkv; ++h) {
        double* kh = Kx + (size_t)i * kd + (size_t)h * D;
        orc_rmsnorm(kh, gk, D, eps, tmp);
        for (int32_t d = 0; d < D; ++d) kh[d] = tmp[d];
        orc_rope_apply(kh, D, c, sn);
      }
    }
    for (int32_t h = 0; h < Hq; ++h) {
      int32_t g = h / group;
#pragma omp parallel for schedule(static)
      for (int32_t i = 0; i < n; ++i) {
        for (int32_t j = 0; j < n; ++j) {
          double a = 0.0;
          for (int32_t d = 0; d < D; ++d) a += Q[(size_t)i * qd + (size_t)h * D + d] * Kx[(size_t)j * kd + (size_t)g * D + d];
          S[(size_t)i * n + j] = (j <= i) ? a * scale : -INFINITY;
        }
        double mx = -INFINITY, sum = 0.0;
        for (int32_t j = 0; j < n; ++j) mx = S[(size_t)i * n + j] > mx ? S[(size_t)i * n + j] : mx;
        for (int32_t j = 0; j < n; ++j) {
          S[(size_t)i * n + j] = exp(S[(size_t)i * n + j] - mx);
          sum += S[(size_t)i * n + j];
        }
        for (int32_t d = 0; d < D; ++d) {
          double a = 0.0;
          for (int32_t j = 0; j < n; ++j) a += S[(size_t)i * n + j] * Vx[(size_t)j * kd + (size_t)g * D + d];
          O[(size_t)i * qd + (size_t)h * D + d] = a / sum;
        }
      }
    }
    matvec(L->wo, 0, H, qd, O, n, T);
    for (size_t e = 0; e < (size_t)n * H; ++e) X[e] += T[e];
    for (int32_t i = 0; i < n; ++i) rmsnorm_w(X + (size_t)i * H, L->mlp_norm, 0, H, eps, xn + (size_t)i * H);
    matvec(L->w_gate, 0, F, H, xn, n, G);
    matvec(L->w_up, 0, F, H, xn, n, U);
    for (size_t e = 0; e < (size_t)n * F; ++e) G[e] = orc_silu(G[e]) * U[e];
    matvec(L->w_down, 0, H, F, G, n, T);
    for (size_t e = 0; e < (size_t)n * H; ++e) X[e] += T[e];
  }
  for (int32_t i = 0; i < n; ++i) rmsnorm_w(X + (size_t)i * H, m->slow_final, 0, H, eps, h_out + (size_t)i * H);
  free(X); free(xn); free(Q); free(Kx); free(Vx); free(O); free(T); free(G); free(U); free(S);
  return 0;
}
