/*
 * CPU oracle of the Dual-AR per-frame decode step (FishAudio S2 shape).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, import or
 * call this code: only the test suite, the smoke check and the CPU baseline of
 * the benchmark do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Precision: every activation, KV entry, logit and reduction is fp64.  Weights
 * arrive as fp32 or as bf16 bit patterns and are widened exactly.  Dot products
 * sum over the input index in ascending order; each output element is produced
 * by one thread, so the thread count never changes a bit.  The RoPE cos/sin
 * table is computed in fp64 and, when rope_bf16 is set, rounded to fp32 and then
 * to bf16 (the model was trained with bf16 RoPE frequencies: "SGLang Day-0
 * Support for FishAudio S2", Engineering Appendix, BF16 RoPE Precision
 * Mismatch).
 *
 * Parity pins: every function here is pinned by a CPU test against closed
 * forms, brute force or reductions to textbook special cases; the one result
 * that no page fixes -- end-to-end values of a trained S2 -- is "parity
 * unpinned" (the pages print no logits, codes or hidden states for any input).
 */
#ifndef S2AR_ORACLE_H
#define S2AR_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn;
} orc_stack;

typedef struct {
  orc_stack slow, fast;
  int32_t vocab_text, n_codebooks, codebook_size;
  double rope_theta, rms_eps;
  int32_t weight_dtype; /* 0: fp32 arrays, 1: bf16 bit patterns (uint16) */
  int32_t rope_bf16;    /* 1: cos/sin rounded to bf16 */
  int32_t max_context;
  int32_t eos_id;       /* -1: no stop token; else a text id in [0, vocab_text) that ends the stream */
} orc_config;

typedef struct orc_model orc_model;
typedef struct orc_state orc_state;

/* tensors: canonical order (see the synthetic-input module); the caller keeps
 * them alive for the model's lifetime.  Returns NULL on a shape error. */
orc_model* orc_model_new(const orc_config* cfg, const void* const* tensors, int32_t n_tensors);
void orc_model_free(orc_model* m);
int32_t orc_n_tensors(const orc_config* cfg);

orc_state* orc_state_new(const orc_model* m);
void orc_state_free(orc_state* s);
int32_t orc_state_pos(const orc_state* s);

/* Input embeddings (fp64 [hidden]). */
int orc_embed_token(const orc_model* m, int32_t token, double* x);
int orc_embed_codes(const orc_model* m, const int32_t* codes /*[n_codebooks]*/, double* x);

/* The Slow pick.  The pages constrain the Slow AR's greedy pick to the semantic ids ("SGLang Day-0
 * Support for FishAudio S2", Background and Motivation) and speak of the model ending early on an EOS
 * token (same page, Attention Backend Divergence Causing Early Stopping), so the EOS id must be a
 * candidate too.  Reading taken: with eos_id >= 0 the candidates are eos_id and the semantic ids, the
 * largest logit wins and a tie goes to the lowest id (the EOS id, a text id, is below every semantic
 * id); the pick is reported as c0 = -1.  With eos_id = -1 only the semantic ids compete.  c0 is the
 * semantic code (id - vocab_text) or -1; the margin is the winner minus the best other candidate.
 * The outputs of prefill and of a Slow step below carry this pick. */
int32_t orc_slow_pick(const double* logits, int32_t vocab_text, int32_t codebook_size, int32_t eos_id,
                      double* margin);

/* Prefill n positions (tokens, optional mask/codes).  The last position goes
 * through the final norm and the Slow head; outputs may be NULL. */
int orc_prefill(const orc_model* m, orc_state* st, const int32_t* tokens, const uint8_t* vq_mask,
                const int32_t* vq_codes, int32_t n, double* h_out, double* logits_out,
                int32_t* c0_out, double* margin_out);

/* One Slow AR step at the next position on the embedding of `codes`.
 * resid_tap: [slow.n_layers][hidden] residual after each layer. */
int orc_slow_step_codes(const orc_model* m, orc_state* st, const int32_t* codes, double* resid_tap,
                        double* h_out, double* logits_out, int32_t* c0_out, double* margin_out);

/* The Fast AR loop: 9 greedy steps on the Slow hidden h.  forced (c1..c9, may
 * be NULL) replaces the model's own pick as the input of the next step.
 * codes_out/margins: [9]; resid_tap: [9][fast.n_layers][hidden];
 * z_tap: [9][hidden]; logits_tap: [9][codebook_size].  All taps may be NULL. */
int orc_fast_loop(const orc_model* m, const double* h, const int32_t* forced, int32_t* codes_out,
                  double* margins, double* resid_tap, double* z_tap, double* logits_tap);

/* Free-running greedy decode of n_frames after a prefill, in the pages' order:
 * frame 1 uses the prefill's (h, c0); frame t >= 2 first runs the Slow step on
 * frame t-1's ten codes.  codes_out: [n_frames][n_codebooks].  A Slow pick of the
 * EOS id (c0 = -1) ends the stream: that frame and every later one are written as
 * n_codebooks values of -1 and nothing more is computed. */
int orc_generate(const orc_model* m, orc_state* st, const double* h0, int32_t c0, int32_t n_frames,
                 int32_t* codes_out);

/* Matrix-form forward over n positions with no KV cache (full causal
 * attention); h_out: [n][hidden] final-normed hidden at every position. */
int orc_full_recompute(const orc_model* m, const int32_t* tokens, const uint8_t* vq_mask,
                       const int32_t* vq_codes, int32_t n, double* h_out);

/* ---- unit functions (the same code the model path runs) ---- */
void orc_rmsnorm(const double* x, const double* g, int32_t n, double eps, double* y);
void orc_rope_row(double theta, int32_t head_dim, int32_t pos, int32_t bf16, double* cos_out, double* sin_out);
void orc_rope_apply(double* v, int32_t head_dim, const double* cos_row, const double* sin_row);
void orc_attention(const double* q, const double* k_cache, const double* v_cache, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t head_dim, int32_t ctx, double* o, double* probs);
double orc_silu(double z);
int32_t orc_argmax(const double* v, int32_t lo, int32_t hi, double* margin);
void orc_matvec_f32(const float* w, int32_t n_rows, int32_t k, const double* x, int32_t n_vec, double* y);
double orc_bf16_round(double v);

/* Symmetric int8 weights with one scale per output row ("s2pro-native": Where it stands, eight-bit
 * weights; The gate that says no, INT8 with per-channel weight scales).  Reading taken: per row,
 * s = max_k |w_k| / 127 and q_k = rint(w_k / s), both in IEEE fp32 with round-to-nearest-even,
 * q in [-127, 127]; a row of zeros has s = 0 and q = 0.  The model then uses q * s.
 * w: bf16 bit patterns [rows][cols]; q: [rows][cols]; s: [rows]. */
void orc_quantize_rows_i8(const uint16_t* w, int64_t rows, int64_t cols, int8_t* q, float* s);
/* out[r][k] = (float)q[r][k] * s[r], an fp32 product */
void orc_dequantize_rows_i8(const int8_t* q, const float* s, int64_t rows, int64_t cols, float* out);

/* FP8 weights, measured only ("s2pro-native", The gate that says no: FP8 runs about twice as fast
 * as bf16 and fails the fidelity gate).  Format: OCP FP8 E4M3 (bias 7, largest finite 448, no
 * infinities), the gfx950 matrix-core format.  Reading taken: one scale per output row, as for int8:
 * s = max_k |w_k| / 448 in fp32, v_k = w_k / s in fp32, q_k = the nearest E4M3 value to v_k with ties
 * to the even code; a row of zeros has s = 0 and q = 0.  The model then uses value(q) * s. */
double orc_f8_value(uint8_t b);
void orc_quantize_rows_f8(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* q, float* s);
/* out[r][k] = (float)value(q[r][k]) * s[r], an fp32 product */
void orc_dequantize_rows_f8(const uint8_t* q, const float* s, int64_t rows, int64_t cols, float* out);

/* Instrumented counters: [slow steps, fast steps, fast layer passes, codes emitted]. */
void orc_get_counters(int64_t* out4);
void orc_reset_counters(void);
void orc_set_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
