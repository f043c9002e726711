/*
 * s2ar -- Dual-AR per-frame decode step (FishAudio S2 shape) on one MI355X.
 *
 * The model and what a frame is ("SGLang Day-0 Support for FishAudio S2",
 * section Architecture, Stage 2; "s2pro-native", section What happens to a
 * sentence; "Fish Audio Abre Codigo do S2", section Arquitetura Dual-AR):
 *   - a Slow AR (Qwen3-style decoder: RMSNorm, GQA with QK-norm and RoPE,
 *     SwiGLU) runs along time over a KV cache and picks one semantic code per
 *     frame, with the pick restricted to the semantic ids (S2 page, Background
 *     and Motivation: constrained decoding);
 *   - a Fast AR runs 9 greedy steps on the Slow hidden state and picks the 9
 *     residual codes;
 *   - the frame's 10 codebook embeddings are summed and injected as the next
 *     Slow input (VQ injection at masked positions).
 * Prompt token ids plus optional 10-codebook VQ codes go in; one 10-code tuple
 * per frame comes out (S2 page, Architecture, Stage 1 and Stage 3).
 *
 * Conventions for every call:
 *   - returns S2AR_OK (0) or a negative S2AR_E_* code; nothing throws or aborts;
 *   - arguments are validated before any device work; a failed call leaves the
 *     context's state as it was (a failed S2AR_E_DEVICE call may leave it
 *     unusable: destroy it);
 *   - all pointers are HOST pointers unless stated otherwise; the library reads
 *     host inputs only during the call and writes host outputs before it
 *     returns;
 *   - the context owns every device allocation (weights, KV pages, workspace,
 *     captured graphs) and frees them in s2ar_destroy;
 *   - a context is not thread-safe; calls are synchronous.
 */
#ifndef S2AR_H
#define S2AR_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S2AR_OK 0
#define S2AR_E_ARG (-1)      /* null pointer, bad size, inconsistent config */
#define S2AR_E_RANGE (-2)    /* token id, code or stream id out of range */
#define S2AR_E_CAPACITY (-3) /* context would exceed max_context, or no free KV page */
#define S2AR_E_STATE (-4)    /* call out of order (decode before prefill) */
#define S2AR_E_NOMEM (-5)    /* device or host allocation failed */
#define S2AR_E_DEVICE (-6)   /* HIP runtime error (message in s2ar_last_error) */
#define S2AR_E_NUMERIC (-7)  /* non-finite logits (checked by s2ar_debug_frame only) */

typedef struct s2ar_ctx s2ar_ctx;

/* Shape of one transformer stack.  q heads per KV head = n_q_heads/n_kv_heads. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn;
} s2ar_stack;

typedef struct {
  s2ar_stack slow, fast;  /* fast.hidden must equal slow.hidden: the Slow hidden feeds the Fast AR */
  int32_t vocab_text;     /* text ids are [0, vocab_text); semantic code c has id vocab_text + c */
  int32_t n_codebooks;    /* 10: one semantic + nine residual codebooks */
  int32_t codebook_size;  /* entries per codebook */
  double rope_theta;      /* RoPE base (1e6 for S2) */
  double rms_eps;         /* RMSNorm epsilon, inside the square root */
  int32_t weight_dtype;   /* 0: fp32 weights, 1: bf16 weights, 2: bf16 tensors with the layer matrices and
                             both heads stored as int8 with one fp32 scale per output row (symmetric:
                             s = max|w| / 127, q = rint(w / s), computed in fp32 at create; a zero row
                             has s = 0); embeddings, codebooks and gains stay bf16.  Prefill and
                             batched decode run the 8-bit codes on the matrix cores as they do bf16
                             weights ("s2pro-native", Where it stands; The gate that says no); 3: as 2 with
                             OCP FP8 E4M3 codes instead of int8 (s = max|w| / 448, q = the E4M3 value
                             nearest w / s, ties to the even code), measured only: the same page
                             reports FP8 weights as fast but failing its fidelity gate. */
  int32_t rope_bf16;      /* 1: round the cos/sin table to bf16 (S2 page, Engineering Appendix) */
  int32_t max_streams;    /* concurrent decode streams (stream ids 0..max_streams-1) */
  int32_t max_context;    /* Slow positions per stream, prompt plus frames */
  int32_t page_size;      /* KV positions per page; must be 16 */
  int32_t kv_dtype;       /* KV cache elements: 0 = fp32 keys and values (default); 1 = bf16 keys and values
                             (half the KV bytes); 2 = bf16 keys, fp32 values; 3 = fp32 keys, bf16 values
                             (a quarter fewer KV bytes).  bf16 entries are the fp32 values rounded to
                             nearest even when appended. */
  int32_t eos_id;         /* -1: no stop token (decode exactly the frames asked for); else a text id in
                             [0, vocab_text) that also competes in the Slow pick, winning ties (it is
                             below every semantic id).  A stream whose pick is that id has ended: its
                             frame, and every later frame of the same call, comes out as n_codebooks
                             values of -1, and a further decode of it is S2AR_E_STATE until a prefill
                             appends to it or it is released.  The stream's position is then the one
                             after the Slow step that picked the stop: the frames that follow the stop in
                             the call leave nothing in its context ("SGLang Day-0 Support for FishAudio S2",
                             Background and Motivation: constrained decoding; Attention Backend
                             Divergence Causing Early Stopping: the model ends on an EOS token). */
  int32_t head_slice;     /* 0: the Slow head computes every row (text and semantic ids), as the pages
                             count a frame's weights; 1: only the codebook_size semantic rows and the
                             eos_id row are kept on the device and computed (the text rows can never be
                             picked), a semantic slice of the head.  The picks are identical; the
                             debug taps then hold those rows' logits only (the others NaN). */
  /* Device memory source, optional: both NULL = hipMalloc / hipFree.  Otherwise every device
   * allocation of the context comes from dev_alloc(bytes, alloc_user), which returns memory of the
   * current device aligned to 256 bytes, or NULL (the call that needed it then fails with
   * S2AR_E_NOMEM and changes nothing); every block goes back through dev_free(ptr, bytes,
   * alloc_user), in s2ar_destroy or when s2ar_create fails.  It lets the caller's caching allocator
   * (PyTorch's, for one) own the device memory, while the library keeps using it only on its own
   * stream; the library zeroes each block it takes.  Setting only one of the two is S2AR_E_ARG. */
  void* (*dev_alloc)(uint64_t bytes, void* alloc_user);
  void (*dev_free)(void* ptr, uint64_t bytes, void* alloc_user);
  void* alloc_user;
} s2ar_config;

/* One weight tensor in host memory: fp32, or bf16 bit patterns (uint16). */
typedef struct {
  const void* host_ptr;
  int64_t nbytes;
} s2ar_tensor;

/*
 * Create a context and upload the weights.
 * tensors: n_tensors entries in canonical order
 *   slow.embed [vocab_text+codebook_size][H]
 *   per Slow layer: attn_norm[H], wq[Hq*D][H], wk[Hkv*D][H], wv[Hkv*D][H],
 *     q_norm[D], k_norm[D], wo[H][Hq*D], mlp_norm[H], w_gate[F][H], w_up[F][H],
 *     w_down[H][F]
 *   slow.final_norm[H], slow.head[vocab_text+codebook_size][H],
 *   codebook.embed[n_codebooks][codebook_size][H],
 *   per Fast layer: the same eleven, fast.final_norm[H], fast.head[codebook_size][H]
 * Matrices are row-major [out][in]; every tensor has fp32 (weight_dtype 0) or bf16 (1, 2, 3) elements and
 * nbytes must equal its element count times the element size.
 * hip_stream: a hipStream_t (may be NULL = the legacy default stream).  The
 * library orders its work after the work already queued on it at each call.
 * On success *out receives the context; on failure *out is set to NULL.
 */
int s2ar_create(const s2ar_config* cfg, const s2ar_tensor* tensors, int32_t n_tensors, void* hip_stream,
                s2ar_ctx** out);

/*
 * Prefill n prompt positions of a stream (appending to its context).
 * tokens: [n] ids in [0, vocab_text+codebook_size).  vq_mask: [n] or NULL;
 * where vq_mask[i] != 0 the input is the sum of the ten codebook embeddings of
 * vq_codes[i][0..9] (each in [0, codebook_size)) instead of the token's
 * embedding (VQ injection: S2 page, Architecture, Stage 2; the voice-clone
 * reference is prepended as VQ positions: Stage 1).  vq_codes: [n][n_codebooks]
 * or NULL when vq_mask is NULL.
 * The last position goes through the Slow head, which leaves the stream ready
 * for its first frame.
 */
int s2ar_prefill(s2ar_ctx* ctx, int32_t stream_id, const int32_t* tokens, const uint8_t* vq_mask,
                 const int32_t* vq_codes, int32_t n);

/*
 * Arithmetic of the prefill's matrix-core products for later s2ar_prefill calls of the context.  The
 * pages fix no precision for prompt prefill; the acceptance bar (hidden-state cosine >= 0.9999 at
 * every layer, logits within 2e-2 of their largest magnitude) holds in both modes at the S2 shape.
 *   0 (default): each fp32 activation enters the bf16 matrix cores as two bf16 halves, hi = bf16(x)
 *     and lo = bf16(x - hi) (about 16 significant bits), against the exact bf16 weights: two
 *     products per weight.
 *   1: each activation is rounded once to IEEE fp16 (11 significant bits) and the weights are taken
 *     as fp16, rounded to nearest (exact for bf16 magnitudes from 2^-17 to 65504; int8 and E4M3 codes
 *     are exact), one product per weight on the fp16 matrix cores; the prefill attention likewise
 *     rounds q, the cached keys and values and its softmax weights once to fp16 (one product
 *     instead of three).  An activation that fp16 cannot hold (beyond 65504 in magnitude) makes
 *     that s2ar_prefill return S2AR_E_NUMERIC: its positions are dropped and the stream is not
 *     ready to decode until a later prefill succeeds.
 * Decoding is the same in both modes (the cache holds the same fp32 or bf16 keys and values).
 * Errors: S2AR_E_ARG (precision not 0 or 1; 1 on a context whose prefill does not run on the
 * matrix cores, fp32 weights, or whose hidden, q-projection or ffn width is not a multiple of 64).
 */
int s2ar_set_prefill_precision(s2ar_ctx* ctx, int32_t precision);

/*
 * Decode one frame for each listed stream (distinct ids, each prefilled).
 * codes_out: [n_streams][n_codebooks]; entry 0 is the semantic code, 1..9 the
 * residual codes, each in [0, codebook_size).  Each stream then advances by
 * one Slow position (its next semantic code is computed ahead).
 */
int s2ar_decode_frame(s2ar_ctx* ctx, const int32_t* stream_ids, int32_t n_streams, int32_t* codes_out);

/* Same as n_frames calls of s2ar_decode_frame with one final host copy;
 * codes_out: [n_frames][n_streams][n_codebooks]. */
int s2ar_decode_frames(s2ar_ctx* ctx, const int32_t* stream_ids, int32_t n_streams, int32_t n_frames,
                       int32_t* codes_out);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Decodes n_frames frames of one stream exactly as
 * s2ar_decode_frames does for that stream (the same kernels, the same codes bit for bit), but
 * enqueues each frame's kernels directly instead of replaying a captured graph (instantiating one
 * allocates), and keeps the frame's scratch -- the greedy-pick partials and the Slow attention
 * split partials -- in a fixed device array of S2AR_NOALLOC_SCRATCH_BYTES bytes instead of the
 * context's workspace.  It calls no hipMalloc, hipFree or other allocating routine; weights, KV
 * pages and per-stream state are the context's, allocated at s2ar_create.
 * codes_out: [n_frames][n_codebooks], caller-owned host memory.  Errors as s2ar_decode_frames, and
 * S2AR_E_CAPACITY when the frame's scratch (about 156 KB of pick partials plus
 * n_q_heads * (head_dim + 2) * 4 bytes per 64 context positions: contexts up to about 15,000
 * positions at the S2 shape) exceeds the array.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (every
 * scratch word a frame reads is written earlier in the same frame, so nothing needs clearing):
 * calls that overlap on one GPU (from several threads, or on several contexts' streams) race and
 * must be serialised by the caller.
 */
#define S2AR_NOALLOC_SCRATCH_BYTES (4u << 20)
int s2ar_decode_frames_noalloc(s2ar_ctx* ctx, int32_t stream_id, int32_t n_frames, int32_t* codes_out);

/* Forget a stream's context and return its KV pages to the pool. */
int s2ar_release_stream(s2ar_ctx* ctx, int32_t stream_id);

/* Share the first n_positions cached positions of stream src_id with stream dst_id, so a common
 * prefix (a reference-audio clip, a system prompt) is prefilled once and reused: radix prefix
 * caching of shared prefixes ("SGLang Day-0 Support for FishAudio S2", Optimizations with SGLang
 * Omni).  dst_id must be empty (never prefilled, or released).  Every KV page of src that lies
 * wholly inside the prefix becomes a page of dst too (the pool counts its holders and frees it when
 * the last one is released; positions only ever append, so no holder writes it again); the partial
 * last page, if any, is copied into a fresh page of dst.  dst then holds n_positions positions but
 * is not ready to decode: a prefill of at least one more position must follow (it produces the
 * hidden state and the first code).  Ordered like the other calls on the context's stream.
 * Errors: S2AR_E_RANGE (stream ids, or n_positions outside [1, position of src]), S2AR_E_STATE
 * (src_id == dst_id, or dst not empty), S2AR_E_CAPACITY (no free page for the copy); on error nothing
 * changes. */
int s2ar_share_prefix(s2ar_ctx* ctx, int32_t src_id, int32_t dst_id, int32_t n_positions);

/* Current Slow position (= context length) of a stream, or a negative code. */
int s2ar_stream_position(const s2ar_ctx* ctx, int32_t stream_id, int32_t* pos_out);

/* Free everything the context owns.  NULL is a no-op. */
void s2ar_destroy(s2ar_ctx* ctx);

/* Message of the last failed call on ctx (or of the last failed s2ar_create
 * when ctx is NULL); valid until the next call. */
const char* s2ar_last_error(const s2ar_ctx* ctx);
const char* s2ar_error_name(int code);

/*
 * Test and measurement support.
 *
 * s2ar_debug_frame decodes one frame of one stream like s2ar_decode_frame, but
 * without the captured graph, copying intermediate values to host buffers
 * (any may be NULL).  forced_codes ([n_codebooks] or NULL) are teacher-forced
 * codes of this frame: forced_codes[0] replaces the semantic code computed
 * ahead, forced_codes[j] replaces the Fast AR's own pick as the input of step
 * j+1, and the forced tuple is what the next Slow step embeds.
 */
typedef struct {
  float* slow_embed;   /* [H]  Slow input: sum of the frame's codebook rows */
  float* slow_resid;   /* [slow.n_layers][H]  residual after each Slow layer */
  float* slow_h;       /* [H]  final-normed Slow hidden (next frame's Fast input) */
  float* slow_logits;  /* [vocab_text+codebook_size] */
  float* fast_resid;   /* [9][fast.n_layers][H] */
  float* fast_z;       /* [9][H]  final-normed Fast hidden per step */
  float* fast_logits;  /* [9][codebook_size] */
  int32_t* own_codes;  /* [n_codebooks]: the library's own picks this frame */
  int32_t* next_c0;    /* [1]: own semantic pick for the next frame */
} s2ar_taps;

int s2ar_debug_frame(s2ar_ctx* ctx, int32_t stream_id, const int32_t* forced_codes, s2ar_taps* taps);

/* The batched multi-stream frame (the kernels s2ar_decode_frame uses for 2..16 streams), run
 * without the captured graph: forced_codes [n][n_codebooks] or NULL, taps [n] (fast_z and
 * slow_embed are not filled).  Needs weight_dtype 1, 2 or 3 and every K dimension divisible by 512
 * (S2AR_E_ARG otherwise); n <= 16. */
int s2ar_debug_frame_batch(s2ar_ctx* ctx, const int32_t* stream_ids, int32_t n, const int32_t* forced_codes,
                           s2ar_taps* taps);

/* Launch one kernel `iters` times on the context's stream, cycling over the
 * layers, and report the mean duration of a launch measured with HIP events on
 * that stream.  which: 0 = Slow fused RMSNorm + gate/up + SwiGLU GEMV;
 * 1 = a plain streaming read of the same gate/up weights (no arithmetic: the
 * device's practical read rate, context for 0).  bytes_out: algorithmic bytes of
 * one launch.  S2AR_E_ARG for another which, iters < 1 or a null avg_ms. */
int s2ar_time_kernel(s2ar_ctx* ctx, int32_t which, int32_t iters, float* avg_ms, int64_t* bytes_out);

/* Decode n_frames frames of one stream as decode_frames does (one frame-graph replay each, back to
 * back on the context's stream) with a HIP event pair around every replay, and write each
 * replay's duration in ms to ms_out[n_frames] (caller-owned host memory).  The stream advances by
 * n_frames positions; the frames' codes are not returned, so a context with a stop id (eos_id >= 0)
 * is refused.  Errors as decode_frames for one stream, and S2AR_E_ARG for a null ms_out, n_frames
 * outside [1, 4096] or eos_id >= 0. */
int s2ar_time_frames(s2ar_ctx* ctx, int32_t stream_id, int32_t n_frames, float* ms_out);

#ifdef __cplusplus
}
#endif
#endif
