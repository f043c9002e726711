// Internal launchers of the gfx950 kernels of the Dual-AR frame.  Host code in
// engine.hip calls these; nothing here is part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2k {

// Epilogue of a weight-streaming GEMV y = W . xin (W: [N][K] row-major).
enum GemvKind : int {
  GEMV_NORM_STORE = 0,   // y[n] = W . rmsnorm(x)            (fused QKV projection)
  GEMV_RESID = 1,        // y[n] += W . x                    (O / down projection + residual)
  GEMV_NORM_SWIGLU = 2,  // rows (2i, 2i+1) = (gate_i, up_i): y[i] = silu(g) * u
  GEMV_NORM_ARGMAX = 3,  // logits y[n] = W . rmsnorm(x); greedy pick over [lo, hi)
};

// x and gain must be readable up to pad_k(K) floats, with zeros past K.
int pad_k(int K);

struct GemvArgs {
  const void* w;          // weights (bf16 bits, fp32, or 8-bit codes when wscale is set), [N][K]
  const float* wscale;    // 8-bit weights: fp32 scale of each row [N]; nullptr for bf16 / fp32
  int w_f8;               // 8-bit weights: 0 = int8, 1 = OCP FP8 E4M3 bytes
  const float* x;         // input vector [pad_k(K)] (fp32, zero past K)
  const float* gain;      // RMSNorm gain [pad_k(K)] (fp32, zero past K) for the NORM kinds
  float eps;
  float* y;               // output (see GemvKind)
  float* xnorm_out;       // optional: normalised input written by block 0 ([K])
  int N, K;
  // greedy pick, first pass (GEMV_NORM_ARGMAX): per-block maximum over rows in [lo, hi)
  int am_lo, am_hi;
  float* am_val;          // [n_blocks] per-block maxima (-inf for blocks outside the range)
  int* am_idx;            // [n_blocks] per-block arg maxima
  // launch_gemv_pick only: the input is codebook row pk_codebook[pk_j][code] (bf16 bits,
  // [codebooks][pk_ncb][K]), code being a head's greedy pick: the largest of the first-pass partials
  // pk_val / pk_idx [pk_b0, pk_b0 + pk_n), lowest index on ties, minus pk_lo (0 if every partial is
  // NaN).  Every block repeats that second pass; block 0 writes the row to pk_x [K] (the residual the
  // layer adds into) and the code to pk_codes[pk_j].
  const float* pk_val;
  const int* pk_idx;
  int pk_b0, pk_n, pk_lo;
  const uint16_t* pk_codebook;
  int pk_ncb, pk_j;
  int* pk_codes;
  float* pk_x;
};

// Number of workgroups a GEMV launch of this shape uses (sizes argmax partials).
int gemv_blocks(int kind, int N);
hipError_t launch_gemv(int kind, bool bf16, const GemvArgs& a, hipStream_t s);
// GEMV_NORM_STORE (bf16 weights, or 8-bit codes with wscale / w_f8 as in launch_gemv) whose input is
// the codebook row of a head's greedy pick (the pk_ fields above): the pick's second pass and the row gather run in the GEMV's own prologue, behind
// its first weight loads.  gemv_pick_fits says whether a launch of this shape is supported (K = 1024
// or 2560, at most 512 partials); launch_gemv_pick returns hipErrorInvalidValue where it is not.
bool gemv_pick_fits(int K, int n_partials);
hipError_t launch_gemv_pick(const GemvArgs& a, hipStream_t s);

struct AttnArgs {
  const float* qkv;        // [M][(Hq + 2 Hkv) D]: q heads, then k heads, then v heads
  const float* q_norm;     // [D]
  const float* k_norm;     // [D]
  const float* rope_cos;   // [positions][D/2], already rounded as the model requires
  const float* rope_sin;
  const int* slots;        // [M] stream slot of each batch row
  const int* pos;          // [slots] position of the new token (context = pos + 1)
  void* k_cache;           // [pages][Hkv][page_size][D], fp32 or bf16 bits (one layer)
  void* v_cache;
  int k_bf16, v_bf16;      // element of the key / value cache: 1 bf16 bits, 0 fp32
  const int* block_table;  // [slots][bt_stride]
  int bt_stride;
  float* out;              // [M][Hq D]
  float* part_ml;          // [M][Hq][max_splits][2]: running max and sum of one context split
  float* part_o;           // [M][Hq][max_splits][D]: unnormalised output of one split
  int max_splits;          // grid extent along the context
  int split;               // positions per split (multiple of 64)
  int M, Hq, Hkv, D, page_size;
  float eps;
  float scale;             // 1 / sqrt(D), applied to q after RoPE
  // prompt rows (prefill): every batch row belongs to stream `fixed_slot` (>= 0) and sits at
  // position row_pos[b]; with append == 0 the rows' keys and values are already in the cache
  int fixed_slot;
  const int* row_pos;
  int append;
  // batched decode: q, k, v are the sum of qkv_S split-K partials qkv_part[s][16][qkv_ldp]
  // (batch row b at row b of each split) instead of qkv; qkv_S == 0 reads qkv
  const float* qkv_part;
  int qkv_S;
  int qkv_ldp;
  // >= 0: every row's position is this constant (the Fast AR's step j sits at position j - 1), and
  // `pos` is not read
  int const_pos;
};
// Attention of the new position over its context; a context longer than `split` is cut into
// splits whose partial results launch_attention_combine merges (needed only when
// max_splits > 1; it does nothing for contexts that fit one split).
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_combine(const AttnArgs& a, hipStream_t s);
// The same attention for long contexts of many streams (the batched step): splits of 256 keys
// (a.split must be 256), four wavefronts of 64 keys each reading the key and value rows straight
// from the cache; split partials merge with launch_attention_combine as above.
hipError_t launch_attention_long(const AttnArgs& a, hipStream_t s);
bool attention_long_supports(int D, int Hq, int Hkv);  // head_dim 64 or 128, 1, 2 or 4 q heads per KV head

// Second pass of the greedy pick over per-block maxima of blocks [b0, b1] (ties to the lowest
// index), followed by the step's bookkeeping (see FinishMode).
enum FinishMode : int { FIN_CODE = 0, FIN_FAST_NEXT = 1, FIN_FAST_LAST = 2, FIN_SLOW = 3 };
struct FinishArgs {
  const float* am_val;
  const int* am_idx;
  int b0, b1, lo;
  int mode;
  int j;                 // index of the code being picked in codes[]
  int* codes;            // [n_codebooks] codes of the stream's current frame
  int* snap;             // FIN_FAST_LAST: copy of the finished frame's codes
  int* pos;              // FIN_SLOW: the stream's Slow position
  const void* codebook;  // [NC][K][H] (bf16 bits or fp32)
  const float* h;        // FIN_SLOW: the final-normed Slow hidden
  float* x;              // next input vector [H]
  int H, K, NC;
  // FIN_SLOW with a stop id: logits[eos_at] is its logit; if it is >= the best semantic logit the
  // pick is the stop (code -1).  eos_at < 0: no stop id.
  const float* logits;
  int eos_at;
};
hipError_t launch_finish(bool bf16, const FinishArgs& f, hipStream_t s);
void set_device_cus(int n);
int device_cus();

// weight formats of the matrix-core kernels: bf16, or 8-bit codes (int8, OCP FP8 E4M3) with an fp32
// scale per output row; the codes are exact in bf16, so the MFMA sees them unrounded
enum WeightFmt : int { W_BF16 = 0, W_I8 = 1, W_F8 = 2 };

// ---- prefill (prefill.hip) ----
enum GemmEpi : int { GEMM_STORE = 0, GEMM_ADD = 1, GEMM_SWIGLU = 2 };
// C[M][N] (=, +=) bf16(A[M][K] * a_scale[m] * a_gain[k]) . W[N][K]^T with fp32 accumulation on the
// matrix cores.  GEMM_SWIGLU: W rows (2i, 2i+1) = (gate_i, up_i); C[m][i] = silu(gate) * up.
// Requires N % 128 == 0, K % 32 == 0, lda % 4 == 0.
struct GemmArgs {
  const uint16_t* a_hi;    // [M][lda] activations as bf16 high parts
  const uint16_t* a_lo;    // [M][lda] and bf16 low parts (x - hi, rounded): x = hi + lo + O(2^-17 |x|)
  int lda;
  const void* w;           // [N][K] weights: bf16, or 8-bit codes (w_fmt) with a scale per row
  const float* wscale;     // 8-bit weights: [N] row scales
  int w_fmt;               // W_BF16, W_I8 or W_F8
  float* c;                // [M][ldc] fp32 output (GEMM_STORE, GEMM_ADD)
  uint16_t* c_hi;          // GEMM_SWIGLU: [M][ldc] silu(g) u as bf16 high and low planes
  uint16_t* c_lo;
  int ldc;
  int M, N, K;
  int epi;
  // split-K workspace for short prompts ([splits][M][N] fp32 partials, part_floats capacity);
  // nullptr: never split.  `split` is set by the launcher.
  float* part;
  size_t part_floats;
  int split;
  // 1: a_hi holds the activations as IEEE fp16 (a_lo unused), the products run on the fp16 matrix
  // cores with the weights converted to fp16, and GEMM_SWIGLU writes one fp16 plane to c_hi,
  // raising *range_flag (device int) for a value fp16 cannot hold.  Needs K % 64 == 0.
  int a_f16;
  int* range_flag;
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
// RMSNorm of M rows and the bf16 split of the result: hi/lo planes of x[m] * (scale[m] * gain),
// scale = 1 / sqrt(mean(x[m]^2) + eps).  One 256-thread block per row.  lo == nullptr: one IEEE
// fp16 plane in hi instead, raising *range_flag for a value fp16 cannot hold.
hipError_t launch_norm_split(const float* x, int ld, int H, float eps, const float* gain, uint16_t* hi, uint16_t* lo,
                             int ldo, int M, int* range_flag, hipStream_t s);

struct PrefillKvArgs {
  const float* qkv;        // [rows][ld] projections of the prompt rows
  int ld;
  const float* k_norm;
  const float* rope_cos;
  const float* rope_sin;
  void* k_cache;           // one layer of the paged pool
  void* v_cache;
  int k_bf16, v_bf16;      // element of the key / value cache: 1 bf16 bits, 0 fp32
  const int* block_table;  // the stream's row of the block table
  int page_size;
  int pos0;                // position of row 0
  int Hq, Hkv, D;
  float eps;
};
hipError_t launch_prefill_append(const PrefillKvArgs& a, int rows, hipStream_t s);

// Causal attention of prompt rows pos0 .. pos0 + rows - 1 over the stream's cache (their own keys
// and values appended beforehand).  q heads are normalised and rotated here.
struct PrefillAttnArgs {
  const float* qkv;        // [rows][ld]
  int ld;
  const float* q_norm;
  const float* rope_cos;
  const float* rope_sin;
  const void* k_cache;     // one layer of the paged pool
  const void* v_cache;
  int k_bf16, v_bf16;      // element of the key / value cache: 1 bf16 bits, 0 fp32
  const int* block_table;  // the stream's row of the block table
  int page_size;
  uint16_t* out_hi;        // [rows][ld_out] attention output as bf16 high and low planes (the
  uint16_t* out_lo;        // O projection's input); out_lo == nullptr: one IEEE fp16 plane in out_hi,
  int* range_flag;         // raising *range_flag for a value fp16 cannot hold
  int ld_out;
  int rows, pos0, Hq, Hkv, D;
  float eps, scale;
  // Key splits: a row block whose causal key range spans more than tps tiles of 64 keys is served
  // by ceil(tiles / tps) workgroups (the heaviest row blocks first).  Each writes its unnormalised
  // output and its per-row (max, sum) to part_o [split][rows][Hq][D] and part_ml [split][rows][Hq][2];
  // a second kernel merges them in split order into the planes.  1 <= tps <= 8.
  int tps;
  float* part_o;
  float* part_ml;
};
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s);
// Key splits the largest row block of a prefill of `rows` rows at positions pos0.. takes.
int prefill_attn_splits(int rows, int pos0, int tps);
hipError_t launch_embed_rows(bool bf16, const void* emb, const void* cb, int K, int H, int NC, const int* tokens,
                             const uint8_t* mask, const int* codes, int p0, int rows, float* x, int ldx,
                             hipStream_t s);
int argmax_block_rows();

// x[b] = sum_k codebook[k][codes[slot][k]] (fp32, k ascending); snap[slot] = codes[slot].
hipError_t launch_embed_codes(bool bf16, const void* codebook, int K, int H, int NC, const int* slots,
                              const int* codes, int* snap, float* x, int ldx, int M, hipStream_t s);
// Fast step j input: j == 1 -> h[slot]; j >= 2 -> codebook[j-1][codes[slot][j-1]].
hipError_t launch_fast_input(bool bf16, const void* codebook, const float* h, int K, int H, int NC,
                             const int* slots, const int* codes, int j, float* x, int ldx, int M, hipStream_t s);
// Prompt position p: mask[p] ? sum of codebook rows of codes[p] : embed[tokens[p]].
hipError_t launch_embed_prompt(bool bf16, const void* embed, const void* codebook, int K, int H, int NC,
                               const int* tokens, const uint8_t* mask, const int* codes, int p, float* x,
                               hipStream_t s);
// pos[slots[b]] += 1
hipError_t launch_advance(const int* slots, int* pos, int M, hipStream_t s);

// Plain streaming read of [p, p + bytes) (measure.hip): context for the GEMV rates.
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t s);

// ---- batched multi-stream decode (batch.hip) ----
enum MgemvEpi : int { MG_STORE = 0, MG_ADD = 1, MG_SWIGLU = 2, MG_ARGMAX = 3 };
// out[j][n] = sum_k W[n][k] * x[j][k] for batch rows j < M <= 16, on the matrix cores (x already
// normalised).  K splits into S ranges, each a multiple of 512; blocks run ipb (64-row tile,
// split) items each.  MG_STORE / MG_SWIGLU reduce the splits in split
// order; MG_ADD leaves part[s][j][n] for k_norm_rows to fold into the residual.  MG_SWIGLU: W rows
// (2i, 2i+1) = (gate_i, up_i), out[j][i] = silu(g) u.  MG_ARGMAX: out = logits and
// am_val/am_idx[16-row group][j] = maxima over rows [am_lo, am_hi) (ties to the lowest row).
struct MgemvArgs {
  const float* x;          // [M][ldx] fp32 batch rows (normalised where a norm precedes)
  int ldx;
  const void* w;           // [N][K] in the tiled layout of launch_tile_weights (bf16) or
                           // launch_tile_weights8 (8-bit codes)
  const float* wscale;     // 8-bit weights: fp32 scale of each row, readable up to mgemv_tiles(N) * 64
  int w_fmt;               // W_BF16, W_I8 or W_F8
  float* out;              // [M][ldo]
  int ldo;
  float* part;             // [S][M][N] split partials (S > 1, and always for MG_ADD)
  int M, N, K, S;
  int ipb;                 // items per block
  int epi;
  int am_lo, am_hi;
  float* am_val;           // [N / 16][16]
  int* am_idx;
  // optional RMSNorm of the input rows, applied while they are staged (split-K form only):
  // x[j][k] / sqrt(sum_c ssq[j][c] / K + eps) * gain[k]
  const float* ssq;        // [M][nssq] partial sums of squares (k_fold_rows), or nullptr
  int nssq;
  const float* gain;
  float eps;
};
int mgemv_tiles(int N);
hipError_t launch_mgemv(const MgemvArgs& a, hipStream_t s);
// Tiled copy for k_mgemv of a row-major bf16 [N][K] matrix (K a multiple of 128): 16-row x 128-K
// blocks of 4 KB, rows zero-padded to a multiple of 64; tiled_weight_elems(N, K) elements.
size_t tiled_weight_elems(int N, int K);
hipError_t launch_tile_weights(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t s);
// The same tiling for 8-bit codes: 16-row x 128-K blocks of 2 KB in which each 16-byte piece is 16
// consecutive codes of one row; tiled_weight_elems(N, K) bytes.
hipError_t launch_tile_weights8(const uint8_t* src, uint8_t* dst, int N, int K, hipStream_t s);

// x[j] += sum_s part[s][j] (split order, when S > 0); xn[j] = RMSNorm(x[j]) * gain.  M rows.
struct NormRowsArgs {
  float* x;
  int ldx;
  const float* part;       // [S][M][H] pending residual partials
  int S, M, H;
  const float* gain;
  float eps;
  float* xn;               // [M][ldx] normalised rows (or nullptr: only fold the partials)
};
hipError_t launch_norm_rows(const NormRowsArgs& a, hipStream_t s);
// x[j] += sum_s part[s][j] (split order, S >= 0) and ssq[j][c] = sum of x[j][e]^2 over the 256-wide
// chunk c (ceil(H / 256) chunks).  grid = (chunks, M).
struct FoldArgs {
  float* x;
  int ldx;
  const float* part;       // [S][16][ldp] pending residual partials
  int S, M, H;
  float* ssq;              // [M][ceil(H / 256)]
};
int fold_chunks(int H);
hipError_t launch_fold_rows(const FoldArgs& a, hipStream_t s);

struct FinishBArgs {
  const float* am_val;     // [blocks][16]
  const int* am_idx;
  int b0, b1, lo;
  int mode, j;
  const int* slots;        // [M] stream slot of each batch row
  int* codes;              // [streams][NC]
  int* snap;               // [streams][NC]
  int* pos;                // [streams]
  const void* codebook;
  float* h;                // [streams][H]
  float* x;                // [M][ldx] next input rows
  int ldx;
  const float* x_res;      // FIN_SLOW: final-normalised batch rows [M][ldx]
  float* xf_slot;          // FIN_SLOW: also write h into the single-stream Fast residual of the slot
  int ld_xf_slot;
  int H, K, NC;
  const float* logits;     // FIN_SLOW with a stop id: row b's logits at logits + b * ld_logits
  int ld_logits;
  int eos_at;              // index of the stop id's logit in a row (< 0: no stop id)
};
hipError_t launch_finish_b(bool bf16, const FinishBArgs& f, int M, hipStream_t s);
hipError_t launch_gather_h(const float* h, const int* slots, int H, float* x, int ldx, int M, hipStream_t s);

}  // namespace s2k
