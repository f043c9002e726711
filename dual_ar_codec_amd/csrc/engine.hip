// Host side of the s2ar C ABI: validation, weight upload and repacking, the paged KV pool,
// per-stream device state, the frame's kernel sequence and its hipGraph capture.
//
// A frame follows the Dual-AR order of the pages ("SGLang Day-0 Support for FishAudio S2",
// Architecture, Stage 2): the Fast AR's nine greedy steps on the Slow hidden, then the Slow
// step on the frame's ten codes.  The engine runs it ahead: prefill leaves (h, c0) for frame 1,
// and each decode call runs Fast(t) and then the Slow step that prepares frame t+1, so that
// one captured graph serves every frame.  All per-frame variables (position, codes, hidden,
// block table) live in device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "s2ar.h"

// Scratch of s2ar_decode_frames_noalloc: the greedy-pick partials and the Slow attention split
// partials of one frame, in a fixed array of every device the library runs on (each device holds
// its own copy until the process ends).  Host code never passes `scratch` itself to a kernel (on
// the host it only names the symbol): the device address comes from hipGetSymbolAddress, once per
// device, at context creation.
static __device__ __align__(256) unsigned char scratch[S2AR_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices] = {};

thread_local std::string g_create_error;

constexpr int kPageSize = 16;
constexpr int kMaxStreams = 256;
// context positions per batch-1 attention workgroup: at the voice-clone contexts (1201..1400) 64
// decodes 254.8 frames/s against 249.2 for 128 and 237.0 for 256; at a context of 100 the three agree
constexpr int kAttnSplit = 64;
// a Slow context of at most kShortCtx positions is attended by one workgroup per KV head (one split
// of kShortCtx positions), so its frame needs no split merge launch at all
constexpr int kShortCtx = 128;

// Slow attention split of a frame whose Slow step attends over ctx positions: (positions per
// workgroup, splits).  Every path (captured graphs, eager frames) uses this one rule, so they agree
// bit for bit.
struct SlowSplit {
  int split, nsplit;
};
SlowSplit slow_split_for(int ctx) {
  if (ctx <= kShortCtx) return {kShortCtx, 1};
  return {kAttnSplit, (ctx + kAttnSplit - 1) / kAttnSplit};
}
// prefill attention: at most this many 64-key tiles per workgroup (longer causal ranges are split)
constexpr int kPrefillAttnTiles = 8;

struct LayerW {
  void* wqkv = nullptr;   // [(Hq + 2 Hkv) D][H]: wq rows, then wk rows, then wv rows
  void* wo = nullptr;     // [H][Hq D]
  void* wgu = nullptr;    // [2F][H]: row 2i = w_gate[i], row 2i+1 = w_up[i]
  void* wdown = nullptr;  // [H][F]
  float* attn_norm = nullptr;
  float* mlp_norm = nullptr;
  float* q_norm = nullptr;
  float* k_norm = nullptr;
  // tiled copies of the four matrices for the batched multi-stream GEMVs (k_mgemv layout: bf16, or
  // the 8-bit codes of an int8 / FP8 context)
  void *tqkv = nullptr, *to = nullptr, *tgu = nullptr, *tdown = nullptr;
  // int8 weights: fp32 scale of every row of the four matrices (same row order)
  float *sqkv = nullptr, *so = nullptr, *sgu = nullptr, *sdown = nullptr;
};

struct Graph {
  hipGraph_t g = nullptr;
  hipGraphExec_t exec = nullptr;
};

}  // namespace

struct s2ar_ctx {
  s2ar_config cfg{};
  bool bf16 = true;  // tables (embeddings, codebooks, gains) arrive as bf16
  bool q8 = false;   // layer matrices and heads are stored as 8-bit codes with per-row scales
  bool f8 = false;   // ... and those codes are FP8 E4M3 (else int8)
  int esz = 2;
  hipStream_t user_stream = nullptr;
  hipStream_t stream = nullptr;
  hipEvent_t ev_order = nullptr, ev_t0 = nullptr, ev_t1 = nullptr;
  std::vector<std::pair<void*, size_t>> dev_allocs;  // every device block and its size
  std::vector<void*> host_allocs;

  // weights
  void* embed = nullptr;
  void* slow_head = nullptr;
  void* codebook = nullptr;
  void* fast_head = nullptr;
  void *slow_head_t = nullptr, *fast_head_t = nullptr;  // tiled copies (batched decode)
  float *slow_head_s = nullptr, *fast_head_s = nullptr;      // int8 weights: row scales
  float* slow_final = nullptr;
  float* fast_final = nullptr;
  std::vector<LayerW> slow, fast;
  float *rope_cos_s = nullptr, *rope_sin_s = nullptr, *rope_cos_f = nullptr, *rope_sin_f = nullptr;

  // KV pools (fp32 or bf16): slow [layers][n_pages][Hkv][page][D]; fast [layers][max_streams][Hkv][page][D]
  char *kv_k = nullptr, *kv_v = nullptr, *fkv_k = nullptr, *fkv_v = nullptr;
  // bytes per layer of the key and value pools (Slow and Fast), and their element sizes
  size_t kv_layer_k = 0, kv_layer_v = 0, fkv_layer_k = 0, fkv_layer_v = 0;
  int k_bf16 = 0, v_bf16 = 0;
  int n_pages = 0, bt_stride = 0;
  int* d_bt = nullptr;       // [max_streams][bt_stride]
  int* h_bt = nullptr;       // pinned mirror
  int* d_fast_bt = nullptr;  // [max_streams]: stream s uses fast page s
  std::vector<int> free_pages;
  std::vector<std::vector<int>> stream_pages;
  std::vector<int> page_refs;  // streams holding each page (shared prefixes hold a page several times)

  // per-stream device state
  int* d_pos = nullptr;       // [max_streams] next Slow position
  int* d_codes = nullptr;     // [max_streams][NC] current frame's codes
  float* d_h = nullptr;       // [max_streams][H] final-normed Slow hidden
  int* d_snap = nullptr;      // [max_streams][NC] codes emitted by the last frame
  int* d_slot_ids = nullptr;  // [max_streams] = 0, 1, 2, ...
  int* d_fast_pos = nullptr;  // [NC-1][max_streams] = j - 1
  std::vector<int> pos;
  std::vector<char> ready;
  std::vector<char> ended;  // the stream's Slow pick was the stop id
  // Slow head as stored: head_rows rows, the semantic ids at rows [head_lo, head_lo + K), and the
  // stop id's logit at row head_eos (-1: none)
  int head_rows = 0, head_lo = 0, head_eos = -1;

  // workspace (batch row 0), every input vector zero-padded to pad_k
  float *x = nullptr, *qkv = nullptr, *att = nullptr, *act = nullptr;
  float* xf = nullptr;  // [max_streams][pad_k(H)]: Fast residual; holds h between frames
  float *slow_logits = nullptr, *fast_logits = nullptr, *z = nullptr;
  float* am_val = nullptr;
  int* am_idx = nullptr;
  float *att_ml = nullptr, *att_o = nullptr;
  int max_splits = 0;
  // batched decode: positions per attention workgroup (16 streams of 920..3948 positions measured
  // 9.80 ms per step at 192, 10.20 at 256, 10.52 at 128)
  int attn_split_b = 192, max_splits_b = 0;
  bool attn_long = false;  // batched Slow attention through launch_attention_long (256-key splits)

  // batched prefill (MFMA): chunk of up to pch prompt rows
  int pch = 0;
  // split-K partials of the prefill GEMMs of short prompts
  float* pgemm_part = nullptr;
  size_t pgemm_part_floats = 0;
  bool mfma_prefill = false;
  // prefill products on the fp16 matrix cores (one fp16 activation plane) instead of the bf16 hi/lo
  // split; f16_prefill_ok: every prefill K is a multiple of 64
  bool prefill_f16 = false, f16_prefill_ok = false;
  int* d_range = nullptr;  // raised by a prefill producer whose value fp16 cannot hold
  float *px = nullptr, *pqkv = nullptr;
  // prefill attention key splits: unnormalised outputs and row states of the splits
  float *patt_o = nullptr, *patt_ml = nullptr;
  // bf16 hi / lo planes of the GEMM inputs: normalised residual, attention output, SwiGLU output
  uint16_t *pxh = nullptr, *pxl = nullptr, *patth = nullptr, *pattl = nullptr, *pacth = nullptr, *pactl = nullptr;
  int* d_iota = nullptr;  // [max_context] = 0, 1, 2, ...
  int* h_pos_stage = nullptr;

  // prompt staging
  int* d_tokens = nullptr;
  uint8_t* d_mask = nullptr;
  int* d_pcodes = nullptr;

  // pinned host staging
  int* h_codes = nullptr;  // [max frames per call chunk][max_streams][NC]
  int h_codes_frames = 0;
  float* h_taps = nullptr;
  size_t h_taps_floats = 0;
  int* h_small = nullptr;  // small int staging (forced codes, own picks)

  std::map<int, Graph> graphs;  // per (stream id, attention bucket)
  unsigned char* scratch_dev = nullptr;  // this device's copy of `scratch`

  // batched multi-stream decode (up to 16 streams per launch, MFMA GEMVs)
  bool batched_ok = false;
  float *bx = nullptr, *bxf = nullptr, *bqkv = nullptr, *batt = nullptr, *bact = nullptr;
  float *blogits = nullptr, *bxn = nullptr, *bpart = nullptr, *bam_val = nullptr, *bssq = nullptr;
  int* bam_idx = nullptr;
  float *batt_ml = nullptr, *batt_o = nullptr;
  size_t bpart_floats = 0;
  uint32_t* d_sink = nullptr;  // never-taken store target of the streaming-read measurement
  int* d_dbg_slots = nullptr;  // [16] batch slots of the eager batched frame
  struct BatchGraph {
    Graph g;
    int* d_slots = nullptr;
  };
  std::map<std::vector<int>, BatchGraph> bgraphs;
  std::string err;
};

namespace {

int set_err(s2ar_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  else g_create_error = msg;
  return code;
}

#define HIP_TRY(ctx, expr)                                                                          \
  do {                                                                                              \
    hipError_t e_ = (expr);                                                                         \
    if (e_ != hipSuccess)                                                                           \
      return set_err(ctx, S2AR_E_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_));         \
  } while (0)

int check_stack(const s2ar_stack& s, const char* name, int epc, std::string& why) {
  char buf[256];
  if (s.n_layers < 1 || s.hidden < 1 || s.n_q_heads < 1 || s.n_kv_heads < 1 || s.head_dim < 1 || s.ffn < 1) {
    snprintf(buf, sizeof buf, "%s: every dimension must be >= 1", name);
    why = buf;
    return -1;
  }
  if (s.n_q_heads % s.n_kv_heads) {
    snprintf(buf, sizeof buf, "%s: n_q_heads must be a multiple of n_kv_heads", name);
    why = buf;
    return -1;
  }
  const int g = s.n_q_heads / s.n_kv_heads;
  if (!(s.head_dim == 64 || s.head_dim == 128) || !(g == 1 || g == 2 || g == 4 || g == 8)) {
    snprintf(buf, sizeof buf, "%s: head_dim must be 64 or 128 and n_q_heads/n_kv_heads in {1,2,4,8}", name);
    why = buf;
    return -1;
  }
  const int64_t dims[3] = {s.hidden, (int64_t)s.n_q_heads * s.head_dim, s.ffn};
  for (int64_t d : dims)
    if (d % epc || d > 14336) {
      snprintf(buf, sizeof buf, "%s: hidden, n_q_heads*head_dim and ffn must be multiples of %d and <= 14336", name, epc);
      why = buf;
      return -1;
    }
  return 0;
}

int validate_config(const s2ar_config* c, std::string& why) {
  if (c->weight_dtype < 0 || c->weight_dtype > 3) {
    why = "weight_dtype must be 0 (fp32), 1 (bf16), 2 (bf16 tensors, int8 matrices) or 3 (bf16 tensors, FP8 matrices)";
    return -1;
  }
  const int epc = c->weight_dtype == 0 ? 4 : 8;
  if (check_stack(c->slow, "slow", epc, why) || check_stack(c->fast, "fast", epc, why)) return -1;
  if (c->slow.hidden != c->fast.hidden) {
    why = "fast.hidden must equal slow.hidden (the Slow hidden feeds the Fast AR)";
    return -1;
  }
  if (c->n_codebooks < 2 || c->n_codebooks - 1 > kPageSize) {
    why = "n_codebooks must be in [2, 17]";
    return -1;
  }
  if (c->codebook_size < 1 || c->vocab_text < 0 || (int64_t)c->vocab_text + c->codebook_size > INT32_MAX / 2) {
    why = "vocab_text >= 0 and codebook_size >= 1 required";
    return -1;
  }
  if (c->page_size != kPageSize) {
    why = "page_size must be 16";
    return -1;
  }
  if (c->max_streams < 1 || c->max_streams > kMaxStreams || c->max_context < 1 || c->max_context > (1 << 20)) {
    why = "max_streams must be in [1, 256] and max_context in [1, 2^20]";
    return -1;
  }
  if (c->kv_dtype < 0 || c->kv_dtype > 3) {
    why = "kv_dtype must be 0 (fp32), 1 (bf16), 2 (bf16 keys, fp32 values) or 3 (fp32 keys, bf16 values)";
    return -1;
  }
  if (c->eos_id < -1 || c->eos_id >= c->vocab_text) {
    why = "eos_id must be -1 (none) or a text id in [0, vocab_text)";
    return -1;
  }
  if (c->head_slice != 0 && c->head_slice != 1) {
    why = "head_slice must be 0 (full head) or 1 (semantic rows plus the eos_id row)";
    return -1;
  }
  if ((c->dev_alloc == nullptr) != (c->dev_free == nullptr)) {
    why = "dev_alloc and dev_free must both be set or both be NULL";
    return -1;
  }
  if (!(c->rope_theta > 0.0) || !(c->rms_eps >= 0.0)) {
    why = "rope_theta must be > 0 and rms_eps >= 0";
    return -1;
  }
  return 0;
}

int32_t n_tensors_for(const s2ar_config* c) { return 1 + 11 * c->slow.n_layers + 3 + 11 * c->fast.n_layers + 2; }

// Expected element counts in canonical order.
std::vector<int64_t> tensor_sizes(const s2ar_config* c) {
  std::vector<int64_t> v;
  const int64_t H = c->slow.hidden, V = (int64_t)c->vocab_text + c->codebook_size, K = c->codebook_size;
  v.push_back(V * H);
  auto layer = [&](const s2ar_stack& s) {
    const int64_t Hd = s.hidden, qd = (int64_t)s.n_q_heads * s.head_dim, kd = (int64_t)s.n_kv_heads * s.head_dim;
    v.push_back(Hd);
    v.push_back(qd * Hd);
    v.push_back(kd * Hd);
    v.push_back(kd * Hd);
    v.push_back(s.head_dim);
    v.push_back(s.head_dim);
    v.push_back(Hd * qd);
    v.push_back(Hd);
    v.push_back((int64_t)s.ffn * Hd);
    v.push_back((int64_t)s.ffn * Hd);
    v.push_back(Hd * s.ffn);
  };
  for (int l = 0; l < c->slow.n_layers; ++l) layer(c->slow);
  v.push_back(H);
  v.push_back(V * H);
  v.push_back((int64_t)c->n_codebooks * K * H);
  for (int l = 0; l < c->fast.n_layers; ++l) layer(c->fast);
  v.push_back(H);
  v.push_back(K * H);
  return v;
}

float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

float round_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  u &= 0xffff0000u;
  std::memcpy(&f, &u, 4);
  return f;
}

// One zeroed device block, from the caller's allocator when the config names one, else hipMalloc.
template <typename T>
int dev_alloc(s2ar_ctx* c, T** p, size_t bytes) {
  void* q = nullptr;
  bytes = bytes ? bytes : 16;
  if (c->cfg.dev_alloc) {
    q = c->cfg.dev_alloc((uint64_t)bytes, c->cfg.alloc_user);
    if (!q) return set_err(c, S2AR_E_NOMEM, "dev_alloc returned NULL for " + std::to_string(bytes) + " bytes");
    c->dev_allocs.push_back({q, bytes});
    if (reinterpret_cast<uintptr_t>(q) % 256)
      return set_err(c, S2AR_E_ARG, "dev_alloc returned a pointer not aligned to 256 bytes");
  } else {
    hipError_t e = hipMalloc(&q, bytes);
    if (e != hipSuccess) return set_err(c, e == hipErrorOutOfMemory ? S2AR_E_NOMEM : S2AR_E_DEVICE,
                                        std::string("hipMalloc: ") + hipGetErrorString(e));
    c->dev_allocs.push_back({q, bytes});
  }
  hipError_t e = hipMemset(q, 0, bytes);
  if (e != hipSuccess) return set_err(c, S2AR_E_DEVICE, std::string("hipMemset: ") + hipGetErrorString(e));
  *p = static_cast<T*>(q);
  return 0;
}

template <typename T>
int host_alloc(s2ar_ctx* c, T** p, size_t bytes) {
  void* q = nullptr;
  hipError_t e = hipHostMalloc(&q, bytes ? bytes : 16, hipHostMallocDefault);
  if (e != hipSuccess) return set_err(c, S2AR_E_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  c->host_allocs.push_back(q);
  std::memset(q, 0, bytes ? bytes : 16);
  *p = static_cast<T*>(q);
  return 0;
}

// Upload a norm gain as fp32, zero-padded to pad_k.
int upload_gain(s2ar_ctx* c, const s2ar_tensor& t, int n, float** out) {
  const int np = s2k::pad_k(n);
  std::vector<float> tmp(np, 0.f);
  for (int i = 0; i < n; ++i)
    tmp[i] = c->bf16 ? bf16_bits_to_float(static_cast<const uint16_t*>(t.host_ptr)[i])
                     : static_cast<const float*>(t.host_ptr)[i];
  if (int rc = dev_alloc(c, out, sizeof(float) * np)) return rc;
  HIP_TRY(c, hipMemcpy(*out, tmp.data(), sizeof(float) * np, hipMemcpyHostToDevice));
  return 0;
}

// Symmetric int8 per output row: s = max|w| / 127 and q = rint(w / s), both in fp32 on the host
// (a row of zeros has s = 0 and q = 0); w is used as q * s.  Eight-bit weights halve the bytes a
// batch-1 frame streams ("s2pro-native", Where it stands), with one scale per output channel
// ("s2pro-native", The gate that says no).
void quantize_rows_i8(const uint16_t* w, size_t rows, size_t cols, int8_t* q, float* s) {
  for (size_t r = 0; r < rows; ++r) {
    const uint16_t* row = w + r * cols;
    float m = 0.f;
    for (size_t k = 0; k < cols; ++k) m = std::fmax(m, std::fabs(bf16_bits_to_float(row[k])));
    const float sc = m / 127.0f;
    s[r] = sc;
    for (size_t k = 0; k < cols; ++k) {
      const float v = sc > 0.f ? std::rint(bf16_bits_to_float(row[k]) / sc) : 0.f;
      q[r * cols + k] = (int8_t)std::fmin(127.f, std::fmax(-127.f, v));
    }
  }
}

// OCP FP8 E4M3 byte nearest to v (|v| <= 448 after the clamp), ties to the even code: below 2^-6 the
// grid is the subnormal step 2^-9; in [2^E, 2^(E+1)) it is 2^(E-3), and rint (round to nearest even
// in the default rounding mode) of the value in those steps gives 8 + mantissa, where 16 carries
// into the next exponent.  Scaling by powers of two is exact, so only rint rounds.
uint8_t f32_to_e4m3(float v) {
  const uint8_t sign = v < 0.f ? 0x80 : 0x00;
  const float a = std::fmin(std::fabs(v), 448.0f);
  if (a < 0.015625f) return sign | (uint8_t)std::rint(a * 512.0f);  // 8 lands on 0x08 = 2^-6
  int x = 0;
  std::frexp(a, &x);
  int E = x - 1;
  int q = (int)std::rint(std::ldexp(a, 3 - E));
  if (q == 16) {
    ++E;
    q = 8;
  }
  return sign | (uint8_t)(((E + 7) << 3) | (q - 8));
}

// Per output row FP8: s = max|w| / 448 and q = E4M3(w / s), both in fp32 on the host; w is used as
// value(q) * s ("s2pro-native", The gate that says no: FP8 weights, measured only).
void quantize_rows_f8(const uint16_t* w, size_t rows, size_t cols, uint8_t* q, float* s) {
  for (size_t r = 0; r < rows; ++r) {
    const uint16_t* row = w + r * cols;
    float m = 0.f;
    for (size_t k = 0; k < cols; ++k) m = std::fmax(m, std::fabs(bf16_bits_to_float(row[k])));
    const float sc = m / 448.0f;
    s[r] = sc;
    for (size_t k = 0; k < cols; ++k) q[r * cols + k] = sc > 0.f ? f32_to_e4m3(bf16_bits_to_float(row[k]) / sc) : 0;
  }
}

// Upload row blocks of bf16 host matrices as one 8-bit matrix (int8 or FP8, as the context stores
// them) plus its row scales; block b's rows
// land at rows first[b] + stride * i (stride 2 interleaves the gate and up rows).
struct QBlock {
  const void* src;
  size_t rows, first, stride;
};
int upload_i8(s2ar_ctx* c, const std::vector<QBlock>& blocks, size_t total_rows, size_t cols, void** w, float** sc) {
  std::vector<int8_t> q(total_rows * cols);
  std::vector<float> s(total_rows);
  std::vector<int8_t> qb;
  std::vector<float> sb;
  for (const QBlock& b : blocks) {
    qb.resize(b.rows * cols);
    sb.resize(b.rows);
    if (c->f8)
      quantize_rows_f8(static_cast<const uint16_t*>(b.src), b.rows, cols, reinterpret_cast<uint8_t*>(qb.data()),
                       sb.data());
    else
      quantize_rows_i8(static_cast<const uint16_t*>(b.src), b.rows, cols, qb.data(), sb.data());
    for (size_t i = 0; i < b.rows; ++i) {
      const size_t r = b.first + b.stride * i;
      std::memcpy(q.data() + r * cols, qb.data() + i * cols, cols);
      s[r] = sb[i];
    }
  }
  if (int rc = dev_alloc(c, w, total_rows * cols)) return rc;
  // scales zero-padded to whole 64-row tiles: the batched kernels read them four rows at a time
  if (int rc = dev_alloc(c, sc, sizeof(float) * ((total_rows + 63) / 64 * 64))) return rc;
  HIP_TRY(c, hipMemcpy(*w, q.data(), total_rows * cols, hipMemcpyHostToDevice));
  HIP_TRY(c, hipMemcpy(*sc, s.data(), sizeof(float) * total_rows, hipMemcpyHostToDevice));
  return 0;
}

int upload_layer_i8(s2ar_ctx* c, const s2ar_stack& s, const s2ar_tensor* t, LayerW* L) {
  const size_t H = s.hidden, qd = (size_t)s.n_q_heads * s.head_dim, kd = (size_t)s.n_kv_heads * s.head_dim,
               F = s.ffn;
  if (int rc = upload_gain(c, t[0], s.hidden, &L->attn_norm)) return rc;
  if (int rc = upload_i8(c, {{t[1].host_ptr, qd, 0, 1}, {t[2].host_ptr, kd, qd, 1}, {t[3].host_ptr, kd, qd + kd, 1}},
                         qd + 2 * kd, H, &L->wqkv, &L->sqkv))
    return rc;
  if (int rc = upload_gain(c, t[4], s.head_dim, &L->q_norm)) return rc;
  if (int rc = upload_gain(c, t[5], s.head_dim, &L->k_norm)) return rc;
  if (int rc = upload_i8(c, {{t[6].host_ptr, H, 0, 1}}, H, qd, &L->wo, &L->so)) return rc;
  if (int rc = upload_gain(c, t[7], s.hidden, &L->mlp_norm)) return rc;
  if (int rc = upload_i8(c, {{t[8].host_ptr, F, 0, 2}, {t[9].host_ptr, F, 1, 2}}, 2 * F, H, &L->wgu, &L->sgu)) return rc;
  return upload_i8(c, {{t[10].host_ptr, H, 0, 1}}, H, F, &L->wdown, &L->sdown);
}

int upload_layer(s2ar_ctx* c, const s2ar_stack& s, const s2ar_tensor* t, LayerW* L) {
  if (c->q8) return upload_layer_i8(c, s, t, L);
  const size_t e = c->esz;
  const size_t H = s.hidden, qd = (size_t)s.n_q_heads * s.head_dim, kd = (size_t)s.n_kv_heads * s.head_dim,
               F = s.ffn;
  if (int rc = upload_gain(c, t[0], s.hidden, &L->attn_norm)) return rc;
  if (int rc = dev_alloc(c, &L->wqkv, (qd + 2 * kd) * H * e)) return rc;
  char* q = static_cast<char*>(L->wqkv);
  HIP_TRY(c, hipMemcpy(q, t[1].host_ptr, qd * H * e, hipMemcpyHostToDevice));
  HIP_TRY(c, hipMemcpy(q + qd * H * e, t[2].host_ptr, kd * H * e, hipMemcpyHostToDevice));
  HIP_TRY(c, hipMemcpy(q + (qd + kd) * H * e, t[3].host_ptr, kd * H * e, hipMemcpyHostToDevice));
  if (int rc = upload_gain(c, t[4], s.head_dim, &L->q_norm)) return rc;
  if (int rc = upload_gain(c, t[5], s.head_dim, &L->k_norm)) return rc;
  if (int rc = dev_alloc(c, &L->wo, H * qd * e)) return rc;
  HIP_TRY(c, hipMemcpy(L->wo, t[6].host_ptr, H * qd * e, hipMemcpyHostToDevice));
  if (int rc = upload_gain(c, t[7], s.hidden, &L->mlp_norm)) return rc;
  if (int rc = dev_alloc(c, &L->wgu, 2 * F * H * e)) return rc;
  // interleave gate and up rows so that one wavefront computes both halves of a SwiGLU unit
  HIP_TRY(c, hipMemcpy2D(L->wgu, 2 * H * e, t[8].host_ptr, H * e, H * e, F, hipMemcpyHostToDevice));
  HIP_TRY(c, hipMemcpy2D(static_cast<char*>(L->wgu) + H * e, 2 * H * e, t[9].host_ptr, H * e, H * e, F,
                         hipMemcpyHostToDevice));
  if (int rc = dev_alloc(c, &L->wdown, H * F * e)) return rc;
  HIP_TRY(c, hipMemcpy(L->wdown, t[10].host_ptr, H * F * e, hipMemcpyHostToDevice));
  return 0;
}

// cos/sin table of rotate-half RoPE: angle = pos * theta^(-2i/D), computed in fp64, rounded
// to fp32 and, for S2, to bf16 (SGLang Day-0 Support for FishAudio S2, Engineering Appendix).
int upload_rope(s2ar_ctx* c, int D, int n_pos, float** cs, float** sn) {
  const int hd = D / 2;
  std::vector<float> vc((size_t)n_pos * hd), vs((size_t)n_pos * hd);
  for (int p = 0; p < n_pos; ++p)
    for (int i = 0; i < hd; ++i) {
      const double inv = std::pow(c->cfg.rope_theta, -2.0 * (double)i / (double)D);
      const double a = (double)p * inv;
      float fc = (float)std::cos(a), fs = (float)std::sin(a);
      if (c->cfg.rope_bf16) {
        fc = round_to_bf16(fc);
        fs = round_to_bf16(fs);
      }
      vc[(size_t)p * hd + i] = fc;
      vs[(size_t)p * hd + i] = fs;
    }
  if (int rc = dev_alloc(c, cs, sizeof(float) * vc.size())) return rc;
  if (int rc = dev_alloc(c, sn, sizeof(float) * vs.size())) return rc;
  HIP_TRY(c, hipMemcpy(*cs, vc.data(), sizeof(float) * vc.size(), hipMemcpyHostToDevice));
  HIP_TRY(c, hipMemcpy(*sn, vs.data(), sizeof(float) * vs.size(), hipMemcpyHostToDevice));
  return 0;
}

void free_ctx(s2ar_ctx* c) {
  if (!c) return;
  if (c->stream) hipStreamSynchronize(c->stream);
  for (auto& kv : c->graphs) {
    if (kv.second.exec) hipGraphExecDestroy(kv.second.exec);
    if (kv.second.g) hipGraphDestroy(kv.second.g);
  }
  for (auto& kv : c->bgraphs) {
    if (kv.second.g.exec) hipGraphExecDestroy(kv.second.g.exec);
    if (kv.second.g.g) hipGraphDestroy(kv.second.g.g);
  }
  for (const auto& b : c->dev_allocs) {
    if (c->cfg.dev_free) c->cfg.dev_free(b.first, (uint64_t)b.second, c->cfg.alloc_user);
    else hipFree(b.first);
  }
  for (void* p : c->host_allocs) hipHostFree(p);
  if (c->ev_order) hipEventDestroy(c->ev_order);
  if (c->ev_t0) hipEventDestroy(c->ev_t0);
  if (c->ev_t1) hipEventDestroy(c->ev_t1);
  if (c->stream) hipStreamDestroy(c->stream);
  delete c;
}

int create_impl(const s2ar_config* cfg, const s2ar_tensor* t, int32_t n_tensors, void* hip_stream, s2ar_ctx** out) {
  s2ar_ctx* c = new (std::nothrow) s2ar_ctx();
  if (!c) return set_err(nullptr, S2AR_E_NOMEM, "out of host memory");
  c->cfg = *cfg;
  c->bf16 = cfg->weight_dtype != 0;
  c->q8 = cfg->weight_dtype == 2 || cfg->weight_dtype == 3;
  c->f8 = cfg->weight_dtype == 3;
  c->esz = c->bf16 ? 2 : 4;
  c->user_stream = static_cast<hipStream_t>(hip_stream);
  auto fail = [&](int rc) {
    g_create_error = c->err;
    free_ctx(c);
    return rc;
  };
#define C_TRY(expr)              \
  do {                           \
    int rc_ = (expr);            \
    if (rc_) return fail(rc_);   \
  } while (0)
#define C_HIP(expr) C_TRY(([&]() -> int { HIP_TRY(c, (expr)); return 0; })())

  C_HIP(hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking));
  {
    int dev = 0, cus = 0;
    C_HIP(hipGetDevice(&dev));
    C_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    s2k::set_device_cus(cus);
  }
  {  // the device address of this device's scratch array, looked up once per device
    int dev = 0;
    C_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(set_err(c, S2AR_E_DEVICE, "device ordinal beyond 63"));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
      void* ptr = nullptr;
      C_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
      g_scratch_addr[dev] = ptr;
    }
    c->scratch_dev = static_cast<unsigned char*>(g_scratch_addr[dev]);
  }
  C_HIP(hipEventCreateWithFlags(&c->ev_order, hipEventDisableTiming));
  C_HIP(hipEventCreate(&c->ev_t0));
  C_HIP(hipEventCreate(&c->ev_t1));

  const s2ar_config& g = c->cfg;
  const int H = g.slow.hidden, NC = g.n_codebooks, K = g.codebook_size;
  const int64_t V = (int64_t)g.vocab_text + K;
  const size_t e = c->esz;

  // weights
  int ti = 0;
  C_TRY(dev_alloc(c, &c->embed, (size_t)V * H * e));
  C_HIP(hipMemcpy(c->embed, t[ti++].host_ptr, (size_t)V * H * e, hipMemcpyHostToDevice));
  c->slow.resize(g.slow.n_layers);
  for (int l = 0; l < g.slow.n_layers; ++l, ti += 11) C_TRY(upload_layer(c, g.slow, t + ti, &c->slow[l]));
  C_TRY(upload_gain(c, t[ti++], H, &c->slow_final));
  // Slow head: every row, or the semantic slice (rows vocab_text.. of the tensor) followed by the
  // stop id's row
  const bool has_eos = g.eos_id >= 0;
  c->head_rows = g.head_slice ? K + (has_eos ? 1 : 0) : (int)V;
  c->head_lo = g.head_slice ? 0 : g.vocab_text;
  c->head_eos = !has_eos ? -1 : (g.head_slice ? K : g.eos_id);
  {
    const char* hp = static_cast<const char*>(t[ti++].host_ptr);
    const size_t rb = (size_t)H * e;  // bytes of one host row
    if (c->q8) {
      std::vector<QBlock> blocks;
      if (g.head_slice) {
        blocks.push_back({hp + (size_t)g.vocab_text * rb, (size_t)K, 0, 1});
        if (has_eos) blocks.push_back({hp + (size_t)g.eos_id * rb, 1, (size_t)K, 1});
      } else {
        blocks.push_back({hp, (size_t)V, 0, 1});
      }
      C_TRY(upload_i8(c, blocks, (size_t)c->head_rows, H, &c->slow_head, &c->slow_head_s));
    } else {
      C_TRY(dev_alloc(c, &c->slow_head, (size_t)c->head_rows * rb));
      char* dh = static_cast<char*>(c->slow_head);
      if (g.head_slice) {
        C_HIP(hipMemcpy(dh, hp + (size_t)g.vocab_text * rb, (size_t)K * rb, hipMemcpyHostToDevice));
        if (has_eos) C_HIP(hipMemcpy(dh + (size_t)K * rb, hp + (size_t)g.eos_id * rb, rb, hipMemcpyHostToDevice));
      } else {
        C_HIP(hipMemcpy(dh, hp, (size_t)V * rb, hipMemcpyHostToDevice));
      }
    }
  }
  C_TRY(dev_alloc(c, &c->codebook, (size_t)NC * K * H * e));
  C_HIP(hipMemcpy(c->codebook, t[ti++].host_ptr, (size_t)NC * K * H * e, hipMemcpyHostToDevice));
  c->fast.resize(g.fast.n_layers);
  for (int l = 0; l < g.fast.n_layers; ++l, ti += 11) C_TRY(upload_layer(c, g.fast, t + ti, &c->fast[l]));
  C_TRY(upload_gain(c, t[ti++], H, &c->fast_final));
  if (c->q8) {
    C_TRY(upload_i8(c, {{t[ti++].host_ptr, (size_t)K, 0, 1}}, (size_t)K, H, &c->fast_head, &c->fast_head_s));
  } else {
    C_TRY(dev_alloc(c, &c->fast_head, (size_t)K * H * e));
    C_HIP(hipMemcpy(c->fast_head, t[ti++].host_ptr, (size_t)K * H * e, hipMemcpyHostToDevice));
  }
  C_TRY(upload_rope(c, g.slow.head_dim, g.max_context, &c->rope_cos_s, &c->rope_sin_s));
  C_TRY(upload_rope(c, g.fast.head_dim, NC - 1, &c->rope_cos_f, &c->rope_sin_f));

  // KV pools
  c->bt_stride = (g.max_context + kPageSize - 1) / kPageSize;
  c->n_pages = c->bt_stride * g.max_streams;
  c->k_bf16 = g.kv_dtype == 1 || g.kv_dtype == 2;
  c->v_bf16 = g.kv_dtype == 1 || g.kv_dtype == 3;
  {
    const size_t slow_elems = (size_t)c->n_pages * g.slow.n_kv_heads * kPageSize * g.slow.head_dim;
    const size_t fast_elems = (size_t)g.max_streams * g.fast.n_kv_heads * kPageSize * g.fast.head_dim;
    c->kv_layer_k = slow_elems * (c->k_bf16 ? 2 : 4);
    c->kv_layer_v = slow_elems * (c->v_bf16 ? 2 : 4);
    c->fkv_layer_k = fast_elems * (c->k_bf16 ? 2 : 4);
    c->fkv_layer_v = fast_elems * (c->v_bf16 ? 2 : 4);
  }
  C_TRY(dev_alloc(c, &c->kv_k, c->kv_layer_k * g.slow.n_layers));
  C_TRY(dev_alloc(c, &c->kv_v, c->kv_layer_v * g.slow.n_layers));
  C_TRY(dev_alloc(c, &c->fkv_k, c->fkv_layer_k * g.fast.n_layers));
  C_TRY(dev_alloc(c, &c->fkv_v, c->fkv_layer_v * g.fast.n_layers));
  C_TRY(dev_alloc(c, &c->d_bt, sizeof(int) * c->n_pages));
  C_TRY(host_alloc(c, &c->h_bt, sizeof(int) * c->n_pages));
  {
    std::vector<int> ids(g.max_streams), fpos((size_t)(NC - 1) * g.max_streams);
    for (int s = 0; s < g.max_streams; ++s) ids[s] = s;
    for (int j = 0; j < NC - 1; ++j)
      for (int s = 0; s < g.max_streams; ++s) fpos[(size_t)j * g.max_streams + s] = j;
    C_TRY(dev_alloc(c, &c->d_fast_bt, sizeof(int) * g.max_streams));
    C_HIP(hipMemcpy(c->d_fast_bt, ids.data(), sizeof(int) * g.max_streams, hipMemcpyHostToDevice));
    C_TRY(dev_alloc(c, &c->d_slot_ids, sizeof(int) * g.max_streams));
    C_HIP(hipMemcpy(c->d_slot_ids, ids.data(), sizeof(int) * g.max_streams, hipMemcpyHostToDevice));
    C_TRY(dev_alloc(c, &c->d_fast_pos, sizeof(int) * fpos.size()));
    C_HIP(hipMemcpy(c->d_fast_pos, fpos.data(), sizeof(int) * fpos.size(), hipMemcpyHostToDevice));
  }
  // pages are handed out in a scrambled order so that a stream's pages are never contiguous
  c->free_pages.resize(c->n_pages);
  for (int i = 0; i < c->n_pages; ++i) c->free_pages[i] = i;
  {
    uint64_t st = 0x2545F4914F6CDD1DULL;
    for (int i = c->n_pages - 1; i > 0; --i) {
      st ^= st << 13;
      st ^= st >> 7;
      st ^= st << 17;
      const int j = (int)(st % (uint64_t)(i + 1));
      std::swap(c->free_pages[i], c->free_pages[j]);
    }
  }
  c->stream_pages.assign(g.max_streams, {});
  for (auto& sp : c->stream_pages) sp.reserve(c->bt_stride);  // appends never reallocate
  c->page_refs.assign(c->n_pages, 0);

  // state
  C_TRY(dev_alloc(c, &c->d_pos, sizeof(int) * g.max_streams));
  C_TRY(dev_alloc(c, &c->d_codes, sizeof(int) * g.max_streams * NC));
  C_TRY(dev_alloc(c, &c->d_h, sizeof(float) * (size_t)g.max_streams * H));
  C_TRY(dev_alloc(c, &c->d_snap, sizeof(int) * g.max_streams * NC));
  C_TRY(dev_alloc(c, &c->d_sink, sizeof(uint32_t)));
  c->pos.assign(g.max_streams, 0);
  c->ready.assign(g.max_streams, 0);
  c->ended.assign(g.max_streams, 0);

  // workspace
  const int qkvd = (g.slow.n_q_heads + 2 * g.slow.n_kv_heads) * g.slow.head_dim;
  const int qkvf = (g.fast.n_q_heads + 2 * g.fast.n_kv_heads) * g.fast.head_dim;
  const int qd = std::max(g.slow.n_q_heads * g.slow.head_dim, g.fast.n_q_heads * g.fast.head_dim);
  const int F = std::max(g.slow.ffn, g.fast.ffn);
  C_TRY(dev_alloc(c, &c->x, sizeof(float) * s2k::pad_k(H)));
  C_TRY(dev_alloc(c, &c->xf, sizeof(float) * (size_t)g.max_streams * s2k::pad_k(H)));
  C_TRY(dev_alloc(c, &c->z, sizeof(float) * s2k::pad_k(H)));
  C_TRY(dev_alloc(c, &c->qkv, sizeof(float) * std::max(qkvd, qkvf)));
  C_TRY(dev_alloc(c, &c->att, sizeof(float) * s2k::pad_k(qd)));
  C_TRY(dev_alloc(c, &c->act, sizeof(float) * s2k::pad_k(F)));
  C_TRY(dev_alloc(c, &c->slow_logits, sizeof(float) * V));
  C_TRY(dev_alloc(c, &c->fast_logits, sizeof(float) * K));
  const int nb = std::max(s2k::gemv_blocks(s2k::GEMV_NORM_ARGMAX, (int)V), s2k::gemv_blocks(s2k::GEMV_NORM_ARGMAX, K));
  C_TRY(dev_alloc(c, &c->am_val, sizeof(float) * nb));
  C_TRY(dev_alloc(c, &c->am_idx, sizeof(int) * nb));
  c->max_splits = (g.max_context + kAttnSplit - 1) / kAttnSplit;
  const int hq = std::max(g.slow.n_q_heads, g.fast.n_q_heads);
  const int dmax = std::max(g.slow.head_dim, g.fast.head_dim);
  C_TRY(dev_alloc(c, &c->att_ml, sizeof(float) * 2 * hq * c->max_splits));
  C_TRY(dev_alloc(c, &c->att_o, sizeof(float) * (size_t)hq * c->max_splits * dmax));
  C_TRY(dev_alloc(c, &c->d_tokens, sizeof(int) * g.max_context));
  C_TRY(dev_alloc(c, &c->d_mask, (size_t)g.max_context));
  C_TRY(dev_alloc(c, &c->d_pcodes, sizeof(int) * (size_t)g.max_context * NC));

  // batched prefill on the matrix cores when the shapes allow it (bf16, N % 128, K % 32)
  {
    const s2ar_stack& st = g.slow;
    const int qkvd_s = (st.n_q_heads + 2 * st.n_kv_heads) * st.head_dim, qd_s = st.n_q_heads * st.head_dim;
    // 8-bit weights need every K a multiple of 64 (the 8-wavefront GEMM only)
    const int kmul = c->q8 ? 64 : 32;
    c->mfma_prefill = c->bf16 && qkvd_s % 128 == 0 && H % 128 == 0 && (2 * st.ffn) % 128 == 0 && H % kmul == 0 &&
                      qd_s % kmul == 0 && st.ffn % kmul == 0;
    if (c->mfma_prefill) {
      c->pch = std::min(g.max_context, 2048);
      C_TRY(dev_alloc(c, &c->px, sizeof(float) * (size_t)c->pch * H));
      {
        const int nsp = s2k::prefill_attn_splits(c->pch, g.max_context - c->pch, kPrefillAttnTiles);
        C_TRY(dev_alloc(c, &c->patt_o, sizeof(float) * (size_t)nsp * c->pch * qd_s));
        C_TRY(dev_alloc(c, &c->patt_ml, sizeof(float) * 2 * (size_t)nsp * c->pch * st.n_q_heads));
      }
      C_TRY(dev_alloc(c, &c->pqkv, sizeof(float) * (size_t)c->pch * qkvd_s));
      C_TRY(dev_alloc(c, &c->pxh, sizeof(uint16_t) * (size_t)c->pch * H));
      C_TRY(dev_alloc(c, &c->pxl, sizeof(uint16_t) * (size_t)c->pch * H));
      C_TRY(dev_alloc(c, &c->patth, sizeof(uint16_t) * (size_t)c->pch * qd_s));
      C_TRY(dev_alloc(c, &c->pattl, sizeof(uint16_t) * (size_t)c->pch * qd_s));
      C_TRY(dev_alloc(c, &c->pacth, sizeof(uint16_t) * (size_t)c->pch * st.ffn));
      C_TRY(dev_alloc(c, &c->pactl, sizeof(uint16_t) * (size_t)c->pch * st.ffn));
      c->pgemm_part_floats = (size_t)4 * 256 * std::max(std::max(qkvd_s, 2 * st.ffn), H);
      C_TRY(dev_alloc(c, &c->pgemm_part, sizeof(float) * c->pgemm_part_floats));
      C_TRY(dev_alloc(c, &c->d_range, 256));
      c->f16_prefill_ok = H % 64 == 0 && qd_s % 64 == 0 && st.ffn % 64 == 0;
      std::vector<int> iota(g.max_context);
      for (int i = 0; i < g.max_context; ++i) iota[i] = i;
      C_TRY(dev_alloc(c, &c->d_iota, sizeof(int) * g.max_context));
      C_HIP(hipMemcpy(c->d_iota, iota.data(), sizeof(int) * g.max_context, hipMemcpyHostToDevice));
    }
  }
  C_TRY(host_alloc(c, &c->h_pos_stage, sizeof(int) * 16));

  // batched decode buffers (bf16 weights, every K a multiple of 512)
  {
    auto k_ok = [](const s2ar_stack& st) {
      return st.hidden % 512 == 0 && (st.n_q_heads * st.head_dim) % 512 == 0 && st.ffn % 512 == 0;
    };
    c->batched_ok = c->bf16 && g.max_streams > 1 && k_ok(g.slow) && k_ok(g.fast);
    if (c->batched_ok) {
      const int MBt = 16;
      const int qkvd_max = std::max((g.slow.n_q_heads + 2 * g.slow.n_kv_heads) * g.slow.head_dim,
                                    (g.fast.n_q_heads + 2 * g.fast.n_kv_heads) * g.fast.head_dim);
      const int qd_max = std::max(g.slow.n_q_heads * g.slow.head_dim, g.fast.n_q_heads * g.fast.head_dim);
      const int f_max = std::max(g.slow.ffn, g.fast.ffn);
      C_TRY(dev_alloc(c, &c->bx, sizeof(float) * MBt * s2k::pad_k(H)));
      C_TRY(dev_alloc(c, &c->bxf, sizeof(float) * MBt * s2k::pad_k(H)));
      C_TRY(dev_alloc(c, &c->bqkv, sizeof(float) * MBt * qkvd_max));
      C_TRY(dev_alloc(c, &c->batt, sizeof(float) * MBt * qd_max));
      C_TRY(dev_alloc(c, &c->bact, sizeof(float) * MBt * f_max));
      C_TRY(dev_alloc(c, &c->blogits, sizeof(float) * MBt * V));
      C_TRY(dev_alloc(c, &c->bxn, sizeof(float) * MBt * s2k::pad_k(H)));
      C_TRY(dev_alloc(c, &c->bssq, sizeof(float) * MBt * s2k::fold_chunks(H)));
      c->bpart_floats = (size_t)32 * MBt * std::max(std::max(qkvd_max, (int)K), std::max(H, 2 * f_max));
      C_TRY(dev_alloc(c, &c->bpart, sizeof(float) * c->bpart_floats));
      const int ngroups = 4 * s2k::mgemv_tiles((int)V);  // 16-row argmax groups
      C_TRY(dev_alloc(c, &c->bam_val, sizeof(float) * (size_t)ngroups * MBt));
      C_TRY(dev_alloc(c, &c->bam_idx, sizeof(int) * (size_t)ngroups * MBt));
      // tiled weight copies for the batched GEMVs; dev_alloc zeroes on the null stream, which the
      // non-blocking engine stream does not wait for, so every buffer is allocated (and the device
      // synchronised) before the tiling kernels run
      struct TileJob {
        const void* src;
        int N, K;
        void** dst;
      };
      std::vector<TileJob> jobs;
      for (int pass = 0; pass < 2; ++pass) {
        const s2ar_stack& st = pass ? g.fast : g.slow;
        std::vector<LayerW>& W = pass ? c->fast : c->slow;
        const int qd = st.n_q_heads * st.head_dim, qkvd = (st.n_q_heads + 2 * st.n_kv_heads) * st.head_dim;
        for (LayerW& L : W) {
          jobs.push_back({L.wqkv, qkvd, st.hidden, &L.tqkv});
          jobs.push_back({L.wo, st.hidden, qd, &L.to});
          jobs.push_back({L.wgu, 2 * st.ffn, st.hidden, &L.tgu});
          jobs.push_back({L.wdown, st.hidden, st.ffn, &L.tdown});
        }
      }
      jobs.push_back({c->slow_head, c->head_rows, H, &c->slow_head_t});
      jobs.push_back({c->fast_head, K, H, &c->fast_head_t});
      const size_t wesz = c->q8 ? 1 : 2;  // bytes per tiled element
      for (const TileJob& j : jobs) C_TRY(dev_alloc(c, j.dst, wesz * s2k::tiled_weight_elems(j.N, j.K)));
      C_HIP(hipDeviceSynchronize());
      for (const TileJob& j : jobs) {
        if (c->q8)
          C_HIP(s2k::launch_tile_weights8(static_cast<const uint8_t*>(j.src), static_cast<uint8_t*>(*j.dst), j.N, j.K,
                                          c->stream));
        else
          C_HIP(s2k::launch_tile_weights(static_cast<const uint16_t*>(j.src), static_cast<uint16_t*>(*j.dst), j.N, j.K,
                                         c->stream));
      }
      C_HIP(hipStreamSynchronize(c->stream));
#ifndef S2AR_ATTN_LONG
#define S2AR_ATTN_LONG 1
#endif
      c->attn_long = S2AR_ATTN_LONG && s2k::attention_long_supports(g.slow.head_dim, g.slow.n_q_heads, g.slow.n_kv_heads);
      if (c->attn_long) c->attn_split_b = 256;
      c->max_splits_b = (g.max_context + c->attn_split_b - 1) / c->attn_split_b;
      C_TRY(dev_alloc(c, &c->batt_ml, sizeof(float) * 2 * MBt * hq * c->max_splits_b));
      C_TRY(dev_alloc(c, &c->batt_o, sizeof(float) * (size_t)MBt * hq * c->max_splits_b * dmax));
      C_TRY(dev_alloc(c, &c->d_dbg_slots, sizeof(int) * MBt));
    }
  }

  c->h_codes_frames = 64;
  C_TRY(host_alloc(c, &c->h_codes, sizeof(int) * (size_t)c->h_codes_frames * g.max_streams * NC));
  const int Lf = g.fast.n_layers;
  c->h_taps_floats = (size_t)H + (size_t)g.slow.n_layers * H + H + V + (size_t)(NC - 1) * Lf * H +
                     (size_t)(NC - 1) * H + (size_t)(NC - 1) * K;
  C_TRY(host_alloc(c, &c->h_taps, sizeof(float) * c->h_taps_floats));
  C_TRY(host_alloc(c, &c->h_small, sizeof(int) * 4 * NC));
  C_HIP(hipDeviceSynchronize());
  *out = c;
  return S2AR_OK;
#undef C_TRY
#undef C_HIP
}

// ------------------------------------------------------------------------------- frame pieces

struct TapPlan {  // host destinations inside h_taps (nullptr = not wanted)
  float *embed = nullptr, *slow_resid = nullptr, *slow_h = nullptr, *slow_logits = nullptr;
  float *fast_resid = nullptr, *fast_z = nullptr, *fast_logits = nullptr;
  int* own = nullptr;       // [NC]
  int* next_c0 = nullptr;   // [1]
  const int* forced = nullptr;  // pinned copy of the forced codes [NC]
};

struct Enq {
  s2ar_ctx* c;
  hipStream_t s;
  hipError_t e = hipSuccess;
  // scratch of the frame's kernels: greedy-pick partials and Slow attention split partials (the
  // context's workspace, or the file-scope scratch array of the allocation-free entry point)
  float* ws_am_val = c->am_val;
  int* ws_am_idx = c->am_idx;
  float* ws_att_ml = c->att_ml;
  float* ws_att_o = c->att_o;
  // Slow attention: positions per workgroup and grid extent along the context (splits past the
  // stream's context exit at once); a merge launch follows when slow_max_splits > 1
  int slow_split = kAttnSplit;
  int slow_max_splits = c->max_splits;
  // the split rule of a frame whose Slow step attends over ctx positions; exact: a grid of exactly
  // the splits needed (eager frames), else the context's capacity (a captured graph serves every
  // context of its bucket)
  void set_slow_ctx(int ctx, bool exact) {
    const SlowSplit ss = slow_split_for(ctx);
    slow_split = ss.split;
    slow_max_splits = ss.nsplit == 1 ? 1 : (exact ? ss.nsplit : c->max_splits);
  }
  void chk(hipError_t r) {
    if (e == hipSuccess && r != hipSuccess) e = r;
  }
  void d2h(void* dst, const void* src, size_t bytes) {
    chk(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s));
  }
  void h2d(void* dst, const void* src, size_t bytes) {
    chk(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s));
  }

  void gemv(int kind, const void* w, const float* wscale, const float* x, const float* gain, float* y, int N, int K,
            float* xnorm_out = nullptr, int lo = 0, int hi = 0, int* code_out = nullptr) {
    s2k::GemvArgs a{};
    a.w = w;
    a.wscale = wscale;
    a.w_f8 = c->f8 ? 1 : 0;
    a.x = x;
    a.gain = gain;
    a.eps = (float)c->cfg.rms_eps;
    a.y = y;
    a.xnorm_out = xnorm_out;
    a.N = N;
    a.K = K;
    a.am_lo = lo;
    a.am_hi = hi;
    a.am_val = ws_am_val;
    a.am_idx = ws_am_idx;
    chk(s2k::launch_gemv(kind, c->bf16, a, s));
  }

  float* xf_of(int slot) const { return c->xf + (size_t)slot * s2k::pad_k(c->cfg.slow.hidden); }

  // The input of the next Fast step (the codebook row of the previous step's pick), gathered by that
  // step's first QKV GEMV: the pick's second pass runs there, behind the GEMV's first weight loads,
  // instead of in a finisher launch of its own.  (The Slow step's input, a sum of ten rows, stays
  // with its finisher: every GEMV block would gather all ten.)
  struct PickIn {
    bool on = false;
    int j = 0, slot = 0;
  } pick_in;
  bool pick_fits() const {
    const s2ar_config& g = c->cfg;
    return c->bf16 && s2k::gemv_pick_fits(g.fast.hidden, (g.codebook_size - 1) / s2k::argmax_block_rows() + 1);
  }

  // pass 2 of a head's greedy pick over rows [lo, hi), then the step's bookkeeping
  void finish(int mode, int j, int slot, int lo, int hi, float* x) {
    const s2ar_config& g = c->cfg;
    const int rb = s2k::argmax_block_rows();
    s2k::FinishArgs f{};
    f.am_val = ws_am_val;
    f.am_idx = ws_am_idx;
    f.b0 = lo / rb;
    f.b1 = (hi - 1) / rb;
    f.lo = lo;
    f.mode = mode;
    f.j = j;
    f.codes = c->d_codes + (size_t)slot * g.n_codebooks;
    f.snap = c->d_snap + (size_t)slot * g.n_codebooks;
    f.pos = c->d_pos + slot;
    f.codebook = c->codebook;
    f.h = c->d_h + (size_t)slot * g.slow.hidden;
    f.x = x;
    f.H = g.slow.hidden;
    f.K = g.codebook_size;
    f.NC = g.n_codebooks;
    f.logits = c->slow_logits;
    f.eos_at = mode == s2k::FIN_SLOW ? c->head_eos : -1;
    chk(s2k::launch_finish(c->bf16, f, s));
  }

  // one stack of layers on the residual `x` of batch row 0 (stream slot `slot`)
  void layers(bool is_slow, int slot, float* x, float* resid_tap) {
    const s2ar_stack& st = is_slow ? c->cfg.slow : c->cfg.fast;
    const std::vector<LayerW>& W = is_slow ? c->slow : c->fast;
    const int H = st.hidden, D = st.head_dim, qd = st.n_q_heads * D;
    const int qkvd = (st.n_q_heads + 2 * st.n_kv_heads) * D;
    for (int l = 0; l < st.n_layers; ++l) {
      const LayerW& L = W[l];
      if (!is_slow && l == 0 && pick_in.on) {
        const s2ar_config& g = c->cfg;
        s2k::GemvArgs a{};
        a.w = L.wqkv;
        a.wscale = L.sqkv;
        a.w_f8 = c->f8 ? 1 : 0;
        a.gain = L.attn_norm;
        a.eps = (float)g.rms_eps;
        a.y = c->qkv;
        a.N = qkvd;
        a.K = H;
        a.pk_val = ws_am_val;
        a.pk_idx = ws_am_idx;
        a.pk_b0 = 0;  // the Fast head's rows [0, codebook_size)
        a.pk_n = (g.codebook_size - 1) / s2k::argmax_block_rows() + 1;
        a.pk_lo = 0;
        a.pk_codebook = static_cast<const uint16_t*>(c->codebook);
        a.pk_ncb = g.codebook_size;
        a.pk_j = pick_in.j;
        a.pk_codes = c->d_codes + (size_t)pick_in.slot * g.n_codebooks;
        a.pk_x = x;
        chk(s2k::launch_gemv_pick(a, s));
        pick_in.on = false;
      } else {
        gemv(s2k::GEMV_NORM_STORE, L.wqkv, L.sqkv, x, L.attn_norm, c->qkv, qkvd, H);
      }
      s2k::AttnArgs a{};
      a.qkv = c->qkv;
      a.q_norm = L.q_norm;
      a.k_norm = L.k_norm;
      a.slots = c->d_slot_ids + slot;
      a.M = 1;
      a.Hq = st.n_q_heads;
      a.Hkv = st.n_kv_heads;
      a.D = D;
      a.page_size = kPageSize;
      a.eps = (float)c->cfg.rms_eps;
      a.scale = (float)(1.0 / std::sqrt((double)D));
      a.out = c->att;
      a.part_ml = ws_att_ml;
      a.part_o = ws_att_o;
      a.k_bf16 = c->k_bf16;
      a.v_bf16 = c->v_bf16;
      a.split = is_slow ? slow_split : kAttnSplit;
      a.fixed_slot = slot;  // a frame graph belongs to one stream: no slot lookup on the device
      a.row_pos = nullptr;
      a.append = 1;
      a.const_pos = is_slow ? -1 : fast_step - 1;
      if (is_slow) {
        a.rope_cos = c->rope_cos_s;
        a.rope_sin = c->rope_sin_s;
        a.pos = c->d_pos;
        a.k_cache = c->kv_k + (size_t)l * c->kv_layer_k;
        a.v_cache = c->kv_v + (size_t)l * c->kv_layer_v;
        a.block_table = c->d_bt;
        a.bt_stride = c->bt_stride;
        a.max_splits = slow_max_splits;
      } else {
        a.rope_cos = c->rope_cos_f;
        a.rope_sin = c->rope_sin_f;
        a.pos = fast_pos_ptr;
        a.k_cache = c->fkv_k + (size_t)l * c->fkv_layer_k;
        a.v_cache = c->fkv_v + (size_t)l * c->fkv_layer_v;
        a.block_table = c->d_fast_bt;
        a.bt_stride = 1;
        a.max_splits = 1;
      }
      chk(s2k::launch_attention(a, s));
      if (a.max_splits > 1) chk(s2k::launch_attention_combine(a, s));
      gemv(s2k::GEMV_RESID, L.wo, L.so, c->att, nullptr, x, H, qd);
      gemv(s2k::GEMV_NORM_SWIGLU, L.wgu, L.sgu, x, L.mlp_norm, c->act, 2 * st.ffn, H);
      gemv(s2k::GEMV_RESID, L.wdown, L.sdown, c->act, nullptr, x, H, st.ffn);
      if (resid_tap) d2h(resid_tap + (size_t)l * H, x, sizeof(float) * H);
    }
  }
  const int* fast_pos_ptr = nullptr;
  int fast_step = 1;  // the Fast step j whose layers are being enqueued (position j - 1)

  // Slow final norm + head + constrained argmax -> codes[slot][0] and h[slot]; the finisher
  // also copies h into the Fast input and advances the stream's position
  void slow_head(int slot, const TapPlan* tp) {
    const s2ar_config& g = c->cfg;
    const int H = g.slow.hidden, V = g.vocab_text + g.codebook_size;
    const int lo = c->head_lo, K = g.codebook_size;
    gemv(s2k::GEMV_NORM_ARGMAX, c->slow_head, c->slow_head_s, c->x, c->slow_final, c->slow_logits, c->head_rows, H,
         c->d_h + (size_t)slot * H, lo, lo + K);
    finish(s2k::FIN_SLOW, 0, slot, lo, lo + K, xf_of(slot));
    if (tp && tp->slow_h) d2h(tp->slow_h, c->d_h + (size_t)slot * H, sizeof(float) * H);
    if (tp && tp->slow_logits) {
      if (g.head_slice) {  // the tap keeps full-vocabulary indexing; the rows not computed stay NaN
        d2h(tp->slow_logits + g.vocab_text, c->slow_logits, sizeof(float) * K);
        if (g.eos_id >= 0) d2h(tp->slow_logits + g.eos_id, c->slow_logits + K, sizeof(float));
      } else {
        d2h(tp->slow_logits, c->slow_logits, sizeof(float) * V);
      }
    }
    if (tp && tp->next_c0) d2h(tp->next_c0, c->d_codes + (size_t)slot * g.n_codebooks, sizeof(int));
  }

  // The 9 greedy Fast AR steps of stream `slot` on h[slot] (already copied into xf by the Slow
  // finisher).  Without taps, each step's finisher gathers the next step's input (or, after the
  // last step, the Slow input of the frame's ten codes); with taps the inputs are gathered by
  // separate kernels after any forced code has been written.
  void fast_loop(int slot, const TapPlan* tp) {
    const s2ar_config& g = c->cfg;
    const int H = g.fast.hidden, K = g.codebook_size, NC = g.n_codebooks, Lf = g.fast.n_layers;
    int* codes = c->d_codes + (size_t)slot * NC;
    for (int j = 1; j < NC; ++j) {
      float* xf = xf_of(slot);
      if (tp)
        chk(s2k::launch_fast_input(c->bf16, c->codebook, c->d_h, K, H, NC, c->d_slot_ids + slot, c->d_codes, j, xf,
                                   H, 1, s));
      fast_pos_ptr = c->d_fast_pos + (size_t)(j - 1) * g.max_streams;
      fast_step = j;
      layers(false, slot, xf, tp && tp->fast_resid ? tp->fast_resid + (size_t)(j - 1) * Lf * H : nullptr);
      gemv(s2k::GEMV_NORM_ARGMAX, c->fast_head, c->fast_head_s, xf, c->fast_final, c->fast_logits, K, H,
           tp && tp->fast_z ? c->z : nullptr, 0, K);
      const int mode = tp ? s2k::FIN_CODE : (j < NC - 1 ? s2k::FIN_FAST_NEXT : s2k::FIN_FAST_LAST);
      if (mode == s2k::FIN_FAST_NEXT && pick_fits()) {
        pick_in.on = true;  // the next step's first QKV GEMV picks code j and gathers its input
        pick_in.j = j;
        pick_in.slot = slot;
      } else {
        finish(mode, j, slot, 0, K, j < NC - 1 ? xf : c->x);
      }
      if (tp && tp->fast_z) d2h(tp->fast_z + (size_t)(j - 1) * H, c->z, sizeof(float) * H);
      if (tp && tp->fast_logits) d2h(tp->fast_logits + (size_t)(j - 1) * K, c->fast_logits, sizeof(float) * K);
      if (tp && tp->own) d2h(tp->own + j, codes + j, sizeof(int));
      if (tp && tp->forced) h2d(codes + j, tp->forced + j, sizeof(int));
    }
  }

  // Slow step on the frame's codes: the input (sum of the ten codebook rows) and the snapshot
  // of the codes come from the last Fast finisher, or from an explicit gather with taps.
  void slow_step(int slot, const TapPlan* tp) {
    const s2ar_config& g = c->cfg;
    if (tp) {
      chk(s2k::launch_embed_codes(c->bf16, c->codebook, g.codebook_size, g.slow.hidden, g.n_codebooks,
                                  c->d_slot_ids + slot, c->d_codes, c->d_snap, c->x, g.slow.hidden, 1, s));
      if (tp->embed) d2h(tp->embed, c->x, sizeof(float) * g.slow.hidden);
    }
    layers(true, slot, c->x, tp ? tp->slow_resid : nullptr);
    slow_head(slot, tp);
  }

  // Prefill `rows` prompt rows (prompt indices p0.., positions pos0..) of stream `slot` on the
  // matrix cores: every projection is one bf16 MFMA GEMM over all rows, the keys and values of
  // the rows are appended first, then each row attends causally over the cache.
  void prefill_rows(int slot, int p0, int pos0, int rows, bool has_mask) {
    const s2ar_config& g = c->cfg;
    const s2ar_stack& st = g.slow;
    const int H = st.hidden, D = st.head_dim, qd = st.n_q_heads * D, F = st.ffn;
    const int qkvd = (st.n_q_heads + 2 * st.n_kv_heads) * D;
    const float eps = (float)g.rms_eps;
    chk(s2k::launch_embed_rows(c->bf16, c->embed, c->codebook, g.codebook_size, H, g.n_codebooks, c->d_tokens,
                               has_mask ? c->d_mask : nullptr, c->d_pcodes, p0, rows, c->px, H, s));
    // the fp16 mode writes and reads one activation plane (the lo planes stay unused)
    const bool f16 = c->prefill_f16;
    uint16_t* const pxl = f16 ? nullptr : c->pxl;
    uint16_t* const pattl = f16 ? nullptr : c->pattl;
    uint16_t* const pactl = f16 ? nullptr : c->pactl;
    auto gemm = [&](const uint16_t* a_hi, const uint16_t* a_lo, int lda, const void* w, const float* wscale, float* out,
                    uint16_t* out_hi, uint16_t* out_lo, int ldc, int N, int K, int epi) {
      s2k::GemmArgs ga{};
      ga.a_hi = a_hi;
      ga.a_lo = a_lo;
      ga.lda = lda;
      ga.w = w;
      ga.wscale = wscale;
      ga.w_fmt = !c->q8 ? s2k::W_BF16 : (c->f8 ? s2k::W_F8 : s2k::W_I8);
      ga.c = out;
      ga.c_hi = out_hi;
      ga.c_lo = out_lo;
      ga.ldc = ldc;
      ga.M = rows;
      ga.N = N;
      ga.K = K;
      ga.epi = epi;
      ga.part = c->pgemm_part;
      ga.part_floats = c->pgemm_part_floats;
      ga.a_f16 = f16;
      ga.range_flag = c->d_range;
      chk(s2k::launch_gemm(ga, s));
    };
    for (int l = 0; l < st.n_layers; ++l) {
      const LayerW& L = c->slow[l];
      chk(s2k::launch_norm_split(c->px, H, H, eps, L.attn_norm, c->pxh, pxl, H, rows, c->d_range, s));
      gemm(c->pxh, pxl, H, L.wqkv, L.sqkv, c->pqkv, nullptr, nullptr, qkvd, qkvd, H, s2k::GEMM_STORE);
      s2k::PrefillKvArgs kv{};
      kv.qkv = c->pqkv;
      kv.ld = qkvd;
      kv.k_norm = L.k_norm;
      kv.rope_cos = c->rope_cos_s;
      kv.rope_sin = c->rope_sin_s;
      kv.k_cache = c->kv_k + (size_t)l * c->kv_layer_k;
      kv.v_cache = c->kv_v + (size_t)l * c->kv_layer_v;
      kv.k_bf16 = c->k_bf16;
      kv.v_bf16 = c->v_bf16;
      kv.block_table = c->d_bt + (size_t)slot * c->bt_stride;
      kv.page_size = kPageSize;
      kv.pos0 = pos0;
      kv.Hq = st.n_q_heads;
      kv.Hkv = st.n_kv_heads;
      kv.D = D;
      kv.eps = eps;
      chk(s2k::launch_prefill_append(kv, rows, s));
      s2k::PrefillAttnArgs pa{};
      pa.qkv = c->pqkv;
      pa.ld = qkvd;
      pa.q_norm = L.q_norm;
      pa.rope_cos = c->rope_cos_s;
      pa.rope_sin = c->rope_sin_s;
      pa.k_cache = kv.k_cache;
      pa.v_cache = kv.v_cache;
      pa.k_bf16 = kv.k_bf16;
      pa.v_bf16 = kv.v_bf16;
      pa.block_table = kv.block_table;
      pa.page_size = kPageSize;
      pa.out_hi = c->patth;
      pa.out_lo = pattl;
      pa.range_flag = c->d_range;
      pa.ld_out = qd;
      pa.rows = rows;
      pa.pos0 = pos0;
      pa.Hq = st.n_q_heads;
      pa.Hkv = st.n_kv_heads;
      pa.D = D;
      pa.eps = eps;
      pa.scale = (float)(1.0 / std::sqrt((double)D));
      pa.tps = kPrefillAttnTiles;
      pa.part_o = c->patt_o;
      pa.part_ml = c->patt_ml;
      chk(s2k::launch_prefill_attn(pa, s));
      gemm(c->patth, pattl, qd, L.wo, L.so, c->px, nullptr, nullptr, H, H, qd, s2k::GEMM_ADD);
      chk(s2k::launch_norm_split(c->px, H, H, eps, L.mlp_norm, c->pxh, pxl, H, rows, c->d_range, s));
      gemm(c->pxh, pxl, H, L.wgu, L.sgu, nullptr, c->pacth, pactl, F, 2 * F, H, s2k::GEMM_SWIGLU);
      gemm(c->pacth, pactl, F, L.wdown, L.sdown, c->px, nullptr, nullptr, H, H, F, s2k::GEMM_ADD);
    }
  }

  // ---- batched decode of M <= 16 streams (slots on the device in `slots`) ----
  // Optional per-stream host destinations for the test-only eager batched frame.
  struct BTap {
    float *slow_resid = nullptr, *slow_h = nullptr, *slow_logits = nullptr, *fast_resid = nullptr;
    float* fast_logits = nullptr;
    int *own = nullptr, *next_c0 = nullptr;
    const int* forced = nullptr;  // pinned [NC] or nullptr
  };
  const BTap* btp = nullptr;  // [M] when running the eager batched frame
  const int* bslots_host = nullptr;
  // returns the number of K splits; an MG_ADD launch leaves that many partials in bpart for the
  // next norm_b to fold into the residual
  // norm_gain != nullptr: the input rows are RMS-normalised on the fly with the sums of squares
  // that fold_b left in bssq
  int mgemv(int epi, const void* w, const float* wscale, const float* x, int ldx, float* out, int ldo, int N, int K,
            int M, int lo = 0, int hi = 0, const float* norm_gain = nullptr) {
    s2k::MgemvArgs a{};
    a.x = x;
    a.ldx = ldx;
    a.w = w;
    a.wscale = wscale;
    a.w_fmt = !c->q8 ? s2k::W_BF16 : (c->f8 ? s2k::W_F8 : s2k::W_I8);
    a.out = out;
    a.ldo = ldo;
    a.part = c->bpart;
    a.M = M;
    a.N = N;
    a.K = K;
    a.epi = epi;
    a.am_lo = lo;
    a.am_hi = hi;
    a.am_val = c->bam_val;
    a.am_idx = c->bam_idx;
    // Work split.  Every launch but the Slow head takes one 512-wide K chunk per item (S = K / 512,
    // the straight-line split-K kernel) with about one block per CU; the Slow head (many tiles)
    // keeps whole rows per item so that the greedy pick stays in the kernel.
    const int tiles = s2k::mgemv_tiles(N), chunks = K / 512;
    if (norm_gain) {
      a.ssq = c->bssq;
      a.nssq = s2k::fold_chunks(K);
      a.gain = norm_gain;
      a.eps = (float)c->cfg.rms_eps;
    }
    if (epi == s2k::MG_ARGMAX && tiles >= 512 && !norm_gain) {
      a.S = 1;
      a.ipb = 1;
    } else {
      a.S = chunks;
      a.ipb = std::max(1, (tiles * chunks + s2k::device_cus() - 1) / s2k::device_cus());
    }
    chk(s2k::launch_mgemv(a, s));
    return a.S;
  }

  // fold `pending` residual partials into xres and leave the per-chunk sums of squares in bssq
  void fold_b(float* xres, int& pending, int H, int M) {
    s2k::FoldArgs f{};
    f.x = xres;
    f.ldx = s2k::pad_k(c->cfg.slow.hidden);
    f.part = c->bpart;
    f.S = pending;
    f.M = M;
    f.H = H;
    f.ssq = c->bssq;
    chk(s2k::launch_fold_rows(f, s));
    pending = 0;
  }

  // fold `pending` residual partials into xres, then bxn = RMSNorm(xres) * gain (gain == nullptr:
  // fold only)
  void norm_b(float* xres, int& pending, int H, int M, const float* gain) {
    s2k::NormRowsArgs n{};
    n.x = xres;
    n.ldx = s2k::pad_k(c->cfg.slow.hidden);
    n.part = c->bpart;
    n.S = pending;
    n.M = M;
    n.H = H;
    n.gain = gain;
    n.eps = (float)c->cfg.rms_eps;
    n.xn = gain ? c->bxn : nullptr;
    chk(s2k::launch_norm_rows(n, s));
    pending = 0;
  }

  // leaves the last down projection's partials pending (returned) for the final norm
  int layers_b(bool is_slow, int M, const int* slots, float* xres) {
    int pending = 0;
    const s2ar_config& g = c->cfg;
    const s2ar_stack& st = is_slow ? g.slow : g.fast;
    const std::vector<LayerW>& W = is_slow ? c->slow : c->fast;
    const int H = st.hidden, D = st.head_dim, qd = st.n_q_heads * D, F = st.ffn;
    const int qkvd = (st.n_q_heads + 2 * st.n_kv_heads) * D, ldx = s2k::pad_k(g.slow.hidden);
    const float eps = (float)g.rms_eps;
    for (int l = 0; l < st.n_layers; ++l) {
      const LayerW& L = W[l];
      fold_b(xres, pending, H, M);
      // q, k, v stay as split-K partials; the attention kernel sums them as it loads them
      const int qkv_S = mgemv(s2k::MG_ADD, L.tqkv, L.sqkv, xres, ldx, nullptr, 0, qkvd, H, M, 0, 0, L.attn_norm);
      s2k::AttnArgs a{};
      a.qkv = c->bqkv;
      a.qkv_part = c->bpart;
      a.qkv_S = qkv_S;
      a.qkv_ldp = s2k::mgemv_tiles(qkvd) * 64;
      a.q_norm = L.q_norm;
      a.k_norm = L.k_norm;
      a.slots = slots;
      a.M = M;
      a.Hq = st.n_q_heads;
      a.Hkv = st.n_kv_heads;
      a.D = D;
      a.page_size = kPageSize;
      a.eps = eps;
      a.scale = (float)(1.0 / std::sqrt((double)D));
      a.out = c->batt;
      a.part_ml = c->batt_ml;
      a.part_o = c->batt_o;
      a.k_bf16 = c->k_bf16;
      a.v_bf16 = c->v_bf16;
      a.split = c->attn_split_b;
      a.fixed_slot = -1;
      a.row_pos = nullptr;
      a.append = 1;
      a.const_pos = is_slow ? -1 : fast_step - 1;  // every stream's Fast step j sits at position j - 1
      if (is_slow) {
        a.rope_cos = c->rope_cos_s;
        a.rope_sin = c->rope_sin_s;
        a.pos = c->d_pos;
        a.k_cache = c->kv_k + (size_t)l * c->kv_layer_k;
        a.v_cache = c->kv_v + (size_t)l * c->kv_layer_v;
        a.block_table = c->d_bt;
        a.bt_stride = c->bt_stride;
        a.max_splits = c->max_splits_b;
      } else {
        a.rope_cos = c->rope_cos_f;
        a.rope_sin = c->rope_sin_f;
        a.pos = fast_pos_ptr;
        a.k_cache = c->fkv_k + (size_t)l * c->fkv_layer_k;
        a.v_cache = c->fkv_v + (size_t)l * c->fkv_layer_v;
        a.block_table = c->d_fast_bt;
        a.bt_stride = 1;
        a.max_splits = 1;
      }
      chk(is_slow && c->attn_long ? s2k::launch_attention_long(a, s) : s2k::launch_attention(a, s));
      if (a.max_splits > 1) chk(s2k::launch_attention_combine(a, s));
      pending = mgemv(s2k::MG_ADD, L.to, L.so, c->batt, qd, nullptr, 0, H, qd, M);
      fold_b(xres, pending, H, M);
      mgemv(s2k::MG_SWIGLU, L.tgu, L.sgu, xres, ldx, c->bact, F, 2 * F, H, M, 0, 0, L.mlp_norm);
      pending = mgemv(s2k::MG_ADD, L.tdown, L.sdown, c->bact, F, nullptr, 0, H, F, M);
      if (btp) {
        norm_b(xres, pending, H, M, nullptr);
        for (int b = 0; b < M; ++b) {
          float* dst = is_slow ? btp[b].slow_resid : btp[b].fast_resid;
          if (dst) d2h(dst + (size_t)(is_slow ? l : tap_step * st.n_layers + l) * H, xres + (size_t)b * ldx, sizeof(float) * H);
        }
      }
    }
    return pending;
  }
  int tap_step = 0;

  void finish_b(int mode, int j, int M, const int* slots, int lo, int hi, float* x) {
    const s2ar_config& g = c->cfg;
    s2k::FinishBArgs f{};
    f.am_val = c->bam_val;
    f.am_idx = c->bam_idx;
    f.b0 = lo / 16;
    f.b1 = (hi - 1) / 16;
    f.lo = lo;
    f.mode = mode;
    f.j = j;
    f.slots = slots;
    f.codes = c->d_codes;
    f.snap = c->d_snap;
    f.pos = c->d_pos;
    f.codebook = c->codebook;
    f.h = c->d_h;
    f.x = x;
    f.ldx = s2k::pad_k(g.slow.hidden);
    f.x_res = c->bxn;
    f.xf_slot = c->xf;
    f.ld_xf_slot = s2k::pad_k(g.slow.hidden);
    f.H = g.slow.hidden;
    f.K = g.codebook_size;
    f.NC = g.n_codebooks;
    f.logits = c->blogits;
    f.ld_logits = c->head_rows;
    f.eos_at = mode == s2k::FIN_SLOW ? c->head_eos : -1;
    chk(s2k::launch_finish_b(c->bf16, f, M, s));
  }

  // one frame of M streams: the Fast loops of all streams in lock step, then their Slow steps
  void frame_b(int M, const int* slots) {
    const s2ar_config& g = c->cfg;
    const int H = g.slow.hidden, K = g.codebook_size, NC = g.n_codebooks, V = g.vocab_text + K;
    const int ldx = s2k::pad_k(H);
    const float eps = (float)g.rms_eps;
    auto code_ptr = [&](int b, int j) { return c->d_codes + (size_t)bslots_host[b] * NC + j; };
    if (btp)
      for (int b = 0; b < M; ++b) {
        if (btp[b].own) d2h(btp[b].own, code_ptr(b, 0), sizeof(int));
        if (btp[b].forced) h2d(code_ptr(b, 0), btp[b].forced, sizeof(int));
      }
    chk(s2k::launch_gather_h(c->d_h, slots, H, c->bxf, ldx, M, s));
    for (int j = 1; j < NC; ++j) {
      fast_pos_ptr = c->d_fast_pos + (size_t)(j - 1) * g.max_streams;
      if (btp && j > 1)  // eager frame: the input honours forced codes
        chk(s2k::launch_fast_input(c->bf16, c->codebook, c->d_h, K, H, NC, slots, c->d_codes, j, c->bxf, ldx, M, s));
      tap_step = j - 1;
      fast_step = j;
      int pending = layers_b(false, M, slots, c->bxf);
      fold_b(c->bxf, pending, H, M);
      mgemv(s2k::MG_ARGMAX, c->fast_head_t, c->fast_head_s, c->bxf, ldx, c->blogits, K, K, H, M, 0, K, c->fast_final);
      if (btp) {
        finish_b(s2k::FIN_CODE, j, M, slots, 0, K, c->bxf);
        for (int b = 0; b < M; ++b) {
          if (btp[b].fast_logits) d2h(btp[b].fast_logits + (size_t)(j - 1) * K, c->blogits + (size_t)b * K, sizeof(float) * K);
          if (btp[b].own) d2h(btp[b].own + j, code_ptr(b, j), sizeof(int));
          if (btp[b].forced) h2d(code_ptr(b, j), btp[b].forced + j, sizeof(int));
        }
      } else {
        finish_b(j < NC - 1 ? s2k::FIN_FAST_NEXT : s2k::FIN_FAST_LAST, j, M, slots, 0, K,
                 j < NC - 1 ? c->bxf : c->bx);
      }
    }
    if (btp)
      chk(s2k::launch_embed_codes(c->bf16, c->codebook, K, H, NC, slots, c->d_codes, c->d_snap, c->bx, ldx, M, s));
    int pending = layers_b(true, M, slots, c->bx);
    norm_b(c->bx, pending, H, M, c->slow_final);
    const int NH = c->head_rows, lo = c->head_lo;
    mgemv(s2k::MG_ARGMAX, c->slow_head_t, c->slow_head_s, c->bxn, ldx, c->blogits, NH, NH, H, M, lo, lo + K);
    finish_b(s2k::FIN_SLOW, 0, M, slots, lo, lo + K, c->bxf);
    if (btp)
      for (int b = 0; b < M; ++b) {
        if (btp[b].slow_logits) {
          if (g.head_slice) {  // full-vocabulary indexing; the rows not computed stay NaN
            d2h(btp[b].slow_logits + g.vocab_text, c->blogits + (size_t)b * NH, sizeof(float) * K);
            if (g.eos_id >= 0) d2h(btp[b].slow_logits + g.eos_id, c->blogits + (size_t)b * NH + K, sizeof(float));
          } else {
            d2h(btp[b].slow_logits, c->blogits + (size_t)b * V, sizeof(float) * V);
          }
        }
        if (btp[b].slow_h) d2h(btp[b].slow_h, c->d_h + (size_t)bslots_host[b] * H, sizeof(float) * H);
        if (btp[b].next_c0) d2h(btp[b].next_c0, code_ptr(b, 0), sizeof(int));
      }
  }

  void frame(int slot, const TapPlan* tp) {
    if (tp && tp->own) d2h(tp->own, c->d_codes + (size_t)slot * c->cfg.n_codebooks, sizeof(int));
    if (tp && tp->forced) h2d(c->d_codes + (size_t)slot * c->cfg.n_codebooks, tp->forced, sizeof(int));
    fast_loop(slot, tp);
    slow_step(slot, tp);
  }
};

int order_after_user(s2ar_ctx* c) {
  HIP_TRY(c, hipEventRecord(c->ev_order, c->user_stream));
  HIP_TRY(c, hipStreamWaitEvent(c->stream, c->ev_order, 0));
  return 0;
}

// Give stream `s` pages for positions [0, upto).
int ensure_pages(s2ar_ctx* c, int s, int upto) {
  auto& pages = c->stream_pages[s];
  const int need = (upto + kPageSize - 1) / kPageSize;
  if (need > c->bt_stride) return set_err(c, S2AR_E_CAPACITY, "context would exceed max_context");
  if (need - (int)pages.size() > (int)c->free_pages.size())
    return set_err(c, S2AR_E_CAPACITY, "no free KV page");
  const int first = (int)pages.size();
  while ((int)pages.size() < need) {
    const int p = c->free_pages.back();
    c->free_pages.pop_back();
    c->page_refs[p] = 1;
    c->h_bt[s * c->bt_stride + (int)pages.size()] = p;
    pages.push_back(p);
  }
  if (need > first)
    HIP_TRY(c, hipMemcpyAsync(c->d_bt + s * c->bt_stride + first, c->h_bt + s * c->bt_stride + first,
                              sizeof(int) * (need - first), hipMemcpyHostToDevice, c->stream));
  return 0;
}

int check_streams(s2ar_ctx* c, const int32_t* ids, int32_t n, int frames) {
  if (!ids || n < 1 || n > c->cfg.max_streams) return set_err(c, S2AR_E_ARG, "stream_ids must list 1..max_streams streams");
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= c->cfg.max_streams) return set_err(c, S2AR_E_RANGE, "stream id out of range");
    for (int k = 0; k < i; ++k)
      if (ids[k] == ids[i]) return set_err(c, S2AR_E_ARG, "stream ids must be distinct");
  }
  for (int i = 0; i < n; ++i)
    if (!c->ready[ids[i]]) return set_err(c, S2AR_E_STATE, "stream has not been prefilled");
  for (int i = 0; i < n; ++i)
    if (c->ended[ids[i]]) return set_err(c, S2AR_E_STATE, "stream has ended (its Slow pick was the stop id)");
  for (int i = 0; i < n; ++i)
    if (c->pos[ids[i]] + frames > c->cfg.max_context)
      return set_err(c, S2AR_E_CAPACITY, "context would exceed max_context");
  int pages_needed = 0;
  for (int i = 0; i < n; ++i) {
    const int need = (c->pos[ids[i]] + frames + kPageSize - 1) / kPageSize;
    pages_needed += std::max(0, need - (int)c->stream_pages[ids[i]].size());
  }
  if (pages_needed > (int)c->free_pages.size()) return set_err(c, S2AR_E_CAPACITY, "no free KV page");
  return 0;
}

// Frame graphs of a stream: one for frames whose Slow context fits one attention workgroup
// (bucket 0, no split merge) and one for longer contexts (bucket 1).
int frame_bucket(int ctx) { return slow_split_for(ctx).nsplit == 1 ? 0 : 1; }

Graph* frame_graph(s2ar_ctx* c, int slot, int bucket, int* rc) {
  const int key = slot * 2 + bucket;
  auto it = c->graphs.find(key);
  if (it != c->graphs.end()) return &it->second;
  Graph g;
  hipError_t e = hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    *rc = set_err(c, S2AR_E_DEVICE, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
    return nullptr;
  }
  Enq q{c, c->stream};
  q.set_slow_ctx(bucket == 0 ? 1 : c->cfg.max_context, false);
  q.frame(slot, nullptr);
  e = hipStreamEndCapture(c->stream, &g.g);
  if (q.e != hipSuccess || e != hipSuccess) {
    if (g.g) hipGraphDestroy(g.g);
    *rc = set_err(c, S2AR_E_DEVICE, std::string("graph capture: ") + hipGetErrorString(q.e != hipSuccess ? q.e : e));
    return nullptr;
  }
  e = hipGraphInstantiate(&g.exec, g.g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(g.g);
    *rc = set_err(c, S2AR_E_DEVICE, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    return nullptr;
  }
  return &(c->graphs[key] = g);
}

s2ar_ctx::BatchGraph* batch_graph(s2ar_ctx* c, const std::vector<int>& ids, int* rc) {
  auto it = c->bgraphs.find(ids);
  if (it != c->bgraphs.end()) return &it->second;
  s2ar_ctx::BatchGraph bg;
  if (int r = dev_alloc(c, &bg.d_slots, sizeof(int) * 16)) {
    *rc = r;
    return nullptr;
  }
  hipError_t e = hipMemcpy(bg.d_slots, ids.data(), sizeof(int) * ids.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    *rc = set_err(c, S2AR_E_DEVICE, std::string("batch graph setup: ") + hipGetErrorString(e));
    return nullptr;
  }
  Enq q{c, c->stream};
  q.frame_b((int)ids.size(), bg.d_slots);
  e = hipStreamEndCapture(c->stream, &bg.g.g);
  if (q.e != hipSuccess || e != hipSuccess) {
    if (bg.g.g) hipGraphDestroy(bg.g.g);
    *rc = set_err(c, S2AR_E_DEVICE, std::string("batch graph capture: ") + hipGetErrorString(q.e != hipSuccess ? q.e : e));
    return nullptr;
  }
  e = hipGraphInstantiate(&bg.g.exec, bg.g.g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(bg.g.g);
    *rc = set_err(c, S2AR_E_DEVICE, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    return nullptr;
  }
  return &(c->bgraphs[ids] = bg);
}

}  // namespace

// ------------------------------------------------------------------------------------ C ABI

extern "C" {

const char* s2ar_error_name(int code) {
  switch (code) {
    case S2AR_OK: return "S2AR_OK";
    case S2AR_E_ARG: return "S2AR_E_ARG";
    case S2AR_E_RANGE: return "S2AR_E_RANGE";
    case S2AR_E_CAPACITY: return "S2AR_E_CAPACITY";
    case S2AR_E_STATE: return "S2AR_E_STATE";
    case S2AR_E_NOMEM: return "S2AR_E_NOMEM";
    case S2AR_E_DEVICE: return "S2AR_E_DEVICE";
    case S2AR_E_NUMERIC: return "S2AR_E_NUMERIC";
  }
  return "S2AR_E_UNKNOWN";
}

const char* s2ar_last_error(const s2ar_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_error.c_str(); }

int s2ar_create(const s2ar_config* cfg, const s2ar_tensor* tensors, int32_t n_tensors, void* hip_stream,
                s2ar_ctx** out) {
  if (out) *out = nullptr;
  if (!cfg || !tensors || !out) return set_err(nullptr, S2AR_E_ARG, "cfg, tensors and out must be non-null");
  std::string why;
  if (validate_config(cfg, why)) return set_err(nullptr, S2AR_E_ARG, why);
  if (n_tensors != n_tensors_for(cfg)) return set_err(nullptr, S2AR_E_ARG, "n_tensors does not match the config");
  const std::vector<int64_t> sizes = tensor_sizes(cfg);
  const int64_t esz = cfg->weight_dtype == 0 ? 4 : 2;  // bf16 tensors for weight_dtype 1, 2 and 3
  for (int i = 0; i < n_tensors; ++i) {
    if (!tensors[i].host_ptr) return set_err(nullptr, S2AR_E_ARG, "tensor " + std::to_string(i) + " is null");
    if (tensors[i].nbytes != sizes[i] * esz)
      return set_err(nullptr, S2AR_E_ARG, "tensor " + std::to_string(i) + " has " + std::to_string(tensors[i].nbytes) +
                                              " bytes, expected " + std::to_string(sizes[i] * esz));
  }
  int dev_count = 0;
  if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count < 1)
    return set_err(nullptr, S2AR_E_DEVICE, "no HIP device is visible");
  return create_impl(cfg, tensors, n_tensors, hip_stream, out);
}

void s2ar_destroy(s2ar_ctx* ctx) { free_ctx(ctx); }

int s2ar_prefill(s2ar_ctx* c, int32_t sid, const int32_t* tokens, const uint8_t* mask, const int32_t* codes,
                 int32_t n) {
  if (!c) return S2AR_E_ARG;
  const s2ar_config& g = c->cfg;
  if (!tokens || n < 1) return set_err(c, S2AR_E_ARG, "tokens must be non-null and n >= 1");
  if (mask && !codes) return set_err(c, S2AR_E_ARG, "vq_codes are required with vq_mask");
  if (sid < 0 || sid >= g.max_streams) return set_err(c, S2AR_E_RANGE, "stream id out of range");
  if ((int64_t)c->pos[sid] + n > g.max_context) return set_err(c, S2AR_E_CAPACITY, "context would exceed max_context");
  const int V = g.vocab_text + g.codebook_size, NC = g.n_codebooks;
  for (int i = 0; i < n; ++i) {
    if (mask && mask[i]) {
      for (int k = 0; k < NC; ++k)
        if (codes[(size_t)i * NC + k] < 0 || codes[(size_t)i * NC + k] >= g.codebook_size)
          return set_err(c, S2AR_E_RANGE, "VQ code out of range at position " + std::to_string(i));
    } else if (tokens[i] < 0 || tokens[i] >= V) {
      return set_err(c, S2AR_E_RANGE, "token id out of range at position " + std::to_string(i));
    }
  }
  const int need = (c->pos[sid] + n + kPageSize - 1) / kPageSize - (int)c->stream_pages[sid].size();
  if (need > (int)c->free_pages.size()) return set_err(c, S2AR_E_CAPACITY, "no free KV page");

  if (int rc = order_after_user(c)) return rc;
  if (int rc = ensure_pages(c, sid, c->pos[sid] + n)) return rc;
  HIP_TRY(c, hipMemcpyAsync(c->d_tokens, tokens, sizeof(int) * n, hipMemcpyHostToDevice, c->stream));
  if (mask) {
    HIP_TRY(c, hipMemcpyAsync(c->d_mask, mask, (size_t)n, hipMemcpyHostToDevice, c->stream));
    HIP_TRY(c, hipMemcpyAsync(c->d_pcodes, codes, sizeof(int) * (size_t)n * NC, hipMemcpyHostToDevice, c->stream));
  }
  Enq q{c, c->stream};
  const bool f16 = c->mfma_prefill && n >= 2 && c->prefill_f16;
  if (f16) q.chk(hipMemsetAsync(c->d_range, 0, sizeof(int), c->stream));
  if (c->mfma_prefill && n >= 2) {
    const int H = g.slow.hidden;
    for (int p0 = 0; p0 < n && q.e == hipSuccess; p0 += c->pch) {
      const int rows = std::min(c->pch, n - p0);
      q.prefill_rows(sid, p0, c->pos[sid] + p0, rows, mask != nullptr);
      if (p0 + rows == n) {  // the last row goes through the Slow head
        q.chk(hipMemcpyAsync(c->x, c->px + (size_t)(rows - 1) * H, sizeof(float) * H, hipMemcpyDeviceToDevice,
                             c->stream));
        c->h_pos_stage[0] = c->pos[sid] + n - 1;  // the finisher advances it to pos + n
        q.chk(hipMemcpyAsync(c->d_pos + sid, c->h_pos_stage, sizeof(int), hipMemcpyHostToDevice, c->stream));
        q.slow_head(sid, nullptr);
      }
    }
  } else {
    for (int p = 0; p < n; ++p) {
      q.chk(s2k::launch_embed_prompt(c->bf16, c->embed, c->codebook, g.codebook_size, g.slow.hidden, NC,
                                     c->d_tokens, mask ? c->d_mask : nullptr, c->d_pcodes, p, c->x, c->stream));
      q.layers(true, sid, c->x, nullptr);
      if (p == n - 1) q.slow_head(sid, nullptr);  // its finisher advances the position
      else q.chk(s2k::launch_advance(c->d_slot_ids + sid, c->d_pos, 1, c->stream));
      if (q.e != hipSuccess) break;
    }
  }
  if (f16) q.chk(hipMemcpyAsync(c->h_pos_stage + 8, c->d_range, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  if (q.e != hipSuccess) return set_err(c, S2AR_E_DEVICE, std::string("prefill launch: ") + hipGetErrorString(q.e));
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  if (f16 && c->h_pos_stage[8]) {
    // an activation beyond fp16's range: the new positions are dropped (the device position goes
    // back to the host's) and the stream's pending pick is gone, so it is not ready to decode
    c->h_pos_stage[0] = c->pos[sid];
    HIP_TRY(c, hipMemcpyAsync(c->d_pos + sid, c->h_pos_stage, sizeof(int), hipMemcpyHostToDevice, c->stream));
    HIP_TRY(c, hipStreamSynchronize(c->stream));
    c->ready[sid] = 0;
    return set_err(c, S2AR_E_NUMERIC, "prefill activation outside the fp16 range (use prefill precision 0)");
  }
  c->pos[sid] += n;
  c->ready[sid] = 1;
  c->ended[sid] = 0;  // the new positions end with a fresh Slow pick
  return S2AR_OK;
}

int s2ar_set_prefill_precision(s2ar_ctx* c, int32_t precision) {
  if (!c) return S2AR_E_ARG;
  if (precision != 0 && precision != 1) return set_err(c, S2AR_E_ARG, "prefill precision must be 0 or 1");
  if (precision == 1 && !(c->mfma_prefill && c->f16_prefill_ok))
    return set_err(c, S2AR_E_ARG, "the fp16 prefill needs the matrix-core prefill and every K a multiple of 64");
  c->prefill_f16 = precision == 1;
  return S2AR_OK;
}

// Advance the streams by the call's frames.  A frame whose semantic code is -1 is the stream's stop:
// it and every later frame of the call come out as -1 and the stream ends.  The device kept running
// the stream's graph after the stop, appending a Slow position per frame built from clamped codes;
// frame f of the call appended position p0 + f, and the stop pick of frame f came from the position
// before it, so the stream is rewound to p0 + f on the host and the device: its cache then holds
// exactly the positions the model decoded, and a later prefill appends after them.
int finish_frames(s2ar_ctx* c, const int32_t* ids, int32_t n, int32_t n_frames, int32_t* codes_out) {
  const int NC = c->cfg.n_codebooks;
  for (int i = 0; i < n; ++i) {
    const int p0 = c->pos[ids[i]];
    int stop = -1;
    for (int f = 0; f < n_frames; ++f) {
      int32_t* row = codes_out + ((size_t)f * n + i) * NC;
      if (stop < 0 && row[0] < 0) stop = f;
      if (stop >= 0) std::fill(row, row + NC, -1);
    }
    if (stop < 0) {
      c->pos[ids[i]] = p0 + n_frames;
    } else {
      c->ended[ids[i]] = 1;
      c->pos[ids[i]] = p0 + stop;
      c->h_pos_stage[0] = p0 + stop;
      HIP_TRY(c, hipMemcpyAsync(c->d_pos + ids[i], c->h_pos_stage, sizeof(int), hipMemcpyHostToDevice, c->stream));
      HIP_TRY(c, hipStreamSynchronize(c->stream));  // the pinned staging is reused
    }
  }
  return S2AR_OK;
}

int s2ar_decode_frames(s2ar_ctx* c, const int32_t* ids, int32_t n, int32_t n_frames, int32_t* codes_out) {
  if (!c) return S2AR_E_ARG;
  if (!codes_out || n_frames < 1) return set_err(c, S2AR_E_ARG, "codes_out must be non-null and n_frames >= 1");
  if (int rc = check_streams(c, ids, n, n_frames)) return rc;
  const int NC = c->cfg.n_codebooks;
  if (c->batched_ok && n > 1) {
    // groups of up to 16 streams, one captured graph per group
    std::vector<s2ar_ctx::BatchGraph*> groups;
    for (int i0 = 0; i0 < n; i0 += 16) {
      std::vector<int> gids(ids + i0, ids + std::min(n, i0 + 16));
      int rc = 0;
      s2ar_ctx::BatchGraph* bg = batch_graph(c, gids, &rc);
      if (!bg) return rc;
      groups.push_back(bg);
    }
    if (int rc = order_after_user(c)) return rc;
    for (int i = 0; i < n; ++i)
      if (int rc = ensure_pages(c, ids[i], c->pos[ids[i]] + n_frames)) return rc;
    const int ms = c->cfg.max_streams;
    int done = 0;
    while (done < n_frames) {
      const int chunk = std::min(n_frames - done, c->h_codes_frames * ms / std::max(ms, 1));
      for (int f = 0; f < chunk; ++f) {
        for (auto* bg : groups) HIP_TRY(c, hipGraphLaunch(bg->g.exec, c->stream));
        HIP_TRY(c, hipMemcpyAsync(c->h_codes + (size_t)f * ms * NC, c->d_snap, sizeof(int) * ms * NC,
                                  hipMemcpyDeviceToHost, c->stream));
      }
      HIP_TRY(c, hipStreamSynchronize(c->stream));
      for (int f = 0; f < chunk; ++f)
        for (int i = 0; i < n; ++i)
          std::memcpy(codes_out + ((size_t)(done + f) * n + i) * NC, c->h_codes + ((size_t)f * ms + ids[i]) * NC,
                      sizeof(int) * NC);
      done += chunk;
    }
    return finish_frames(c, ids, n, n_frames, codes_out);
  }
  // the graphs of every bucket the call's frames reach, captured before any work is queued
  std::vector<Graph*> gs(2 * (size_t)n, nullptr);
  for (int i = 0; i < n; ++i)
    for (int b = frame_bucket(c->pos[ids[i]] + 1); b <= frame_bucket(c->pos[ids[i]] + n_frames); ++b) {
      int rc = 0;
      gs[2 * i + b] = frame_graph(c, ids[i], b, &rc);
      if (!gs[2 * i + b]) return rc;
    }
  if (int rc = order_after_user(c)) return rc;
  for (int i = 0; i < n; ++i)
    if (int rc = ensure_pages(c, ids[i], c->pos[ids[i]] + n_frames)) return rc;
  int done = 0;
  while (done < n_frames) {
    const int chunk = std::min(n_frames - done, c->h_codes_frames * c->cfg.max_streams / n);
    for (int f = 0; f < chunk; ++f)
      for (int i = 0; i < n; ++i) {
        // frame done + f of stream i: its Slow step attends over pos + done + f + 1 positions
        const Graph* gr = gs[2 * i + frame_bucket(c->pos[ids[i]] + done + f + 1)];
        HIP_TRY(c, hipGraphLaunch(gr->exec, c->stream));
        HIP_TRY(c, hipMemcpyAsync(c->h_codes + ((size_t)f * n + i) * NC, c->d_snap + (size_t)ids[i] * NC,
                                  sizeof(int) * NC, hipMemcpyDeviceToHost, c->stream));
      }
    HIP_TRY(c, hipStreamSynchronize(c->stream));
    std::memcpy(codes_out + (size_t)done * n * NC, c->h_codes, sizeof(int) * (size_t)chunk * n * NC);
    done += chunk;
  }
  return finish_frames(c, ids, n, n_frames, codes_out);
}

int s2ar_decode_frame(s2ar_ctx* c, const int32_t* ids, int32_t n, int32_t* codes_out) {
  return s2ar_decode_frames(c, ids, n, 1, codes_out);
}

int s2ar_decode_frames_noalloc(s2ar_ctx* c, int32_t sid, int32_t n_frames, int32_t* codes_out) {
  if (!c) return S2AR_E_ARG;
  if (!codes_out || n_frames < 1) return set_err(c, S2AR_E_ARG, "codes_out must be non-null and n_frames >= 1");
  if (int rc = check_streams(c, &sid, 1, n_frames)) return rc;
  const s2ar_config& g = c->cfg;
  const int NC = g.n_codebooks;
  // scratch layout: pick partials (values, then indices), then the Slow attention split partials
  // of the call's longest frame ((max, sum) pairs, then outputs), each 256-byte aligned
  auto up256 = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t nb = (size_t)std::max(s2k::gemv_blocks(s2k::GEMV_NORM_ARGMAX, c->head_rows),
                                     s2k::gemv_blocks(s2k::GEMV_NORM_ARGMAX, g.codebook_size));
  const int hq = g.slow.n_q_heads, D = g.slow.head_dim;
  const int max_nsplit = slow_split_for(c->pos[sid] + n_frames).nsplit;
  const size_t am_bytes = up256(sizeof(float) * nb), ml_bytes = up256(sizeof(float) * 2 * hq * max_nsplit);
  const size_t need = 2 * am_bytes + ml_bytes + up256(sizeof(float) * (size_t)hq * max_nsplit * D);
  if (need > S2AR_NOALLOC_SCRATCH_BYTES)
    return set_err(c, S2AR_E_CAPACITY, "frame scratch of " + std::to_string(need) + " bytes exceeds the " +
                                           std::to_string(S2AR_NOALLOC_SCRATCH_BYTES) + "-byte scratch array");
  if (int rc = order_after_user(c)) return rc;
  if (int rc = ensure_pages(c, sid, c->pos[sid] + n_frames)) return rc;
  unsigned char* sc = c->scratch_dev;
  int done = 0;
  while (done < n_frames) {
    const int chunk = std::min(n_frames - done, c->h_codes_frames);
    Enq q{c, c->stream};
    q.ws_am_val = reinterpret_cast<float*>(sc);
    q.ws_am_idx = reinterpret_cast<int*>(sc + am_bytes);
    q.ws_att_ml = reinterpret_cast<float*>(sc + 2 * am_bytes);
    q.ws_att_o = reinterpret_cast<float*>(sc + 2 * am_bytes + ml_bytes);
    for (int f = 0; f < chunk && q.e == hipSuccess; ++f) {
      q.set_slow_ctx(c->pos[sid] + done + f + 1, true);
      q.frame(sid, nullptr);
      q.d2h(c->h_codes + (size_t)f * NC, c->d_snap + (size_t)sid * NC, sizeof(int) * NC);
    }
    if (q.e != hipSuccess) return set_err(c, S2AR_E_DEVICE, std::string("noalloc frame: ") + hipGetErrorString(q.e));
    HIP_TRY(c, hipStreamSynchronize(c->stream));
    std::memcpy(codes_out + (size_t)done * NC, c->h_codes, sizeof(int) * (size_t)chunk * NC);
    done += chunk;
  }
  return finish_frames(c, &sid, 1, n_frames, codes_out);
}

int s2ar_debug_frame(s2ar_ctx* c, int32_t sid, const int32_t* forced, s2ar_taps* taps) {
  if (!c) return S2AR_E_ARG;
  if (int rc = check_streams(c, &sid, 1, 1)) return rc;
  const s2ar_config& g = c->cfg;
  const int NC = g.n_codebooks, H = g.slow.hidden, K = g.codebook_size, V = g.vocab_text + K;
  if (forced)
    for (int k = 0; k < NC; ++k)
      if (forced[k] < 0 || forced[k] >= K) return set_err(c, S2AR_E_RANGE, "forced code out of range");
  s2ar_taps none{};
  const s2ar_taps& T = taps ? *taps : none;
  TapPlan tp;
  float* f = c->h_taps;
  tp.embed = f;
  f += H;
  tp.slow_resid = f;
  f += (size_t)g.slow.n_layers * H;
  tp.slow_h = f;
  f += H;
  tp.slow_logits = f;
  f += V;
  tp.fast_resid = f;
  f += (size_t)(NC - 1) * g.fast.n_layers * H;
  tp.fast_z = f;
  f += (size_t)(NC - 1) * H;
  tp.fast_logits = f;
  tp.own = c->h_small;
  tp.next_c0 = c->h_small + NC;
  if (forced) {
    std::memcpy(c->h_small + 2 * NC, forced, sizeof(int) * NC);
    tp.forced = c->h_small + 2 * NC;
  }
  if (g.head_slice) std::fill(tp.slow_logits, tp.slow_logits + V, NAN);
  if (int rc = order_after_user(c)) return rc;
  if (int rc = ensure_pages(c, sid, c->pos[sid] + 1)) return rc;
  Enq q{c, c->stream};
  q.set_slow_ctx(c->pos[sid] + 1, true);
  q.frame(sid, &tp);
  if (q.e != hipSuccess) return set_err(c, S2AR_E_DEVICE, std::string("debug frame: ") + hipGetErrorString(q.e));
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  c->pos[sid] += 1;
  auto put = [](float* dst, const float* src, size_t n) {
    if (dst) std::memcpy(dst, src, sizeof(float) * n);
  };
  put(T.slow_embed, tp.embed, H);
  put(T.slow_resid, tp.slow_resid, (size_t)g.slow.n_layers * H);
  put(T.slow_h, tp.slow_h, H);
  put(T.slow_logits, tp.slow_logits, V);
  put(T.fast_resid, tp.fast_resid, (size_t)(NC - 1) * g.fast.n_layers * H);
  put(T.fast_z, tp.fast_z, (size_t)(NC - 1) * H);
  put(T.fast_logits, tp.fast_logits, (size_t)(NC - 1) * K);
  if (T.own_codes) std::memcpy(T.own_codes, tp.own, sizeof(int) * NC);
  if (T.next_c0) *T.next_c0 = *tp.next_c0;
  bool finite = true;
  for (int i = g.head_slice ? g.vocab_text : 0; i < V && finite; ++i) finite = std::isfinite(tp.slow_logits[i]);
  if (g.eos_id >= 0) finite = finite && std::isfinite(tp.slow_logits[g.eos_id]);
  for (int i = 0; i < (NC - 1) * K && finite; ++i) finite = std::isfinite(tp.fast_logits[i]);
  if (!finite) return set_err(c, S2AR_E_NUMERIC, "non-finite logits");
  return S2AR_OK;
}

int s2ar_debug_frame_batch(s2ar_ctx* c, const int32_t* ids, int32_t n, const int32_t* forced, s2ar_taps* taps) {
  if (!c) return S2AR_E_ARG;
  if (!c->batched_ok) return set_err(c, S2AR_E_ARG, "batched decode needs bf16 tables and K dims divisible by 512");
  if (n > 16) return set_err(c, S2AR_E_ARG, "at most 16 streams per batched debug frame");
  if (int rc = check_streams(c, ids, n, 1)) return rc;
  const s2ar_config& g = c->cfg;
  const int NC = g.n_codebooks, H = g.slow.hidden, K = g.codebook_size, V = g.vocab_text + K;
  if (forced)
    for (int i = 0; i < n * NC; ++i)
      if (forced[i] < 0 || forced[i] >= K) return set_err(c, S2AR_E_RANGE, "forced code out of range");
  const size_t per = (size_t)g.slow.n_layers * H + H + V + (size_t)(NC - 1) * g.fast.n_layers * H + (size_t)(NC - 1) * K;
  float* stage = nullptr;
  int* istage = nullptr;
  if (hipHostMalloc(&stage, sizeof(float) * per * n, hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc(&istage, sizeof(int) * (size_t)n * NC * 3, hipHostMallocDefault) != hipSuccess) {
    if (stage) hipHostFree(stage);
    return set_err(c, S2AR_E_NOMEM, "pinned staging for taps");
  }
  std::vector<Enq::BTap> bt(n);
  for (int b = 0; b < n; ++b) {
    float* f = stage + per * b;
    bt[b].slow_resid = f;
    f += (size_t)g.slow.n_layers * H;
    bt[b].slow_h = f;
    f += H;
    bt[b].slow_logits = f;
    if (g.head_slice) std::fill(f, f + V, NAN);  // rows the semantic-slice head does not compute
    f += V;
    bt[b].fast_resid = f;
    f += (size_t)(NC - 1) * g.fast.n_layers * H;
    bt[b].fast_logits = f;
    bt[b].own = istage + (size_t)b * NC;
    bt[b].next_c0 = istage + (size_t)n * NC + b;
    if (forced) {
      std::memcpy(istage + (size_t)2 * n * NC + (size_t)b * NC, forced + (size_t)b * NC, sizeof(int) * NC);
      bt[b].forced = istage + (size_t)2 * n * NC + (size_t)b * NC;
    }
  }
  std::vector<int> idv(ids, ids + n);
  int rc = 0;
  int* d_slots = c->d_dbg_slots;
  hipError_t e = hipMemcpy(d_slots, ids, sizeof(int) * n, hipMemcpyHostToDevice);
  if (e == hipSuccess && (rc = order_after_user(c)) == 0) {
    for (int i = 0; i < n && rc == 0; ++i) rc = ensure_pages(c, ids[i], c->pos[ids[i]] + 1);
    if (rc == 0) {
      Enq q{c, c->stream};
      q.btp = bt.data();
      q.bslots_host = idv.data();
      q.frame_b(n, d_slots);
      e = q.e;
      if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    }
  }
  if (rc == 0 && e != hipSuccess) rc = set_err(c, S2AR_E_DEVICE, std::string("batched debug frame: ") + hipGetErrorString(e));
  if (rc == 0) {
    for (int i = 0; i < n; ++i) c->pos[ids[i]] += 1;
    for (int b = 0; b < n && taps; ++b) {
      const s2ar_taps& T = taps[b];
      auto put = [](float* dst, const float* src, size_t cnt) {
        if (dst) std::memcpy(dst, src, sizeof(float) * cnt);
      };
      put(T.slow_resid, bt[b].slow_resid, (size_t)g.slow.n_layers * H);
      put(T.slow_h, bt[b].slow_h, H);
      put(T.slow_logits, bt[b].slow_logits, V);
      put(T.fast_resid, bt[b].fast_resid, (size_t)(NC - 1) * g.fast.n_layers * H);
      put(T.fast_logits, bt[b].fast_logits, (size_t)(NC - 1) * K);
      if (T.own_codes) std::memcpy(T.own_codes, bt[b].own, sizeof(int) * NC);
      if (T.next_c0) *T.next_c0 = *bt[b].next_c0;
    }
  }
  hipHostFree(stage);
  hipHostFree(istage);
  return rc;
}

int s2ar_release_stream(s2ar_ctx* c, int32_t sid) {
  if (!c) return S2AR_E_ARG;
  if (sid < 0 || sid >= c->cfg.max_streams) return set_err(c, S2AR_E_RANGE, "stream id out of range");
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  for (int p : c->stream_pages[sid])
    if (--c->page_refs[p] == 0) c->free_pages.push_back(p);
  c->stream_pages[sid].clear();
  c->pos[sid] = 0;
  c->ready[sid] = 0;
  c->ended[sid] = 0;
  const int zero = 0;
  HIP_TRY(c, hipMemcpy(c->d_pos + sid, &zero, sizeof(int), hipMemcpyHostToDevice));
  return S2AR_OK;
}

int s2ar_share_prefix(s2ar_ctx* c, int32_t src, int32_t dst, int32_t n) {
  if (!c) return S2AR_E_ARG;
  const int ms = c->cfg.max_streams;
  if (src < 0 || src >= ms || dst < 0 || dst >= ms) return set_err(c, S2AR_E_RANGE, "stream id out of range");
  if (src == dst) return set_err(c, S2AR_E_STATE, "a stream cannot share a prefix with itself");
  if (c->pos[dst] != 0 || !c->stream_pages[dst].empty()) return set_err(c, S2AR_E_STATE, "destination stream is not empty");
  if (n < 1 || n > c->pos[src]) return set_err(c, S2AR_E_RANGE, "n_positions must be in [1, position of the source]");
  const int full = n / kPageSize, part = n % kPageSize;
  if (part && c->free_pages.empty()) return set_err(c, S2AR_E_CAPACITY, "no free KV page");
  if (int rc = order_after_user(c)) return rc;
  const std::vector<int>& sp = c->stream_pages[src];
  std::vector<int>& dp = c->stream_pages[dst];
  int* bt = c->h_bt + dst * c->bt_stride;
  for (int i = 0; i < full; ++i) {
    ++c->page_refs[sp[i]];
    dp.push_back(sp[i]);
    bt[i] = sp[i];
  }
  if (part) {  // the partial last page: a private copy (its remaining slots are dst's to fill)
    const int p = c->free_pages.back();
    c->free_pages.pop_back();
    c->page_refs[p] = 1;
    dp.push_back(p);
    bt[full] = p;
    for (int l = 0; l < c->cfg.slow.n_layers; ++l)
      for (int kv = 0; kv < 2; ++kv) {
        const size_t layer = kv ? c->kv_layer_v : c->kv_layer_k;
        const size_t page_bytes = layer / c->n_pages;  // [Hkv][16][D] of one layer
        char* base = (kv ? c->kv_v : c->kv_k) + (size_t)l * layer;
        HIP_TRY(c, hipMemcpyAsync(base + (size_t)p * page_bytes, base + (size_t)sp[full] * page_bytes, page_bytes,
                                  hipMemcpyDeviceToDevice, c->stream));
      }
  }
  HIP_TRY(c, hipMemcpyAsync(c->d_bt + dst * c->bt_stride, bt, sizeof(int) * dp.size(), hipMemcpyHostToDevice, c->stream));
  // the device position too: the next prefill (position by position, or its last row) appends at n
  c->h_pos_stage[0] = n;
  HIP_TRY(c, hipMemcpyAsync(c->d_pos + dst, c->h_pos_stage, sizeof(int), hipMemcpyHostToDevice, c->stream));
  HIP_TRY(c, hipStreamSynchronize(c->stream));  // the pinned staging may change on the next call
  c->pos[dst] = n;
  c->ready[dst] = 0;
  c->ended[dst] = 0;
  return S2AR_OK;
}

int s2ar_stream_position(const s2ar_ctx* c, int32_t sid, int32_t* pos_out) {
  if (!c || !pos_out) return S2AR_E_ARG;
  if (sid < 0 || sid >= c->cfg.max_streams) return S2AR_E_RANGE;
  *pos_out = c->pos[sid];
  return S2AR_OK;
}

int s2ar_time_frames(s2ar_ctx* c, int32_t sid, int32_t n_frames, float* ms_out) {
  if (!c) return S2AR_E_ARG;
  if (!ms_out || n_frames < 1 || n_frames > 4096)
    return set_err(c, S2AR_E_ARG, "ms_out must be non-null and n_frames in [1, 4096]");
  if (c->cfg.eos_id >= 0)
    return set_err(c, S2AR_E_ARG, "time_frames returns no codes, so it cannot see a stop: use a context without eos_id");
  if (int rc = check_streams(c, &sid, 1, n_frames)) return rc;
  int rc = 0;
  Graph* grs[2] = {nullptr, nullptr};
  for (int b = frame_bucket(c->pos[sid] + 1); b <= frame_bucket(c->pos[sid] + n_frames); ++b)
    if (!(grs[b] = frame_graph(c, sid, b, &rc))) return rc;
  if ((rc = order_after_user(c))) return rc;
  if ((rc = ensure_pages(c, sid, c->pos[sid] + n_frames))) return rc;
  std::vector<hipEvent_t> ev(2 * (size_t)n_frames, nullptr);
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < ev.size() && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
  for (int f = 0; f < n_frames && e == hipSuccess; ++f) {
    const Graph* gr = grs[frame_bucket(c->pos[sid] + f + 1)];
    e = hipEventRecord(ev[2 * f], c->stream);
    if (e == hipSuccess) e = hipGraphLaunch(gr->exec, c->stream);
    if (e == hipSuccess) e = hipEventRecord(ev[2 * f + 1], c->stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  for (int f = 0; f < n_frames && e == hipSuccess; ++f) e = hipEventElapsedTime(&ms_out[f], ev[2 * f], ev[2 * f + 1]);
  for (hipEvent_t x : ev)
    if (x) hipEventDestroy(x);
  if (e != hipSuccess) return set_err(c, S2AR_E_DEVICE, std::string("time frames: ") + hipGetErrorString(e));
  c->pos[sid] += n_frames;
  return S2AR_OK;
}

int s2ar_time_kernel(s2ar_ctx* c, int32_t which, int32_t iters, float* avg_ms, int64_t* bytes_out) {
  if (!c) return S2AR_E_ARG;
  if (which < 0 || which > 1 || iters < 1 || !avg_ms)
    return set_err(c, S2AR_E_ARG, "which must be 0 or 1, iters >= 1, avg_ms non-null");
  const s2ar_stack& st = c->cfg.slow;
  const size_t wbytes = (size_t)2 * st.ffn * st.hidden * (c->q8 ? 1 : c->esz);
  Enq q{c, c->stream};
  HIP_TRY(c, hipEventRecord(c->ev_t0, c->stream));
  for (int i = 0; i < iters; ++i) {
    const LayerW& L = c->slow[i % st.n_layers];
    if (which == 0) q.gemv(s2k::GEMV_NORM_SWIGLU, L.wgu, L.sgu, c->x, L.mlp_norm, c->act, 2 * st.ffn, st.hidden);
    else q.chk(s2k::launch_stream_read(L.wgu, wbytes, c->d_sink, c->stream));
  }
  HIP_TRY(c, hipEventRecord(c->ev_t1, c->stream));
  if (q.e != hipSuccess) return set_err(c, S2AR_E_DEVICE, std::string("time kernel: ") + hipGetErrorString(q.e));
  HIP_TRY(c, hipEventSynchronize(c->ev_t1));
  float ms = 0.f;
  HIP_TRY(c, hipEventElapsedTime(&ms, c->ev_t0, c->ev_t1));
  *avg_ms = ms / (float)iters;
  if (bytes_out)
    *bytes_out = which == 0 ? (int64_t)wbytes + (int64_t)st.hidden * 4 * 2 + (int64_t)st.ffn * 4 +
                                  (c->q8 ? (int64_t)2 * st.ffn * 4 : 0)
                            : (int64_t)wbytes;
  return S2AR_OK;
}

}  // extern "C"
