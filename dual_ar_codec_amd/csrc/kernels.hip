// gfx950 kernels of the Dual-AR per-frame decode step.
//
// At batch 1 a frame streams every weight once (the Fast stack nine times),
// so the frame is bound by HBM reads ("s2pro-native", Where it stands).  The
// kernels below are shaped for that:
//   * weight-streaming GEMV: every lane issues all of its 16-byte weight loads
//     for its rows before touching the input, the input vector sits in LDS
//     (RMSNorm fused into that staging), each 64-lane wavefront reduces its
//     rows with cross-lane shuffles, and the epilogue fuses the residual add,
//     SwiGLU, or the first pass of the greedy pick;
//   * decode attention over a paged bf16 KV cache: one workgroup per (chunk of
//     64 positions, KV head, stream) holds the K/V tile in LDS and serves the
//     q heads of that group, one wavefront per q head; QK-norm, RoPE and the
//     KV append of the new position are fused in; the last workgroup of a head
//     group merges the chunks in chunk order;
//   * codebook gather-sum for VQ injection and the Fast-step input gather.
// Every reduction has a fixed order, so a launch is bitwise reproducible.
#include "kernels.h"

#include <limits.h>
#include <math.h>

#include <algorithm>

namespace s2k {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int GEMV_WAVES = 4;
constexpr int GEMV_THREADS = GEMV_WAVES * WAVE;

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf_one(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float -> bf16 bits, round to nearest even (values here are finite)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

template <bool BF16>
__device__ __forceinline__ float load_w(const void* p, size_t i) {
  if constexpr (BF16) return bf_one(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// acc += <16-byte weight chunk, 8 (bf16) or 4 (fp32) inputs from LDS>, in element order
template <bool BF16>
__device__ __forceinline__ float dot_chunk(const u32x4 w, const float* x, float acc) {
  if constexpr (BF16) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(x);
    const f32x4 b = *reinterpret_cast<const f32x4*>(x + 4);
    acc = fmaf(bf_lo(w.x), a.x, acc);
    acc = fmaf(bf_hi(w.x), a.y, acc);
    acc = fmaf(bf_lo(w.y), a.z, acc);
    acc = fmaf(bf_hi(w.y), a.w, acc);
    acc = fmaf(bf_lo(w.z), b.x, acc);
    acc = fmaf(bf_hi(w.z), b.y, acc);
    acc = fmaf(bf_lo(w.w), b.z, acc);
    acc = fmaf(bf_hi(w.w), b.w, acc);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(x);
    acc = fmaf(__uint_as_float(w.x), a.x, acc);
    acc = fmaf(__uint_as_float(w.y), a.y, acc);
    acc = fmaf(__uint_as_float(w.z), a.z, acc);
    acc = fmaf(__uint_as_float(w.w), a.w, acc);
  }
  return acc;
}

__host__ __device__ constexpr int rows_per_wave(int kind) { return kind == GEMV_RESID ? 1 : 2; }

// Weight formats of the GEMVs: fp32, bf16, or int8 with an fp32 scale per output row (the row's
// dot product is taken on the integers and scaled once).  A lane's chunk is 16 bytes (fp32, bf16)
// or 8 bytes (int8), so every format has 8 (bf16, int8) or 4 (fp32) elements per chunk.
constexpr int WF_F32 = 0, WF_BF16 = 1, WF_I8 = 2, WF_F8 = 3;
template <int WF>
struct WFmt {
  using CT = u32x4;
  static constexpr int EPC = WF == WF_F32 ? 4 : 8;
  static constexpr int ESZ = WF == WF_F32 ? 4 : 2;
  static __device__ __forceinline__ float dot(const CT w, const float* x, float acc) {
    return dot_chunk<WF == WF_BF16>(w, x, acc);
  }
};
template <>
struct WFmt<WF_I8> {
  using CT = u32x2;
  static constexpr int EPC = 8;
  static constexpr int ESZ = 1;
  // acc += <8 int8 weights (byte k of the chunk is element k), 8 inputs from LDS>, in element order
  static __device__ __forceinline__ float dot(const CT w, const float* x, float acc) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(x);
    const f32x4 b = *reinterpret_cast<const f32x4*>(x + 4);
    acc = fmaf((float)(int8_t)(w.x & 0xffu), a.x, acc);
    acc = fmaf((float)(int8_t)((w.x >> 8) & 0xffu), a.y, acc);
    acc = fmaf((float)(int8_t)((w.x >> 16) & 0xffu), a.z, acc);
    acc = fmaf((float)(int8_t)(w.x >> 24), a.w, acc);
    acc = fmaf((float)(int8_t)(w.y & 0xffu), b.x, acc);
    acc = fmaf((float)(int8_t)((w.y >> 8) & 0xffu), b.y, acc);
    acc = fmaf((float)(int8_t)((w.y >> 16) & 0xffu), b.z, acc);
    acc = fmaf((float)(int8_t)(w.y >> 24), b.w, acc);
    return acc;
  }
};

// OCP FP8 E4M3 bytes (gfx950's matrix-core FP8 format), decoded exactly to fp32 two at a time by the
// hardware conversion; byte k of the chunk is element k.
template <>
struct WFmt<WF_F8> {
  using CT = u32x2;
  static constexpr int EPC = 8;
  static constexpr int ESZ = 1;
  static __device__ __forceinline__ float dot(const CT w, const float* x, float acc) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(x);
    const f32x4 b = *reinterpret_cast<const f32x4*>(x + 4);
    const auto w01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const auto w23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const auto w45 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const auto w67 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    acc = fmaf(w01[0], a.x, acc);
    acc = fmaf(w01[1], a.y, acc);
    acc = fmaf(w23[0], a.z, acc);
    acc = fmaf(w23[1], a.w, acc);
    acc = fmaf(w45[0], b.x, acc);
    acc = fmaf(w45[1], b.y, acc);
    acc = fmaf(w67[0], b.z, acc);
    acc = fmaf(w67[1], b.w, acc);
    return acc;
  }
};

// ---------------------------------------------------------------------------------------------
// Weight-streaming GEMV.  Workgroup = 4 wavefronts; wavefront w of block b owns rows
// (4b + w) * R ... + R - 1.  NCH > 0: K == NCH * 64 * elements-per-chunk and all weight loads of
// the wavefront are issued up front; NCH == 0: any K divisible by the chunk width / 8, looped.
// Int8 weights: each row's sum is multiplied by the row's scale before the epilogue.
template <int WF, int NCH, int KIND, int WPB = GEMV_WAVES>
__device__ __forceinline__ void gemv_impl(const GemvArgs& a) {
  extern __shared__ float xs[];
  using F = WFmt<WF>;
  using CT = typename F::CT;
  constexpr int R = rows_per_wave(KIND);
  constexpr int EPC = F::EPC;
  constexpr bool NORM = KIND != GEMV_RESID;
  constexpr int NT = WPB * WAVE;
  __shared__ float red[WPB];
  __shared__ int bidx[WPB];

  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  const int K = a.K;
  const int row0 = (blockIdx.x * WPB + wid) * R;
  const size_t row_bytes = (size_t)K * F::ESZ;
  float sc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) sc[r] = (WF == WF_I8 || WF == WF_F8) ? a.wscale[min(row0 + r, a.N - 1)] : 1.f;

  // 1. loads: the input vector (and gain) first, then every weight chunk of this wavefront's
  //    rows.  vmcnt retires in issue order, so staging the input only waits for the input.
  constexpr int XL = NCH > 0 ? (NCH * WAVE * EPC + NT * 4 - 1) / (NT * 4) : 1;
  // x and gain are zero-padded to KP floats (a multiple of 1024), and so is the LDS copy: a block
  // whose threads do not divide KP (5 wavefronts) stops at KP
  constexpr int KP = (NCH * WAVE * EPC + 1023) / 1024 * 1024;
  constexpr bool XFULL = XL * NT * 4 <= KP;
  f32x4 xv[XL], gv[XL];
  CT wv[R][NCH > 0 ? NCH : 1];
  if constexpr (NCH > 0) {
#pragma unroll
    for (int t = 0; t < XL; ++t) {
      const int k = (t * NT + threadIdx.x) * 4;
      xv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      gv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (XFULL || k < KP) {
        xv[t] = *reinterpret_cast<const f32x4*>(a.x + k);
        if constexpr (NORM) gv[t] = *reinterpret_cast<const f32x4*>(a.gain + k);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, a.N - 1);
      const CT* wp = reinterpret_cast<const CT*>(static_cast<const char*>(a.w) + (size_t)row * row_bytes);
#pragma unroll
      for (int c = 0; c < NCH; ++c) wv[r][c] = __builtin_nontemporal_load(wp + c * WAVE + lane);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load above the LDS staging
  }

  // 2. stage the input in LDS, RMSNorm fused: x * rsqrt(mean(x^2) + eps) * gain
  float ss = 0.f;
  if constexpr (NCH > 0) {
#pragma unroll
    for (int t = 0; t < XL; ++t) {
      const int k = (t * NT + threadIdx.x) * 4;
      const f32x4 v = xv[t];
      if (XFULL || k < KP) *reinterpret_cast<f32x4*>(xs + k) = v;
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
  } else {
    for (int k = threadIdx.x * 4; k < K; k += NT * 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.x + k);
      *reinterpret_cast<f32x4*>(xs + k) = v;
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
  }
  if constexpr (NORM) {
    ss = wave_sum(ss);
    if (lane == 0) red[wid] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) tot += red[w];
    const float scale = rsqrtf(tot / (float)K + a.eps);
    const bool keep = blockIdx.x == 0 && a.xnorm_out != nullptr;
    auto norm4 = [&](int k, f32x4 g) {
      f32x4 v = *reinterpret_cast<f32x4*>(xs + k);
      v.x = v.x * scale * g.x;
      v.y = v.y * scale * g.y;
      v.z = v.z * scale * g.z;
      v.w = v.w * scale * g.w;
      *reinterpret_cast<f32x4*>(xs + k) = v;
      if (keep && k < K) *reinterpret_cast<f32x4*>(a.xnorm_out + k) = v;
    };
    if constexpr (NCH > 0) {
#pragma unroll
      for (int t = 0; t < XL; ++t) {
        const int k = (t * NT + threadIdx.x) * 4;
        if (XFULL || k < KP) norm4(k, gv[t]);
      }
    } else {
      for (int k = threadIdx.x * 4; k < K; k += NT * 4) norm4(k, *reinterpret_cast<const f32x4*>(a.gain + k));
    }
  }
  __syncthreads();

  // 3. per-lane partial dot products, then the wavefront reduction
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float* xp = xs + (c * WAVE + lane) * EPC;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = F::dot(wv[r][c], xp, acc[r]);
    }
  } else {
    const int nch = (K / EPC + WAVE - 1) / WAVE;
    for (int c = 0; c < nch; ++c) {
      const int e = (c * WAVE + lane) * EPC;
      if (e < K) {
        const float* xp = xs + e;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = min(row0 + r, a.N - 1);
          const CT* wp = reinterpret_cast<const CT*>(static_cast<const char*>(a.w) + (size_t)row * row_bytes);
          acc[r] = F::dot(__builtin_nontemporal_load(wp + c * WAVE + lane), xp, acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]) * sc[r];

  // 4. epilogue
  if constexpr (KIND == GEMV_NORM_STORE) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane == r && row0 + r < a.N) a.y[row0 + r] = acc[r];
  } else if constexpr (KIND == GEMV_RESID) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane == r && row0 + r < a.N) a.y[row0 + r] += acc[r];
  } else if constexpr (KIND == GEMV_NORM_SWIGLU) {
#pragma unroll
    for (int r = 0; r < R; r += 2)
      if (lane == r && row0 + r + 1 < a.N) {
        const float gt = acc[r];
        a.y[(row0 + r) >> 1] = gt / (1.0f + expf(-gt)) * acc[r + 1];
      }
  } else {  // GEMV_NORM_ARGMAX: logits, then this block's (max, argmax) over rows in [lo, hi)
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane == r && row0 + r < a.N) a.y[row0 + r] = acc[r];
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
      if (row >= a.am_lo && row < a.am_hi && row < a.N && acc[r] > bv) {
        bv = acc[r];
        bi = row;
      }
    }
    if (lane == 0) {
      red[wid] = bv;
      bidx[wid] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = red[0];
      int i = bidx[0];
      for (int w = 1; w < WPB; ++w)
        if (red[w] > v) {
          v = red[w];
          i = bidx[w];
        }
      a.am_val[blockIdx.x] = v;
      a.am_idx[blockIdx.x] = i;
    }
  }
}

template <bool BF16, int NCH, int KIND, int WPB = GEMV_WAVES>
__global__ __launch_bounds__(WPB * WAVE) void k_gemv(const GemvArgs a) {
  gemv_impl<BF16 ? WF_BF16 : WF_F32, NCH, KIND, WPB>(a);
}

template <int WF, int NCH, int KIND, int WPB = GEMV_WAVES>
__global__ __launch_bounds__(WPB * WAVE) void k_gemv_q(const GemvArgs a) {
  gemv_impl<WF, NCH, KIND, WPB>(a);
}

int argmax_block_rows() { return GEMV_WAVES * rows_per_wave(GEMV_NORM_ARGMAX); }

// Second pass of the greedy pick plus the bookkeeping that follows it (one block of 256):
//   FIN_CODE:      codes[j] = pick
//   FIN_FAST_NEXT: codes[j] = pick; x = codebook[j][pick]           (input of Fast step j+1)
//   FIN_FAST_LAST: codes[j] = pick; x = sum_k codebook[k][codes[k]] (Slow input, k ascending),
//                  snap = codes
//   FIN_SLOW:      codes[0] = pick; x = h (input of Fast step 1); pos += 1
template <bool BF16>
__global__ __launch_bounds__(256) void k_finish(const FinishArgs f) {
  __shared__ float red[4];
  __shared__ int bidx[4];
  __shared__ int s_code;
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
  float v = -INFINITY;
  int i = INT_MAX;
  for (int b = f.b0 + threadIdx.x; b <= f.b1; b += 256) {
    const float pv = f.am_val[b];
    const int pi = f.am_idx[b];
    if (pv > v || (pv == v && pi < i)) {
      v = pv;
      i = pi;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, WAVE);
    const int oi = __shfl_xor(i, o, WAVE);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
  if (lane == 0) {
    red[wid] = v;
    bidx[wid] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    v = red[0];
    i = bidx[0];
    for (int w = 1; w < 4; ++w)
      if (red[w] > v || (red[w] == v && bidx[w] < i)) {
        v = red[w];
        i = bidx[w];
      }
    s_code = (i == INT_MAX) ? 0 : i - f.lo;  // all-NaN logits: code 0 (the debug path flags it)
    // the stop id is a text id, below every semantic id, so it also wins a tie
    if (f.mode == FIN_SLOW && f.eos_at >= 0 && f.logits[f.eos_at] >= v) s_code = -1;
  }
  __syncthreads();
  // every block found the same pick; block b handles elements [256 b, 256 b + 256) of the next
  // input, block 0 the scalar bookkeeping (read before written: codes[j] is not read below)
  const int code = s_code;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (f.mode == FIN_FAST_NEXT) {
    if (e < f.H) f.x[e] = load_w<BF16>(f.codebook, ((size_t)f.j * f.K + code) * f.H + e);
  } else if (f.mode == FIN_FAST_LAST) {
    if (e < f.H) {
      float acc = 0.f;
      for (int k = 0; k < f.NC; ++k) {
        // c0 is -1 once the stream picked its stop id: the gather stays in bounds, the result is unused
        const int ck = min(max((k == f.j) ? code : f.codes[k], 0), f.K - 1);
        acc += load_w<BF16>(f.codebook, ((size_t)k * f.K + ck) * f.H + e);
      }
      f.x[e] = acc;
    }
    if (blockIdx.x == 0 && threadIdx.x < f.NC) f.snap[threadIdx.x] = (threadIdx.x == f.j) ? code : f.codes[threadIdx.x];
  } else if (f.mode == FIN_SLOW) {
    if (e < f.H) f.x[e] = f.h[e];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    f.codes[f.j] = code;
    if (f.mode == FIN_SLOW) f.pos[0] += 1;
  }
}

hipError_t launch_finish(bool bf16, const FinishArgs& f, hipStream_t s) {
  const dim3 grid(f.mode == FIN_CODE ? 1 : (f.H + 255) / 256);
  if (bf16) hipLaunchKernelGGL(k_finish<true>, grid, dim3(256), 0, s, f);
  else hipLaunchKernelGGL(k_finish<false>, grid, dim3(256), 0, s, f);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Grid-stride weight-streaming GEMV.  A tile is WPB wavefronts x R rows; block b walks tiles
// b, b + grid, ...  The next tile's weights are issued before the current tile is reduced
// (register double buffer), and the input is staged in LDS once per block.  The greedy-pick
// kind leaves one (max, argmax) per block, over all the rows the block visited.  PICK: the input is
// the codebook row of a head's greedy pick, whose second pass every block repeats after its first
// weight loads are issued (the partials and gains load first, so only the row gather waits behind
// the weights).
template <int WF, int NCH, int KIND, int R, int WPB, bool PICK = false>
__device__ __forceinline__ void gemv2_impl(const GemvArgs& a) {
  extern __shared__ float xs[];
  using F = WFmt<WF>;
  using CT = typename F::CT;
  constexpr int EPC = F::EPC;
  constexpr int NT = WPB * WAVE;
  constexpr int K = NCH * WAVE * EPC;
  constexpr int XL = (K + NT * 4 - 1) / (NT * 4);
  constexpr bool NORM = KIND != GEMV_RESID;
  constexpr int RPT = WPB * R;
  __shared__ float red[WPB];
  __shared__ int bidx[WPB];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  const int n_tiles = (a.N + RPT - 1) / RPT;
  int tile = blockIdx.x;
  if (tile >= n_tiles) return;
  constexpr size_t row_bytes = (size_t)K * F::ESZ;

  f32x4 xv[XL], gv[XL];
  constexpr int PKL = (2 * 4 * WAVE + NT - 1) / NT;  // pick partials per thread (at most 512 in all)
  float pv[PKL];
  int pi[PKL];
  if constexpr (PICK) {
#pragma unroll
    for (int u = 0; u < PKL; ++u) {
      const int b = u * NT + threadIdx.x;
      pv[u] = b < a.pk_n ? a.pk_val[a.pk_b0 + b] : -INFINITY;
      pi[u] = b < a.pk_n ? a.pk_idx[a.pk_b0 + b] : INT_MAX;
    }
  }
#pragma unroll
  for (int t = 0; t < XL; ++t) {
    const int k = (t * NT + threadIdx.x) * 4;
    if (XL * NT * 4 == K || k < K) {
      if constexpr (!PICK) xv[t] = *reinterpret_cast<const f32x4*>(a.x + k);
      if constexpr (NORM) gv[t] = *reinterpret_cast<const f32x4*>(a.gain + k);
    }
  }
  if constexpr (PICK) __builtin_amdgcn_sched_barrier(0);  // the partials and gains ahead of the weights
  CT wa[R][NCH], wb[R][NCH];
  float sa[R], sb[R];  // int8: the rows' scales, loaded with their weights
  auto issue = [&](CT (&wv)[R][NCH], float (&sv)[R], int tl) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(tl * RPT + wid * R + r, a.N - 1);
      const CT* wp = reinterpret_cast<const CT*>(static_cast<const char*>(a.w) + (size_t)row * row_bytes);
#pragma unroll
      for (int c = 0; c < NCH; ++c) wv[r][c] = __builtin_nontemporal_load(wp + c * WAVE + lane);
      sv[r] = (WF == WF_I8 || WF == WF_F8) ? a.wscale[row] : 1.f;
    }
  };
  issue(wa, sa, tile);
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (PICK) {
    __shared__ float pk_red[WPB];
    __shared__ int pk_bidx[WPB];
    float v = -INFINITY;
    int i = INT_MAX;
    auto take = [&](float ov, int oi) {
      if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
      }
    };
#pragma unroll
    for (int u = 0; u < PKL; ++u) take(pv[u], pi[u]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, WAVE);
      const int oi = __shfl_xor(i, o, WAVE);
      take(ov, oi);
    }
    if (lane == 0) {
      pk_red[wid] = v;
      pk_bidx[wid] = i;
    }
    __syncthreads();
    v = pk_red[0];
    i = pk_bidx[0];
#pragma unroll
    for (int w = 1; w < WPB; ++w) take(pk_red[w], pk_bidx[w]);
    const int code = i == INT_MAX ? 0 : i - a.pk_lo;
    const uint16_t* row = a.pk_codebook + ((size_t)a.pk_j * a.pk_ncb + code) * K;
    const bool keep_x = blockIdx.x == 0;
#pragma unroll
    for (int t = 0; t < XL; ++t) {
      const int k = (t * NT + threadIdx.x) * 4;
      if (XL * NT * 4 == K || k < K) {
        const uint2 raw = *reinterpret_cast<const uint2*>(row + k);
        xv[t] = f32x4{bf_one((uint16_t)(raw.x & 0xffffu)), bf_one((uint16_t)(raw.x >> 16)),
                      bf_one((uint16_t)(raw.y & 0xffffu)), bf_one((uint16_t)(raw.y >> 16))};
        if (keep_x) *reinterpret_cast<f32x4*>(a.pk_x + k) = xv[t];
      }
    }
    if (keep_x && threadIdx.x == 0) a.pk_codes[a.pk_j] = code;
  }

  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < XL; ++t) {
    const int k = (t * NT + threadIdx.x) * 4;
    if (XL * NT * 4 == K || k < K) {
      *reinterpret_cast<f32x4*>(xs + k) = xv[t];
      ss = fmaf(xv[t].x, xv[t].x, ss);
      ss = fmaf(xv[t].y, xv[t].y, ss);
      ss = fmaf(xv[t].z, xv[t].z, ss);
      ss = fmaf(xv[t].w, xv[t].w, ss);
    }
  }
  if constexpr (NORM) {
    ss = wave_sum(ss);
    if (lane == 0) red[wid] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) tot += red[w];
    const float scale = rsqrtf(tot / (float)K + a.eps);
    const bool keep = blockIdx.x == 0 && a.xnorm_out != nullptr;
#pragma unroll
    for (int t = 0; t < XL; ++t) {
      const int k = (t * NT + threadIdx.x) * 4;
      if (XL * NT * 4 == K || k < K) {
        f32x4 v = xv[t];
        v.x = v.x * scale * gv[t].x;
        v.y = v.y * scale * gv[t].y;
        v.z = v.z * scale * gv[t].z;
        v.w = v.w * scale * gv[t].w;
        *reinterpret_cast<f32x4*>(xs + k) = v;
        if (keep) *reinterpret_cast<f32x4*>(a.xnorm_out + k) = v;
      }
    }
  }
  __syncthreads();

  float bv = -INFINITY;
  int bi = INT_MAX;
  auto process = [&](CT (&wv)[R][NCH], const float (&sv)[R], int tl) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float* xp = xs + (c * WAVE + lane) * EPC;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = F::dot(wv[r][c], xp, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]) * sv[r];
    const int row0 = tl * RPT + wid * R;
    if constexpr (KIND == GEMV_NORM_STORE) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == r && row0 + r < a.N) a.y[row0 + r] = acc[r];
    } else if constexpr (KIND == GEMV_RESID) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == r && row0 + r < a.N) a.y[row0 + r] += acc[r];
    } else if constexpr (KIND == GEMV_NORM_SWIGLU) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
        if (lane == r && row0 + r + 1 < a.N) {
          const float gt = acc[r];
          a.y[(row0 + r) >> 1] = gt / (1.0f + expf(-gt)) * acc[r + 1];
        }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (lane == r && row < a.N) a.y[row] = acc[r];
        if (row >= a.am_lo && row < a.am_hi && row < a.N && acc[r] > bv) {
          bv = acc[r];
          bi = row;
        }
      }
    }
  };
  while (true) {
    const int t1 = tile + gridDim.x;
    if (t1 < n_tiles) issue(wb, sb, t1);
    process(wa, sa, tile);
    if (t1 >= n_tiles) break;
    const int t2 = t1 + gridDim.x;
    if (t2 < n_tiles) issue(wa, sa, t2);
    process(wb, sb, t1);
    if (t2 >= n_tiles) break;
    tile = t2;
  }
  if constexpr (KIND == GEMV_NORM_ARGMAX) {
    if (lane == 0) {
      red[wid] = bv;
      bidx[wid] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = red[0];
      int i = bidx[0];
      for (int w = 1; w < WPB; ++w)
        if (red[w] > v || (red[w] == v && bidx[w] < i)) {
          v = red[w];
          i = bidx[w];
        }
      a.am_val[blockIdx.x] = v;
      a.am_idx[blockIdx.x] = i;
    }
  }
}

template <bool BF16, int NCH, int KIND, int R, int WPB>
__global__ __launch_bounds__(WPB * WAVE) void k_gemv2(const GemvArgs a) {
  gemv2_impl<BF16 ? WF_BF16 : WF_F32, NCH, KIND, R, WPB>(a);
}

template <int WF, int NCH, int KIND, int R, int WPB>
__global__ __launch_bounds__(WPB * WAVE) void k_gemv2_q(const GemvArgs a) {
  gemv2_impl<WF, NCH, KIND, R, WPB>(a);
}

template <int WF, int NCH>
__global__ __launch_bounds__(8 * WAVE) void k_gemv2_pick(const GemvArgs a) {
  gemv2_impl<WF, NCH, GEMV_NORM_STORE, 1, 8, true>(a);
}

int pad_k(int K) { return (K + 1023) / 1024 * 1024; }

int gemv_blocks(int kind, int N) {
  const int rows = GEMV_WAVES * rows_per_wave(kind);
  return (N + rows - 1) / rows;
}

template <bool BF16, int KIND>
static hipError_t gemv_dispatch(const GemvArgs& a, hipStream_t s) {
  constexpr int EPC = BF16 ? 8 : 4;
  const dim3 grid(gemv_blocks(KIND, a.N)), block(GEMV_THREADS);
  const size_t lds = (size_t)pad_k(a.K) * sizeof(float);
  const int nch = (a.K % (WAVE * EPC) == 0) ? a.K / (WAVE * EPC) : -1;
#define S2_NCH(n) \
  case n:         \
    hipLaunchKernelGGL((k_gemv<BF16, n, KIND>), grid, block, lds, s, a); \
    return hipGetLastError();
  switch (nch) {
    S2_NCH(1)
    S2_NCH(2)
    S2_NCH(3)
    S2_NCH(4)
    S2_NCH(5)
    S2_NCH(6)
    S2_NCH(8)
    S2_NCH(12)
    S2_NCH(16)
    S2_NCH(19)
    default:
      hipLaunchKernelGGL((k_gemv<BF16, 0, KIND>), grid, block, lds, s, a);
      return hipGetLastError();
  }
#undef S2_NCH
}

template <int WF, int KIND>
static hipError_t gemv_dispatch_q(const GemvArgs& a, hipStream_t s) {
  const dim3 grid(gemv_blocks(KIND, a.N)), block(GEMV_THREADS);
  const size_t lds = (size_t)pad_k(a.K) * sizeof(float);
  const int nch = (a.K % (WAVE * 8) == 0) ? a.K / (WAVE * 8) : -1;
#define S2_NCH(n) \
  case n:         \
    hipLaunchKernelGGL((k_gemv_q<WF, n, KIND>), grid, block, lds, s, a); \
    return hipGetLastError();
  switch (nch) {
    S2_NCH(1)
    S2_NCH(2)
    S2_NCH(3)
    S2_NCH(4)
    S2_NCH(5)
    S2_NCH(6)
    S2_NCH(8)
    S2_NCH(12)
    S2_NCH(16)
    S2_NCH(19)
    default:
      hipLaunchKernelGGL((k_gemv_q<WF, 0, KIND>), grid, block, lds, s, a);
      return hipGetLastError();
  }
#undef S2_NCH
}

static int g_cus = 256;
void set_device_cus(int n) { g_cus = n > 0 ? n : 256; }
int device_cus() { return g_cus; }

// Launch shapes of the grid-stride kernel, picked per matrix shape on MI355X: it is used where it
// beat the one-shot kernel inside a whole frame (QKV and gate/up); the residual GEMVs (O, down) take
// the one-shot kernel, whose every wavefront issues all the loads of its row at once.
template <int NCH, int KIND, int R, int WPB>
static hipError_t gemv2_launch(const GemvArgs& a, int blocks_per_cu, hipStream_t s) {
  const int tiles = (a.N + R * WPB - 1) / (R * WPB);
  const int grid = std::min(tiles, g_cus * blocks_per_cu);
  hipLaunchKernelGGL((k_gemv2<true, NCH, KIND, R, WPB>), dim3(grid), dim3(WPB * WAVE), (size_t)pad_k(a.K) * 4, s, a);
  return hipGetLastError();
}

template <int WF, int NCH, int KIND, int R, int WPB>
static hipError_t gemv2_launch_q(const GemvArgs& a, int blocks_per_cu, hipStream_t s) {
  const int tiles = (a.N + R * WPB - 1) / (R * WPB);
  const int grid = std::min(tiles, g_cus * blocks_per_cu);
  hipLaunchKernelGGL((k_gemv2_q<WF, NCH, KIND, R, WPB>), dim3(grid), dim3(WPB * WAVE), (size_t)pad_k(a.K) * 4, s, a);
  return hipGetLastError();
}

bool gemv_pick_fits(int K, int n_partials) {
  return (K == 2 * WAVE * 8 || K == 5 * WAVE * 8) && n_partials >= 1 && n_partials <= 2 * 4 * WAVE;
}

hipError_t launch_gemv_pick(const GemvArgs& a, hipStream_t s) {
  if (!gemv_pick_fits(a.K, a.pk_n) || !a.pk_val || !a.pk_idx || !a.pk_codebook || !a.pk_codes || !a.pk_x ||
      a.pk_j < 0 || a.pk_ncb < 1)
    return hipErrorInvalidValue;
  const int tiles = (a.N + 8 - 1) / 8;
  const int grid = std::min(tiles, g_cus);  // the launch shape of the plain QKV GEMV
  const size_t lds = (size_t)pad_k(a.K) * 4;
  const bool k5 = a.K == 5 * WAVE * 8;  // else 2 chunks (K 1024); bf16 and 8-bit codes take 8 per lane
#define S2_PK(WF)                                                                                         \
  if (k5) hipLaunchKernelGGL((k_gemv2_pick<WF, 5>), dim3(grid), dim3(8 * WAVE), lds, s, a);              \
  else hipLaunchKernelGGL((k_gemv2_pick<WF, 2>), dim3(grid), dim3(8 * WAVE), lds, s, a);
  if (!a.wscale) { S2_PK(WF_BF16) }
  else if (a.w_f8) { S2_PK(WF_F8) }
  else { S2_PK(WF_I8) }
#undef S2_PK
  return hipGetLastError();
}

// 8-bit weights with per-row scales (int8 or FP8 E4M3), the launch shapes of the bf16 kernels
template <int WF>
static hipError_t launch_gemv_q(int kind, const GemvArgs& a, hipStream_t s) {
  const int nch = a.K % (WAVE * 8) == 0 ? a.K / (WAVE * 8) : -1;
  if (kind == GEMV_NORM_STORE && nch == 5) return gemv2_launch_q<WF, 5, GEMV_NORM_STORE, 1, 8>(a, 1, s);
  if (kind == GEMV_NORM_SWIGLU && nch == 5) return gemv2_launch_q<WF, 5, GEMV_NORM_SWIGLU, 2, 8>(a, 1, s);
  // O and down: one block of 10 wavefronts per CU, as for bf16 weights
  if (kind == GEMV_RESID && a.N % (10 * g_cus) == 0 && (nch == 8 || nch == 19)) {
    const dim3 grid(a.N / 10), block(10 * WAVE);
    const size_t lds = (size_t)pad_k(a.K) * sizeof(float);
    if (nch == 8) hipLaunchKernelGGL((k_gemv_q<WF, 8, GEMV_RESID, 10>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_gemv_q<WF, 19, GEMV_RESID, 10>), grid, block, lds, s, a);
    return hipGetLastError();
  }
  switch (kind) {
    case GEMV_NORM_STORE: return gemv_dispatch_q<WF, GEMV_NORM_STORE>(a, s);
    case GEMV_RESID: return gemv_dispatch_q<WF, GEMV_RESID>(a, s);
    case GEMV_NORM_SWIGLU: return gemv_dispatch_q<WF, GEMV_NORM_SWIGLU>(a, s);
    case GEMV_NORM_ARGMAX: return gemv_dispatch_q<WF, GEMV_NORM_ARGMAX>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int kind, bool bf16, const GemvArgs& a, hipStream_t s) {
  if (a.wscale) {
    if (a.K % 8) return hipErrorInvalidValue;
    return a.w_f8 ? launch_gemv_q<WF_F8>(kind, a, s) : launch_gemv_q<WF_I8>(kind, a, s);
  }
  if (bf16 && a.K % (WAVE * 8) == 0) {
    const int nch = a.K / (WAVE * 8);
    // QKV and gate/up: one block of 8 wavefronts per CU, which stages the input once per CU (two
    // blocks of 4 per CU: 273.7 against 274.8 frames/s at the S2 shape)
    if (kind == GEMV_NORM_STORE && nch == 5) return gemv2_launch<5, GEMV_NORM_STORE, 1, 8>(a, 1, s);
    if (kind == GEMV_NORM_SWIGLU && nch == 5) return gemv2_launch<5, GEMV_NORM_SWIGLU, 2, 8>(a, 1, s);
    // residual projections of 2560 rows (O, down at the S2 shape): blocks of 10 wavefronts, one row
    // each, so the 256 blocks sit exactly one per CU (4-wavefront blocks leave 2.5 per CU, and the
    // CUs holding three set the launch's length: 267.3 -> 271.9 frames/s with 5-wavefront blocks;
    // 10 wavefronts halve the input staged per CU again: 272.7 -> 274.1)
    if (kind == GEMV_RESID && a.N % (10 * g_cus) == 0 && (nch == 8 || nch == 19)) {
      const dim3 grid(a.N / 10), block(10 * WAVE);
      const size_t lds = (size_t)pad_k(a.K) * sizeof(float);
      if (nch == 8) hipLaunchKernelGGL((k_gemv<true, 8, GEMV_RESID, 10>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((k_gemv<true, 19, GEMV_RESID, 10>), grid, block, lds, s, a);
      return hipGetLastError();
    }
  }
  switch (kind) {
    case GEMV_NORM_STORE: return bf16 ? gemv_dispatch<true, GEMV_NORM_STORE>(a, s) : gemv_dispatch<false, GEMV_NORM_STORE>(a, s);
    case GEMV_RESID: return bf16 ? gemv_dispatch<true, GEMV_RESID>(a, s) : gemv_dispatch<false, GEMV_RESID>(a, s);
    case GEMV_NORM_SWIGLU: return bf16 ? gemv_dispatch<true, GEMV_NORM_SWIGLU>(a, s) : gemv_dispatch<false, GEMV_NORM_SWIGLU>(a, s);
    case GEMV_NORM_ARGMAX: return bf16 ? gemv_dispatch<true, GEMV_NORM_ARGMAX>(a, s) : gemv_dispatch<false, GEMV_NORM_ARGMAX>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------
// Decode attention.  grid = (max_splits, Hkv, M), block = G wavefronts (G = Hq / Hkv), one per
// q head of the KV group.  A block walks its split in chunks of 64 positions (one per lane):
// the chunk's K and V rows are staged in LDS (the next chunk's loads are already in flight in
// registers), scores use the lane's row, and the running softmax is rescaled per chunk.

template <bool KVB>
struct KvT;
template <>
struct KvT<true> {
  using T = uint16_t;
  static __device__ __forceinline__ float ld(const T* p, size_t i) { return bf_one(p[i]); }
  static __device__ __forceinline__ T cvt(float f) { return f2bf(f); }
  static __device__ __forceinline__ float round(float f) { return bf_one(f2bf(f)); }
};
template <>
struct KvT<false> {
  using T = float;
  static __device__ __forceinline__ float ld(const T* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ T cvt(float f) { return f; }
  static __device__ __forceinline__ float round(float f) { return f; }
};

// rotate-half RoPE of one head held as PER values per lane (element d = lane + 64 i); the
// partner of element d is d +- D/2: the same lane when D = 128, lane ^ 32 when D = 64
template <int D>
__device__ __forceinline__ void rope_lane(float (&v)[D / WAVE], const float* crow, const float* srow, int lane) {
  if constexpr (D == 128) {
    const float cs = crow[lane], sn = srow[lane];
    const float x0 = v[0], x1 = v[1];
    v[0] = x0 * cs - x1 * sn;
    v[1] = x1 * cs + x0 * sn;
  } else {
    const int i = lane & 31;
    const float cs = crow[i], sn = srow[i];
    const float partner = __shfl_xor(v[0], 32, WAVE);
    v[0] = lane < 32 ? v[0] * cs - partner * sn : v[0] * cs + partner * sn;
  }
}

template <int D, int G, bool KB, bool VB>
__global__ __launch_bounds__(G * WAVE) void k_attn(const AttnArgs a) {
  using KK = KvT<KB>;
  using VV = KvT<VB>;
  using TK = typename KK::T;
  using TV = typename VV::T;
  constexpr int CH = WAVE;                   // positions per chunk, one per lane in the scores
  constexpr int NT = G * WAVE;               // threads
  constexpr int KSTR = KB ? D + 8 : D + 4;   // K row padded by one 16-byte piece: 16-byte aligned rows
                                             // whose 16-byte reads by consecutive lanes spread over the banks
  constexpr int PER = D / WAVE;
  constexpr int EPK = 16 / sizeof(TK);       // elements per 16-byte piece of a key / value row
  constexpr int EPV = 16 / sizeof(TV);
  constexpr int CPRK = D / EPK;              // 16-byte pieces per key / value row
  constexpr int CPRV = D / EPV;
  constexpr int PK = CH * CPRK / NT;         // key / value pieces per thread per chunk
  constexpr int PV = CH * CPRV / NT;
  constexpr int MAXSPLIT = 256;
  constexpr int MAXPG = MAXSPLIT / 16;       // pages of one split (page size 16)
  static_assert(CH * CPRK % NT == 0 && CH * CPRV % NT == 0, "tile pieces must divide evenly");
  __shared__ __attribute__((aligned(16))) float q_s[G][D];
  __shared__ float kn_s[D];
  __shared__ float vn_s[D];
  __shared__ __attribute__((aligned(16))) TK k_s[CH * KSTR];
  __shared__ __attribute__((aligned(16))) TV v_s[CH * D];
  __shared__ float p_s[G][CH];
  __shared__ int rowoff_s[MAXSPLIT];
  __shared__ int page_s[MAXPG];

  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  const int slot = a.fixed_slot >= 0 ? a.fixed_slot : a.slots[b];
  const int s0 = sp * a.split;
  // The position and the page-table entries of this split's (at most 16) pages do not depend on
  // each other: both loads go out together, so the cache offsets cost one round trip after the
  // slot.  Entries past the stream's last page are read (in bounds of the table) but never used.
  const int pg0 = s0 / a.page_size;
  int pg = 0;
  if (threadIdx.x < MAXPG && pg0 + (int)threadIdx.x < a.bt_stride)
    pg = a.block_table[slot * a.bt_stride + pg0 + threadIdx.x];
  // a single q|k|v row (batch 1) is read before the position too: its q head is needed whatever
  // the position is (split partials, summed below, wait for the early exit instead)
  constexpr int PERQ = D / WAVE;
  float qv[PERQ];
  if (a.qkv_S == 0) {
    const float* qrow = a.qkv + (size_t)b * (a.Hq + 2 * a.Hkv) * D + (size_t)(g * G + w) * D;
#pragma unroll
    for (int i = 0; i < PERQ; ++i) qv[i] = qrow[lane + i * WAVE];
  }
  const int pos = a.const_pos >= 0 ? a.const_pos : (a.row_pos ? a.row_pos[b] : a.pos[slot]);
  const int ctx = pos + 1;
  const int nsplit = (ctx + a.split - 1) / a.split;
  if (sp >= nsplit) return;
  const int s1 = min(s0 + a.split, ctx);
  const bool has_new = a.append && pos >= s0 && pos < s1;
  const int h = g * G + w;
  const float* qkv = a.qkv + (size_t)b * (a.Hq + 2 * a.Hkv) * D;
  TK* kc = static_cast<TK*>(a.k_cache);
  TV* vc = static_cast<TV*>(a.v_cache);
  if (threadIdx.x < MAXPG) page_s[threadIdx.x] = pg;

  // this wave's q head (and, for wave 0 of the split holding pos, the new k and v): elements
  // n[i] of this row's q | k | v vector, each the sum of the split partials in split order; every
  // partial of every element is loaded before the first add
  auto qkv_sum = [&](const int* n, float* out, int cnt) {
    if (a.qkv_S == 0) {
      for (int i = 0; i < cnt; ++i) out[i] = qkv[n[i]];
      return;
    }
    const float* p = a.qkv_part + (size_t)b * a.qkv_ldp;
    const size_t st = (size_t)16 * a.qkv_ldp;
    for (int i = 0; i < cnt; ++i) out[i] = 0.f;
    for (int s0 = 0; s0 < a.qkv_S; s0 += 8) {
      float t[2 * PER][8];
#pragma unroll
      for (int i = 0; i < 2 * PER; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u) t[i][u] = (i < cnt && s0 + u < a.qkv_S) ? p[(s0 + u) * st + n[i]] : 0.f;
#pragma unroll
      for (int i = 0; i < 2 * PER; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i < cnt && s0 + u < a.qkv_S) out[i] += t[i][u];
    }
  };
  float kv[PER], vv[PER];
  if (a.qkv_S != 0) {
    int n[2 * PER];
    float o[2 * PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) n[i] = h * D + lane + i * WAVE;
    qkv_sum(n, o, PER);
#pragma unroll
    for (int i = 0; i < PER; ++i) qv[i] = o[i];
  }
  const bool mk = has_new && w == 0;
  if (mk) {
    int n[2 * PER];
    float o[2 * PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      n[i] = (a.Hq + g) * D + lane + i * WAVE;
      n[PER + i] = (a.Hq + a.Hkv + g) * D + lane + i * WAVE;
    }
    qkv_sum(n, o, 2 * PER);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      kv[i] = o[i];
      vv[i] = o[PER + i];
    }
  }
  __syncthreads();
  // cache offsets of every position of the split
  for (int t = threadIdx.x; t < s1 - s0; t += NT) {
    const int jj = s0 + t;
    rowoff_s[t] = (int)((((size_t)page_s[jj / a.page_size - pg0] * a.Hkv + g) * a.page_size + jj % a.page_size) * D);
  }
  __syncthreads();

  // K and V pieces of one chunk: issued a chunk ahead, so the loads of chunk c + 1 are in flight
  // while chunk c is scored and accumulated
  u32x4 kt[PK], vt[PV];
  auto issue = [&](int j0) {
    const int nv = min(CH, s1 - j0);
    const int jn = has_new ? pos - j0 : -1;  // the new position is not in the cache yet
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int pi = threadIdx.x + u * NT, j = pi / CPRK, q = pi % CPRK;
      if (j < nv && j != jn) kt[u] = *reinterpret_cast<const u32x4*>(kc + rowoff_s[j0 - s0 + j] + q * EPK);
    }
#pragma unroll
    for (int u = 0; u < PV; ++u) {
      const int pi = threadIdx.x + u * NT, j = pi / CPRV, q = pi % CPRV;
      if (j < nv && j != jn) vt[u] = *reinterpret_cast<const u32x4*>(vc + rowoff_s[j0 - s0 + j] + q * EPV);
    }
  };
  issue(s0);
  {  // QK-norm and RoPE while the first tile is in flight
    const float* crow = a.rope_cos + (size_t)pos * (D / 2);
    const float* srow = a.rope_sin + (size_t)pos * (D / 2);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) ss = fmaf(qv[i], qv[i], ss);
    const float r = rsqrtf(wave_sum(ss) / (float)D + a.eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) qv[i] = qv[i] * r * a.q_norm[lane + i * WAVE];
    rope_lane<D>(qv, crow, srow, lane);
#pragma unroll
    for (int i = 0; i < PER; ++i) q_s[w][lane + i * WAVE] = qv[i] * a.scale;
    if (mk) {
      ss = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) ss = fmaf(kv[i], kv[i], ss);
      const float rk = rsqrtf(wave_sum(ss) / (float)D + a.eps);
#pragma unroll
      for (int i = 0; i < PER; ++i) kv[i] = kv[i] * rk * a.k_norm[lane + i * WAVE];
      rope_lane<D>(kv, crow, srow, lane);
      const int page = page_s[pos / a.page_size - pg0];
      const size_t off = (((size_t)page * a.Hkv + g) * a.page_size + pos % a.page_size) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int d = lane + i * WAVE;
        kn_s[d] = KK::round(kv[i]);
        vn_s[d] = VV::round(vv[i]);
        kc[off + d] = KK::cvt(kv[i]);  // append the new position to the paged cache
        vc[off + d] = VV::cvt(vv[i]);
      }
    }
  }

  // Scores: lane j dots q with key j, reading the key row 16 bytes at a time into four partial sums
  // (added in a fixed order).  Weighted sum: the lanes split into KG key groups x DG groups of eight
  // dimensions; lane (kg, dg) accumulates keys kg, kg + KG, ... over its eight dimensions (one
  // 16-byte V read per key for bf16), and the key groups are added by a butterfly at the end.
  constexpr int DG = D / 8, KG = WAVE / DG;
  const int dg = lane % DG, kg = lane / DG;
  float m_run = -INFINITY, l_run = 0.f, o8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o8[e] = 0.f;
  for (int j0 = s0; j0 < s1; j0 += CH) {
    const int nv = min(CH, s1 - j0);
    const int jn = has_new ? pos - j0 : -1;  // row of the new position in this chunk (if any)
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int pi = threadIdx.x + u * NT, j = pi / CPRK, q = pi % CPRK;
      if (j < nv && j != jn) *reinterpret_cast<u32x4*>(k_s + j * KSTR + q * EPK) = kt[u];
    }
#pragma unroll
    for (int u = 0; u < PV; ++u) {
      const int pi = threadIdx.x + u * NT, j = pi / CPRV, q = pi % CPRV;
      if (j < nv && j != jn) *reinterpret_cast<u32x4*>(v_s + j * D + q * EPV) = vt[u];
    }
    if (mk && jn >= 0 && jn < nv)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int d = lane + i * WAVE;
        k_s[jn * KSTR + d] = KK::cvt(kn_s[d]);
        v_s[jn * D + d] = VV::cvt(vn_s[d]);
      }
    __syncthreads();
    if (j0 + CH < s1) issue(j0 + CH);

    float s = -INFINITY;
    if (lane < nv) {
      const TK* kr = k_s + lane * KSTR;
      const float* qr = q_s[w];
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / EPK; ++c) {
        const u32x4 kp = *reinterpret_cast<const u32x4*>(kr + c * EPK);
        if constexpr (KB) {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(qr + c * 8);
          const f32x4 qb = *reinterpret_cast<const f32x4*>(qr + c * 8 + 4);
          float t = acc[c & 3];
          t = fmaf(qa.x, bf_lo(kp.x), t);
          t = fmaf(qa.y, bf_hi(kp.x), t);
          t = fmaf(qa.z, bf_lo(kp.y), t);
          t = fmaf(qa.w, bf_hi(kp.y), t);
          t = fmaf(qb.x, bf_lo(kp.z), t);
          t = fmaf(qb.y, bf_hi(kp.z), t);
          t = fmaf(qb.z, bf_lo(kp.w), t);
          t = fmaf(qb.w, bf_hi(kp.w), t);
          acc[c & 3] = t;
        } else {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(qr + c * 4);
          float t = acc[c & 3];
          t = fmaf(qa.x, __uint_as_float(kp.x), t);
          t = fmaf(qa.y, __uint_as_float(kp.y), t);
          t = fmaf(qa.z, __uint_as_float(kp.z), t);
          t = fmaf(qa.w, __uint_as_float(kp.w), t);
          acc[c & 3] = t;
        }
      }
      s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float p = (lane < nv) ? expf(s - m_new) : 0.f;
    const float corr = expf(m_run - m_new);
    l_run = l_run * corr + wave_sum(p);
    p_s[w][lane] = p;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] *= corr;
    for (int j = kg; j < nv; j += KG) {
      const float pj = p_s[w][j];
      const TV* vr = v_s + (size_t)j * D + dg * 8;
      if constexpr (VB) {
        const u32x4 vp = *reinterpret_cast<const u32x4*>(vr);
        o8[0] = fmaf(pj, bf_lo(vp.x), o8[0]);
        o8[1] = fmaf(pj, bf_hi(vp.x), o8[1]);
        o8[2] = fmaf(pj, bf_lo(vp.y), o8[2]);
        o8[3] = fmaf(pj, bf_hi(vp.y), o8[3]);
        o8[4] = fmaf(pj, bf_lo(vp.z), o8[4]);
        o8[5] = fmaf(pj, bf_hi(vp.z), o8[5]);
        o8[6] = fmaf(pj, bf_lo(vp.w), o8[6]);
        o8[7] = fmaf(pj, bf_hi(vp.w), o8[7]);
      } else {
        const f32x4 va = *reinterpret_cast<const f32x4*>(vr);
        const f32x4 vb = *reinterpret_cast<const f32x4*>(vr + 4);
        o8[0] = fmaf(pj, va.x, o8[0]);
        o8[1] = fmaf(pj, va.y, o8[1]);
        o8[2] = fmaf(pj, va.z, o8[2]);
        o8[3] = fmaf(pj, va.w, o8[3]);
        o8[4] = fmaf(pj, vb.x, o8[4]);
        o8[5] = fmaf(pj, vb.y, o8[5]);
        o8[6] = fmaf(pj, vb.z, o8[6]);
        o8[7] = fmaf(pj, vb.w, o8[7]);
      }
    }
    m_run = m_new;
    __syncthreads();
  }
  // add the key groups (a fixed butterfly: every lane of a dimension group ends with the same sum)
#pragma unroll
  for (int o = DG; o < WAVE; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] += __shfl_xor(o8[e], o, WAVE);

  if (nsplit == 1) {
    if (kg == 0) {
      float* out = a.out + ((size_t)b * a.Hq + h) * D + dg * 8;
      const float inv = 1.0f / l_run;
      *reinterpret_cast<f32x4*>(out) = f32x4{o8[0] * inv, o8[1] * inv, o8[2] * inv, o8[3] * inv};
      *reinterpret_cast<f32x4*>(out + 4) = f32x4{o8[4] * inv, o8[5] * inv, o8[6] * inv, o8[7] * inv};
    }
    return;
  }
  const size_t pi = ((size_t)b * a.Hq + h) * a.max_splits + sp;
  if (lane == 0) {
    a.part_ml[pi * 2] = m_run;
    a.part_ml[pi * 2 + 1] = l_run;
  }
  if (kg == 0) {
    float* po = a.part_o + pi * D + dg * 8;
    *reinterpret_cast<f32x4*>(po) = f32x4{o8[0], o8[1], o8[2], o8[3]};
    *reinterpret_cast<f32x4*>(po + 4) = f32x4{o8[4], o8[5], o8[6], o8[7]};
  }
}

// Merge the splits of every q head in split order.  grid = (Hq, M), one wavefront each.
template <int D>
__global__ __launch_bounds__(WAVE) void k_attn_combine(const AttnArgs a) {
  constexpr int PER = D / WAVE;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int pos = a.const_pos >= 0 ? a.const_pos
                                   : (a.row_pos ? a.row_pos[b] : a.pos[a.fixed_slot >= 0 ? a.fixed_slot : a.slots[b]]);
  const int nsplit = (pos + 1 + a.split - 1) / a.split;
  if (nsplit == 1) return;  // the attention kernel wrote the output itself
  const size_t base = ((size_t)b * a.Hq + h) * a.max_splits;
  // the first 16 splits' outputs are loaded before anything else (they do not depend on the max)
  constexpr int SF = 16;
  float tf[SF][PER];
#pragma unroll
  for (int u = 0; u < SF; ++u)
#pragma unroll
    for (int i = 0; i < PER; ++i) tf[u][i] = u < nsplit ? a.part_o[(base + u) * D + lane + i * WAVE] : 0.f;
  // the splits' (max, sum) are read one split per lane, 64 at a time, and each split's weight is
  // passed from its lane; the sums still run in split order, so the loads of up to eight splits'
  // outputs go out together instead of one dependent round trip per split
  float M = -INFINITY;
  for (int c0 = 0; c0 < nsplit; c0 += WAVE)
    if (c0 + lane < nsplit) M = fmaxf(M, a.part_ml[(base + c0 + lane) * 2]);
  M = wave_max(M);
  float L = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += WAVE) {
    const int cn = min(WAVE, nsplit - c0);
    float e = 0.f, l = 0.f;
    if (lane < cn) {
      e = expf(a.part_ml[(base + c0 + lane) * 2] - M);
      l = a.part_ml[(base + c0 + lane) * 2 + 1];
    }
    int u0 = 0;
    if (c0 == 0) {  // splits 0 .. SF - 1, loaded up front
#pragma unroll
      for (int u = 0; u < SF; ++u) {
        const float eu = __shfl(e, u, WAVE), lu = __shfl(l, u, WAVE);
        if (u < cn) {
          L = fmaf(eu, lu, L);
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] = fmaf(eu, tf[u][i], acc[i]);
        }
      }
      u0 = SF;
    }
    for (; u0 < cn; u0 += 8) {
      float t[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < PER; ++i)
          t[u][i] = (u0 + u < cn) ? a.part_o[(base + c0 + u0 + u) * D + lane + i * WAVE] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float eu = __shfl(e, u0 + u, WAVE), lu = __shfl(l, u0 + u, WAVE);
        if (u0 + u < cn) {
          L = fmaf(eu, lu, L);
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] = fmaf(eu, t[u][i], acc[i]);
        }
      }
    }
  }
  float* out = a.out + ((size_t)b * a.Hq + h) * D;
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) out[lane + i * WAVE] = acc[i] * inv;
}

// ---------------------------------------------------------------------------------------------
// Decode attention over long paged contexts (the batched multi-stream step).  grid = (splits of
// LONG_SPLIT keys, Hkv, M), block = 4 wavefronts; wavefront w takes keys s0 + 64 w .. + 63 of its
// split.  Nothing is staged in LDS: every load reads cache rows straight into registers, LPK
// adjacent lanes covering one row 16 bytes each, so a load instruction reads KPI whole rows (one
// contiguous run of a page).
//   Scores: lane (r, c) holds the q slice of its 16-byte column c for the G heads of the KV group
// (read once from LDS) and forms partial dot products; a reduce-scatter over the LPK lanes of a
// row (halving exchanges, one shuffle per retained value) leaves lane (r, c) with the whole score
// of key KPI c + r.  The loads go in groups of four, the next group in flight while one is used.
//   Weighted sum: lane (rv, cv) accumulates dimensions cv EPV .. + EPV of the keys KPV i + rv,
// the weights read from LDS, then the KPV key lanes are added by shuffles.
//   Each wavefront keeps one softmax state per head over its 64 keys; the four wavefronts' (max,
// sum, output) merge in LDS in wavefront order.
constexpr int LONG_SPLIT = 256;
constexpr int kBufWord3 = 0x00020000;  // fourth descriptor word of a raw (untyped) gfx9 buffer
constexpr int kNonTemp = 2;            // nontemporal cache policy of a buffer load

template <int D, int G, bool KB, bool VB>
__global__ __launch_bounds__(256, 4) void k_attn_long(const AttnArgs a) {
  using KK = KvT<KB>;
  using VV = KvT<VB>;
  using TK = typename KK::T;
  using TV = typename VV::T;
  constexpr int NW = 4, CH = WAVE, PER = D / WAVE, PS = 16;
  constexpr int EPK = 16 / sizeof(TK), LPK = D / EPK, KPI = WAVE / LPK, NI = LPK;
  constexpr int QK = 4, RK = NI / QK;  // key loads per group, groups
  constexpr int EPV = 16 / sizeof(TV), LPV = D / EPV, KPV = WAVE / LPV, NIV = LPV;
  constexpr int QV = 4, RV = NIV / QV;
  static_assert(KPI <= PS && PS % KPI == 0 && KPV <= PS && PS % KPV == 0, "load rows inside one page");
  static_assert(RK >= 1 && RV >= 1 && G <= NW, "shape");
  __shared__ __attribute__((aligned(16))) float q_s[G][D];
  __shared__ __attribute__((aligned(16))) float kn_s[D];
  __shared__ __attribute__((aligned(16))) float vn_s[D];
  __shared__ __attribute__((aligned(16))) float p_s[NW][CH][G];
  __shared__ float m_s[NW][G], l_s[NW][G];
  __shared__ __attribute__((aligned(16))) float o_s[NW][G][D];

  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int r = lane / LPK, c = lane % LPK;
  const int rv = lane / LPV, cv = lane % LPV;
  // values the whole block shares, read by vector loads (the kernel writes global memory): marked
  // wave-uniform so that the buffer resources built from them stay in scalar registers
  const int slot = __builtin_amdgcn_readfirstlane(a.fixed_slot >= 0 ? a.fixed_slot : a.slots[b]);
  const int s0 = sp * LONG_SPLIT, k0 = s0 + CH * w;
  // this wavefront's four page-table entries (read in bounds of the table, used below ctx only)
  int pgw[CH / PS];
#pragma unroll
  for (int q = 0; q < CH / PS; ++q) {
    const int pi = k0 / PS + q;
    pgw[q] = __builtin_amdgcn_readfirstlane(pi < a.bt_stride ? a.block_table[slot * a.bt_stride + pi] : 0);
  }
  const int pos = __builtin_amdgcn_readfirstlane(a.const_pos >= 0 ? a.const_pos : (a.row_pos ? a.row_pos[b] : a.pos[slot]));
  const int ctx = pos + 1;
  const int nsplit = (ctx + LONG_SPLIT - 1) / LONG_SPLIT;
  if (sp >= nsplit) return;
  const int s1 = min(s0 + LONG_SPLIT, ctx);
  const bool has_new = a.append && pos >= s0 && pos < s1;
  const int nk = max(0, min(CH, s1 - k0));   // keys of this wavefront
  const int jn = has_new ? pos - k0 : -1;    // the new position, relative to k0
  TK* kc = static_cast<TK*>(a.k_cache);
  TV* vc = static_cast<TV*>(a.v_cache);
  // One buffer resource per page of this wavefront: the page's 16 rows of this KV head, cut at
  // the end of the split's cached keys (the new position, appended by this kernel, is not read
  // back), so loads past it return zeros without touching memory.
  const int e1 = has_new ? pos : s1;
  __amdgpu_buffer_rsrc_t kr_[CH / PS], vr_[CH / PS];
#pragma unroll
  for (int q = 0; q < CH / PS; ++q) {
    const int rows = max(0, min(PS, e1 - (k0 + q * PS)));
    const size_t base = ((size_t)(rows > 0 ? pgw[q] : 0) * a.Hkv + g) * PS * D;
    kr_[q] = __builtin_amdgcn_make_buffer_rsrc(kc + base, (short)0, rows * D * (int)sizeof(TK), kBufWord3);
    vr_[q] = __builtin_amdgcn_make_buffer_rsrc(vc + base, (short)0, rows * D * (int)sizeof(TV), kBufWord3);
  }
  // lane byte offsets inside a page; the whole offset goes in the vector operand (the scalar
  // offset is left 0), which is what the range check covers
  const int koff = (r * D + c * EPK) * (int)sizeof(TK), voff = (rv * D + cv * EPV) * (int)sizeof(TV);
  // key loads: group j holds instructions j, j + RK, j + 2 RK, j + 3 RK; instruction i reads rows
  // KPI i .. KPI i + KPI - 1 of the wavefront's keys
  auto kload = [&](u32x4 (&buf)[QK], int j) {
#pragma unroll
    for (int t = 0; t < QK; ++t) {
      const int k = KPI * (j + RK * t);
      buf[t] = __builtin_amdgcn_raw_buffer_load_b128(kr_[k / PS], koff + (k % PS) * D * (int)sizeof(TK), 0, kNonTemp);
    }
  };
  u32x4 kb[2][QK];
  kload(kb[0], 0);
  if constexpr (RK > 1) kload(kb[1], 1);

  // element n of this batch row's q | k | v vector: the qkv row, or the sum of the split-K partials
  // in split order
  auto qkv_elem = [&](int n, float (&out)[PER]) {
    if (a.qkv_S == 0) {
      const float* qrow = a.qkv + (size_t)b * (a.Hq + 2 * a.Hkv) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) out[i] = qrow[n + i * WAVE];
      return;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) out[i] = 0.f;
    const float* p = a.qkv_part + (size_t)b * a.qkv_ldp;
    const size_t st = (size_t)16 * a.qkv_ldp;
    for (int s8 = 0; s8 < a.qkv_S; s8 += 8) {
      float t[PER][8];
#pragma unroll
      for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u) t[i][u] = (s8 + u < a.qkv_S) ? p[(s8 + u) * st + n + i * WAVE] : 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s8 + u < a.qkv_S) out[i] += t[i][u];
    }
  };
  const float* crow = a.rope_cos + (size_t)pos * (D / 2);
  const float* srow = a.rope_sin + (size_t)pos * (D / 2);
  if (w < G) {  // q head g G + w: QK-norm, RoPE, scale
    float qv[PER];
    qkv_elem((g * G + w) * D + lane, qv);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) ss = fmaf(qv[i], qv[i], ss);
    const float rq = rsqrtf(wave_sum(ss) / (float)D + a.eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) qv[i] = qv[i] * rq * a.q_norm[lane + i * WAVE];
    rope_lane<D>(qv, crow, srow, lane);
#pragma unroll
    for (int i = 0; i < PER; ++i) q_s[w][lane + i * WAVE] = qv[i] * a.scale;
  }
  if (has_new && w == NW - 1) {  // the new key (QK-norm, RoPE) and value, appended to the cache
    float kv[PER], vv[PER];
    qkv_elem((a.Hq + g) * D + lane, kv);
    qkv_elem((a.Hq + a.Hkv + g) * D + lane, vv);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) ss = fmaf(kv[i], kv[i], ss);
    const float rk = rsqrtf(wave_sum(ss) / (float)D + a.eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) kv[i] = kv[i] * rk * a.k_norm[lane + i * WAVE];
    rope_lane<D>(kv, crow, srow, lane);
    const size_t off = (((size_t)a.block_table[slot * a.bt_stride + pos / PS] * a.Hkv + g) * PS + pos % PS) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + i * WAVE;
      kn_s[d] = KK::round(kv[i]);
      vn_s[d] = VV::round(vv[i]);
      kc[off + d] = KK::cvt(kv[i]);
      vc[off + d] = VV::cvt(vv[i]);
    }
  }
  __syncthreads();

  // ---- scores
  float qf[G][EPK];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPK; e += 4) {
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(&q_s[h][c * EPK + e]);
      qf[h][e] = q4.x;
      qf[h][e + 1] = q4.y;
      qf[h][e + 2] = q4.z;
      qf[h][e + 3] = q4.w;
    }
  float ret[RK][G];
#pragma unroll
  for (int j = 0; j < RK; ++j) {
    float v[QK][G];
#pragma unroll
    for (int t = 0; t < QK; ++t) {
      float kx[EPK];
      const u32x4 kr = kb[j & 1][t];
      if constexpr (KB) {
        kx[0] = bf_lo(kr.x); kx[1] = bf_hi(kr.x); kx[2] = bf_lo(kr.y); kx[3] = bf_hi(kr.y);
        kx[4] = bf_lo(kr.z); kx[5] = bf_hi(kr.z); kx[6] = bf_lo(kr.w); kx[7] = bf_hi(kr.w);
      } else {
        kx[0] = __uint_as_float(kr.x); kx[1] = __uint_as_float(kr.y);
        kx[2] = __uint_as_float(kr.z); kx[3] = __uint_as_float(kr.w);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPK; ++e) acc = fmaf(qf[h][e], kx[e], acc);
        v[t][h] = acc;
      }
    }
    if (j + 2 < RK) kload(kb[j & 1], j + 2);
    __builtin_amdgcn_sched_barrier(0);  // keep the two-group pipeline as written
    // within the group: exchanges over lane bits LPK/2 .. LPK/QK keep instruction j + RK (c / RK)
#pragma unroll
    for (int n = QK, m = LPK / 2; n > 1; n >>= 1, m >>= 1) {
      const bool hi = (c & m) != 0;
#pragma unroll
      for (int k = 0; k < n / 2; ++k)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float send = hi ? v[k][h] : v[k + n / 2][h];
          const float keep = hi ? v[k + n / 2][h] : v[k][h];
          v[k][h] = keep + __shfl_xor(send, m, WAVE);
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) ret[j][h] = v[0][h];
  }
  // value loads (instructions 4 j .. 4 j + 3 in group j), the first groups in flight during the softmax
  auto vload = [&](u32x4 (&buf)[QV], int j) {
#pragma unroll
    for (int t = 0; t < QV; ++t) {
      const int k = KPV * (QV * j + t);
      buf[t] = __builtin_amdgcn_raw_buffer_load_b128(vr_[k / PS], voff + (k % PS) * D * (int)sizeof(TV), 0, kNonTemp);
    }
  };
  u32x4 vb[2][QV];
  vload(vb[0], 0);
  if constexpr (RV > 1) vload(vb[1], 1);
  // across the groups: exchanges over lane bits RK/2 .. 1 keep group c % RK
#pragma unroll
  for (int n = RK, m = RK / 2; n > 1; n >>= 1, m >>= 1) {
    const bool hi = (c & m) != 0;
#pragma unroll
    for (int k = 0; k < n / 2; ++k)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float send = hi ? ret[k][h] : ret[k + n / 2][h];
        const float keep = hi ? ret[k + n / 2][h] : ret[k][h];
        ret[k][h] = keep + __shfl_xor(send, m, WAVE);
      }
  }
  // lane (r, c) now holds the scores of key KPI c + r; the new position (read as zeros) gets
  // its score from LDS
  const int kq = KPI * c + r;
  const bool live = kq < nk;
  if (jn >= 0 && jn < CH) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) t = fmaf(q_s[h][lane + i * WAVE], kn_s[lane + i * WAVE], t);
      t = wave_sum(t);
      if (kq == jn) ret[0][h] = t;
    }
  }
  float mh[G], lh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mh[h] = wave_max(live ? ret[0][h] : -INFINITY);
    const float pw = live ? expf(ret[0][h] - mh[h]) : 0.f;
    lh[h] = wave_sum(pw);
    p_s[w][kq][h] = pw;
  }
  __syncthreads();

  // ---- weighted sum
  float o[G][EPV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int j = 0; j < RV; ++j) {
#pragma unroll
    for (int t = 0; t < QV; ++t) {
      const int kk = KPV * (QV * j + t) + rv;
      float vx[EPV];
      const u32x4 vr = vb[j & 1][t];
      if constexpr (VB) {
        vx[0] = bf_lo(vr.x); vx[1] = bf_hi(vr.x); vx[2] = bf_lo(vr.y); vx[3] = bf_hi(vr.y);
        vx[4] = bf_lo(vr.z); vx[5] = bf_hi(vr.z); vx[6] = bf_lo(vr.w); vx[7] = bf_hi(vr.w);
      } else {
        vx[0] = __uint_as_float(vr.x); vx[1] = __uint_as_float(vr.y);
        vx[2] = __uint_as_float(vr.z); vx[3] = __uint_as_float(vr.w);
      }
      float pk[G];
      if constexpr (G == 4) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&p_s[w][kk][0]);
        pk[0] = p4.x; pk[1] = p4.y; pk[2] = p4.z; pk[3] = p4.w;
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pk[h] = p_s[w][kk][h];
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPV; ++e) o[h][e] = fmaf(pk[h], vx[e], o[h][e]);
    }
    if (j + 2 < RV) vload(vb[j & 1], j + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the new position's value (read as zeros), weighted once, in key lane 0
  if (jn >= 0 && jn < CH) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pn = rv == 0 ? p_s[w][jn][h] : 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) o[h][e] = fmaf(pn, vn_s[cv * EPV + e], o[h][e]);
    }
  }
  // add the KPV key lanes of each column
#pragma unroll
  for (int m = LPV; m < WAVE; m <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPV; ++e) o[h][e] += __shfl_xor(o[h][e], m, WAVE);
  if (rv == 0)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPV; ++e) o_s[w][h][cv * EPV + e] = o[h][e];
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_s[w][h] = mh[h];
      l_s[w][h] = lh[h];
    }
  __syncthreads();
  // merge the four wavefronts in wavefront order
  for (int idx = tid; idx < G * D; idx += NW * WAVE) {
    const int h = idx / D, d = idx % D;
    float M = m_s[0][h];
#pragma unroll
    for (int v = 1; v < NW; ++v) M = fmaxf(M, m_s[v][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float e = m_s[v][h] == -INFINITY ? 0.f : expf(m_s[v][h] - M);
      L = fmaf(e, l_s[v][h], L);
      O = fmaf(e, o_s[v][h][d], O);
    }
    const int hq = g * G + h;
    if (nsplit == 1) {
      a.out[((size_t)b * a.Hq + hq) * D + d] = O / L;
    } else {
      const size_t pi = ((size_t)b * a.Hq + hq) * a.max_splits + sp;
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_ml[pi * 2] = M;
        a.part_ml[pi * 2 + 1] = L;
      }
    }
  }
}

hipError_t launch_attention_long(const AttnArgs& a, hipStream_t s) {
  if (a.split != LONG_SPLIT || a.page_size != 16 || a.Hkv <= 0 || a.Hq % a.Hkv) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const dim3 grid(a.max_splits, a.Hkv, a.M);
#define S2_ATL(DD, GG)                                                                                        \
  if (a.D == DD && G == GG) {                                                                                 \
    if (a.k_bf16 && a.v_bf16) hipLaunchKernelGGL((k_attn_long<DD, GG, true, true>), grid, dim3(256), 0, s, a);  \
    else if (a.k_bf16) hipLaunchKernelGGL((k_attn_long<DD, GG, true, false>), grid, dim3(256), 0, s, a);        \
    else if (a.v_bf16) hipLaunchKernelGGL((k_attn_long<DD, GG, false, true>), grid, dim3(256), 0, s, a);        \
    else hipLaunchKernelGGL((k_attn_long<DD, GG, false, false>), grid, dim3(256), 0, s, a);                     \
    return hipGetLastError();                                                                                 \
  }
  S2_ATL(64, 1) S2_ATL(64, 2) S2_ATL(64, 4)
  S2_ATL(128, 1) S2_ATL(128, 2) S2_ATL(128, 4)
#undef S2_ATL
  return hipErrorInvalidValue;
}

bool attention_long_supports(int D, int Hq, int Hkv) {
  return (D == 64 || D == 128) && Hkv > 0 && Hq % Hkv == 0 && (Hq / Hkv == 1 || Hq / Hkv == 2 || Hq / Hkv == 4);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.split > 256 || a.split % 64 || a.page_size != 16) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const dim3 grid(a.max_splits, a.Hkv, a.M);
#define S2_ATT(DD, GG)                                                                                   \
  if (a.D == DD && G == GG) {                                                                            \
    if (a.k_bf16 && a.v_bf16) hipLaunchKernelGGL((k_attn<DD, GG, true, true>), grid, dim3(GG * WAVE), 0, s, a);        \
    else if (a.k_bf16) hipLaunchKernelGGL((k_attn<DD, GG, true, false>), grid, dim3(GG * WAVE), 0, s, a);              \
    else if (a.v_bf16) hipLaunchKernelGGL((k_attn<DD, GG, false, true>), grid, dim3(GG * WAVE), 0, s, a);              \
    else hipLaunchKernelGGL((k_attn<DD, GG, false, false>), grid, dim3(GG * WAVE), 0, s, a);                           \
    return hipGetLastError();                                                                            \
  }
  S2_ATT(64, 1) S2_ATT(64, 2) S2_ATT(64, 4) S2_ATT(64, 8)
  S2_ATT(128, 1) S2_ATT(128, 2) S2_ATT(128, 4) S2_ATT(128, 8)
#undef S2_ATT
  return hipErrorInvalidValue;
}

hipError_t launch_attention_combine(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.Hq, a.M);
  if (a.D == 64) hipLaunchKernelGGL(k_attn_combine<64>, grid, dim3(WAVE), 0, s, a);
  else if (a.D == 128) hipLaunchKernelGGL(k_attn_combine<128>, grid, dim3(WAVE), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Embedding gathers.

template <bool BF16>
__global__ __launch_bounds__(256) void k_embed_codes(const void* cb, int K, int H, int NC, const int* slots,
                                                     const int* codes, int* codes_snap, float* x, int ldx) {
  const int b = blockIdx.y;
  const int slot = slots[b];
  const int* cd = codes + (size_t)slot * NC;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < NC) codes_snap[(size_t)slot * NC + threadIdx.x] = cd[threadIdx.x];
  if (i >= H) return;
  float acc = 0.f;
  for (int k = 0; k < NC; ++k) acc += load_w<BF16>(cb, ((size_t)k * K + min(max(cd[k], 0), K - 1)) * H + i);
  x[(size_t)b * ldx + i] = acc;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_fast_input(const void* cb, const float* hs, int K, int H, int NC,
                                                    const int* slots, const int* codes, int j, float* x, int ldx) {
  const int b = blockIdx.y;
  const int slot = slots[b];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H) return;
  float v;
  if (j == 1) v = hs[(size_t)slot * H + i];
  else v = load_w<BF16>(cb, ((size_t)(j - 1) * K + codes[(size_t)slot * NC + j - 1]) * H + i);
  x[(size_t)b * ldx + i] = v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_embed_prompt(const void* emb, const void* cb, int K, int H, int NC,
                                                      const int* tokens, const uint8_t* mask, const int* codes,
                                                      int p, float* x) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H) return;
  float acc = 0.f;
  if (mask != nullptr && mask[p]) {
    const int* cd = codes + (size_t)p * NC;
    for (int k = 0; k < NC; ++k) acc += load_w<BF16>(cb, ((size_t)k * K + cd[k]) * H + i);
  } else {
    acc = load_w<BF16>(emb, (size_t)tokens[p] * H + i);
  }
  x[i] = acc;
}

__global__ void k_advance(const int* slots, int* pos, int M) {
  const int b = threadIdx.x;
  if (b < M) pos[slots[b]] += 1;
}

hipError_t launch_embed_codes(bool bf16, const void* cb, int K, int H, int NC, const int* slots, const int* codes,
                              int* codes_snap, float* x, int ldx, int M, hipStream_t s) {
  const dim3 grid((H + 255) / 256, M);
  if (bf16) hipLaunchKernelGGL(k_embed_codes<true>, grid, dim3(256), 0, s, cb, K, H, NC, slots, codes, codes_snap, x, ldx);
  else hipLaunchKernelGGL(k_embed_codes<false>, grid, dim3(256), 0, s, cb, K, H, NC, slots, codes, codes_snap, x, ldx);
  return hipGetLastError();
}

hipError_t launch_fast_input(bool bf16, const void* cb, const float* h, int K, int H, int NC, const int* slots,
                             const int* codes, int j, float* x, int ldx, int M, hipStream_t s) {
  const dim3 grid((H + 255) / 256, M);
  if (bf16) hipLaunchKernelGGL(k_fast_input<true>, grid, dim3(256), 0, s, cb, h, K, H, NC, slots, codes, j, x, ldx);
  else hipLaunchKernelGGL(k_fast_input<false>, grid, dim3(256), 0, s, cb, h, K, H, NC, slots, codes, j, x, ldx);
  return hipGetLastError();
}

hipError_t launch_embed_prompt(bool bf16, const void* emb, const void* cb, int K, int H, int NC, const int* tokens,
                               const uint8_t* mask, const int* codes, int p, float* x, hipStream_t s) {
  const dim3 grid((H + 255) / 256);
  if (bf16) hipLaunchKernelGGL(k_embed_prompt<true>, grid, dim3(256), 0, s, emb, cb, K, H, NC, tokens, mask, codes, p, x);
  else hipLaunchKernelGGL(k_embed_prompt<false>, grid, dim3(256), 0, s, emb, cb, K, H, NC, tokens, mask, codes, p, x);
  return hipGetLastError();
}

hipError_t launch_advance(const int* slots, int* pos, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_advance, dim3(1), dim3(64), 0, s, slots, pos, M);
  return hipGetLastError();
}

}  // namespace s2k
