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

namespace s2k {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

// ---------------------------------------------------------------------------------------------
// Weight-streaming GEMV.  Workgroup = 4 wavefronts; wavefront w of block b owns rows
// (4b + w) * R ... + R - 1.  NCH > 0: K == NCH * 64 * elements-per-chunk and all weight loads of
// the wavefront are issued up front; NCH == 0: any K divisible by the chunk width / 8, looped.
template <bool BF16, int NCH, int KIND>
__global__ __launch_bounds__(GEMV_THREADS) void k_gemv(const GemvArgs a) {
  extern __shared__ float xs[];
  constexpr int R = rows_per_wave(KIND);
  constexpr int EPC = BF16 ? 8 : 4;
  constexpr bool NORM = KIND != GEMV_RESID;
  __shared__ float red[GEMV_WAVES];
  __shared__ int bidx[GEMV_WAVES];
  __shared__ int s_last;

  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  const int K = a.K;
  const int row0 = (blockIdx.x * GEMV_WAVES + wid) * R;
  const size_t row_bytes = (size_t)K * (BF16 ? 2 : 4);

  // 1. loads: the input vector (and gain) first, then every weight chunk of this wavefront's
  //    rows.  vmcnt retires in issue order, so staging the input only waits for the input.
  constexpr int XL = NCH > 0 ? (NCH * WAVE * EPC + GEMV_THREADS * 4 - 1) / (GEMV_THREADS * 4) : 1;
  f32x4 xv[XL], gv[XL];
  u32x4 wv[R][NCH > 0 ? NCH : 1];
  if constexpr (NCH > 0) {
#pragma unroll
    for (int t = 0; t < XL; ++t) {  // x and gain are zero-padded to a multiple of 1024 floats
      const int k = (t * GEMV_THREADS + threadIdx.x) * 4;
      xv[t] = *reinterpret_cast<const f32x4*>(a.x + k);
      if constexpr (NORM) gv[t] = *reinterpret_cast<const f32x4*>(a.gain + k);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, a.N - 1);
      const u32x4* wp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.w) + (size_t)row * row_bytes);
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
      const int k = (t * GEMV_THREADS + threadIdx.x) * 4;
      const f32x4 v = xv[t];
      *reinterpret_cast<f32x4*>(xs + k) = v;
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
  } else {
    for (int k = threadIdx.x * 4; k < K; k += GEMV_THREADS * 4) {
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
    for (int w = 0; w < GEMV_WAVES; ++w) tot += red[w];
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
      for (int t = 0; t < XL; ++t) norm4((t * GEMV_THREADS + threadIdx.x) * 4, gv[t]);
    } else {
      for (int k = threadIdx.x * 4; k < K; k += GEMV_THREADS * 4) norm4(k, *reinterpret_cast<const f32x4*>(a.gain + k));
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
      for (int r = 0; r < R; ++r) acc[r] = dot_chunk<BF16>(wv[r][c], xp, acc[r]);
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
          const u32x4* wp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.w) + (size_t)row * row_bytes);
          acc[r] = dot_chunk<BF16>(__builtin_nontemporal_load(wp + c * WAVE + lane), xp, acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);

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
  } else {  // GEMV_NORM_ARGMAX
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
      for (int w = 1; w < GEMV_WAVES; ++w)
        if (red[w] > v) {
          v = red[w];
          i = bidx[w];
        }
      a.am_val[blockIdx.x] = v;
      a.am_idx[blockIdx.x] = i;
      __threadfence();
      const unsigned t = atomicAdd(a.am_counter, 1u);
      s_last = (t == gridDim.x - 1);
    }
    __syncthreads();
    if (s_last) {  // second pass: the last workgroup reduces the per-block picks
      __threadfence();
      constexpr int RB = GEMV_WAVES * R;
      const int b0 = a.am_lo / RB, b1 = (a.am_hi - 1) / RB;
      float v = -INFINITY;
      int i = INT_MAX;
      for (int b = b0 + threadIdx.x; b <= b1; b += GEMV_THREADS) {
        const float pv = __hip_atomic_load(a.am_val + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int pi = __hip_atomic_load(a.am_idx + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        for (int w = 1; w < GEMV_WAVES; ++w)
          if (red[w] > v || (red[w] == v && bidx[w] < i)) {
            v = red[w];
            i = bidx[w];
          }
        *a.am_code_out = (i == INT_MAX) ? 0 : i - a.am_lo;
        *a.am_counter = 0u;
      }
    }
  }
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

hipError_t launch_gemv(int kind, bool bf16, const GemvArgs& a, hipStream_t s) {
  switch (kind) {
    case GEMV_NORM_STORE: return bf16 ? gemv_dispatch<true, GEMV_NORM_STORE>(a, s) : gemv_dispatch<false, GEMV_NORM_STORE>(a, s);
    case GEMV_RESID: return bf16 ? gemv_dispatch<true, GEMV_RESID>(a, s) : gemv_dispatch<false, GEMV_RESID>(a, s);
    case GEMV_NORM_SWIGLU: return bf16 ? gemv_dispatch<true, GEMV_NORM_SWIGLU>(a, s) : gemv_dispatch<false, GEMV_NORM_SWIGLU>(a, s);
    case GEMV_NORM_ARGMAX: return bf16 ? gemv_dispatch<true, GEMV_NORM_ARGMAX>(a, s) : gemv_dispatch<false, GEMV_NORM_ARGMAX>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------
// Decode attention.  grid = (max_chunks, Hkv, M), block = G wavefronts (G = Hq / Hkv).
template <int D, int G>
__global__ __launch_bounds__(G * WAVE) void k_attn(const AttnArgs a) {
  constexpr int CH = WAVE;     // positions per chunk: one per lane
  constexpr int KSTR = D + 2;  // padded row stride of the K tile (bf16 elements)
  constexpr int PER = D / WAVE;
  constexpr int HD = D / 2;
  constexpr int CPR = D * 2 / 16;  // 16-byte pieces per cached row
  __shared__ float q_s[G][D];
  __shared__ float kn_s[D];
  __shared__ float vn_s[D];
  __shared__ __attribute__((aligned(16))) uint16_t k_s[CH * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[CH * D];
  __shared__ float p_s[G][CH];
  __shared__ int s_last;

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  const int slot = a.slots[b];
  const int pos = a.pos[slot];
  const int ctx = pos + 1;
  const int nch = (ctx + CH - 1) / CH;
  if (c >= nch) return;
  const int j0 = c * CH;
  const int nvalid = min(CH, ctx - j0);
  const bool has_new = pos >= j0 && pos < j0 + CH;
  const int h = g * G + w;
  const float* qkv = a.qkv + (size_t)b * (a.Hq + 2 * a.Hkv) * D;
  const float* crow = a.rope_cos + (size_t)pos * HD;
  const float* srow = a.rope_sin + (size_t)pos * HD;

  // per-head RMSNorm of q (and of the new k), then rotate-half RoPE at pos
  {
    float qv[PER], ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      qv[i] = qkv[h * D + lane + i * WAVE];
      ss = fmaf(qv[i], qv[i], ss);
    }
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int i = 0; i < PER; ++i) q_s[w][lane + i * WAVE] = qv[i] * r * a.q_norm[lane + i * WAVE];
    if (has_new && w == 0) {
      const float* kp = qkv + (size_t)(a.Hq + g) * D;
      const float* vp = qkv + (size_t)(a.Hq + a.Hkv + g) * D;
      float kv[PER];
      ss = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        kv[i] = kp[lane + i * WAVE];
        ss = fmaf(kv[i], kv[i], ss);
        vn_s[lane + i * WAVE] = vp[lane + i * WAVE];
      }
      ss = wave_sum(ss);
      const float rk = rsqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int i = 0; i < PER; ++i) kn_s[lane + i * WAVE] = kv[i] * rk * a.k_norm[lane + i * WAVE];
    }
  }
  __syncthreads();
  for (int i = lane; i < HD; i += WAVE) {
    const float cs = crow[i], sn = srow[i];
    const float x0 = q_s[w][i], x1 = q_s[w][i + HD];
    q_s[w][i] = (x0 * cs - x1 * sn) * a.scale;
    q_s[w][i + HD] = (x1 * cs + x0 * sn) * a.scale;
    if (has_new && w == 0) {
      const float k0 = kn_s[i], k1 = kn_s[i + HD];
      kn_s[i] = k0 * cs - k1 * sn;
      kn_s[i + HD] = k1 * cs + k0 * sn;
    }
  }
  __syncthreads();

  // stage the chunk's cached K/V rows (the new position comes from registers)
  for (int i = threadIdx.x; i < CH * CPR; i += G * WAVE) {
    const int j = i / CPR, q = i % CPR;
    const int jj = j0 + j;
    if (j < nvalid && jj != pos) {
      const int page = a.block_table[slot * a.bt_stride + jj / a.page_size];
      const size_t off = (((size_t)page * a.Hkv + g) * a.page_size + jj % a.page_size) * D + q * 8;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(a.k_cache + off);
      const u32x4 vv = *reinterpret_cast<const u32x4*>(a.v_cache + off);
      uint32_t* kd = reinterpret_cast<uint32_t*>(k_s + j * KSTR + q * 8);
      kd[0] = kv.x;
      kd[1] = kv.y;
      kd[2] = kv.z;
      kd[3] = kv.w;
      *reinterpret_cast<u32x4*>(v_s + j * D + q * 8) = vv;
    }
  }
  if (has_new && w == 0) {
    const int jn = pos - j0;
    const int page = a.block_table[slot * a.bt_stride + pos / a.page_size];
    const size_t off = (((size_t)page * a.Hkv + g) * a.page_size + pos % a.page_size) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane + i * WAVE;
      const uint16_t kb = f2bf(kn_s[d]), vb = f2bf(vn_s[d]);
      k_s[jn * KSTR + d] = kb;
      v_s[jn * D + d] = vb;
      a.k_cache[off + d] = kb;
      a.v_cache[off + d] = vb;
    }
  }
  __syncthreads();

  // scores: lane = position, wavefront = q head
  float s = -INFINITY;
  if (lane < nvalid) {
    const uint16_t* kr = k_s + lane * KSTR;
    float acc = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; d += 2) {
      const uint32_t kk = *reinterpret_cast<const uint32_t*>(kr + d);
      acc = fmaf(q_s[w][d], bf_lo(kk), acc);
      acc = fmaf(q_s[w][d + 1], bf_hi(kk), acc);
    }
    s = acc;
  }
  const float m = wave_max(s);
  const float p = (lane < nvalid) ? expf(s - m) : 0.f;
  const float l = wave_sum(p);
  p_s[w][lane] = p;
  __syncthreads();
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int j = 0; j < nvalid; ++j) {
    const float pj = p_s[w][j];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = fmaf(pj, bf_one(v_s[j * D + lane + i * WAVE]), o[i]);
  }

  float* out = a.out + ((size_t)b * a.Hq + h) * D;
  if (nch == 1) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < PER; ++i) out[lane + i * WAVE] = o[i] * inv;
    return;
  }
  const size_t pi = ((size_t)b * a.Hq + h) * a.max_chunks + c;
  if (lane == 0) {
    a.part_ml[pi * 2] = m;
    a.part_ml[pi * 2 + 1] = l;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) a.part_o[pi * D + lane + i * WAVE] = o[i];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned t = atomicAdd(a.counters + b * a.Hkv + g, 1u);
    s_last = (t == (unsigned)nch - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // merge the chunks of q head h in chunk order
  const size_t base = ((size_t)b * a.Hq + h) * a.max_chunks;
  float M = -INFINITY;
  for (int cc = 0; cc < nch; ++cc)
    M = fmaxf(M, __hip_atomic_load(a.part_ml + (base + cc) * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  float L = 0.f, acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int cc = 0; cc < nch; ++cc) {
    const float mc = __hip_atomic_load(a.part_ml + (base + cc) * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float lc = __hip_atomic_load(a.part_ml + (base + cc) * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float e = expf(mc - M);
    L = fmaf(e, lc, L);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      acc[i] = fmaf(e, __hip_atomic_load(a.part_o + (base + cc) * D + lane + i * WAVE, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT), acc[i]);
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) out[lane + i * WAVE] = acc[i] * inv;
  if (threadIdx.x == 0) a.counters[b * a.Hkv + g] = 0u;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid(a.max_chunks, a.Hkv, a.M);
#define S2_ATT(DD, GG)                                                          \
  if (a.D == DD && G == GG) {                                                   \
    hipLaunchKernelGGL((k_attn<DD, GG>), grid, dim3(GG * WAVE), 0, s, a);       \
    return hipGetLastError();                                                   \
  }
  S2_ATT(64, 1) S2_ATT(64, 2) S2_ATT(64, 4) S2_ATT(64, 8)
  S2_ATT(128, 1) S2_ATT(128, 2) S2_ATT(128, 4) S2_ATT(128, 8)
#undef S2_ATT
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------
// Embedding gathers.

template <bool BF16>
__global__ __launch_bounds__(256) void k_embed_codes(const void* cb, int K, int H, int NC, const int* slots,
                                                     const int* codes, int* codes_snap, float* x) {
  const int b = blockIdx.y;
  const int slot = slots[b];
  const int* cd = codes + (size_t)slot * NC;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < NC) codes_snap[(size_t)b * NC + threadIdx.x] = cd[threadIdx.x];
  if (i >= H) return;
  float acc = 0.f;
  for (int k = 0; k < NC; ++k) acc += load_w<BF16>(cb, ((size_t)k * K + cd[k]) * H + i);
  x[(size_t)b * H + i] = acc;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_fast_input(const void* cb, const float* hs, int K, int H, int NC,
                                                    const int* slots, const int* codes, int j, float* x) {
  const int b = blockIdx.y;
  const int slot = slots[b];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H) return;
  float v;
  if (j == 1) v = hs[(size_t)slot * H + i];
  else v = load_w<BF16>(cb, ((size_t)(j - 1) * K + codes[(size_t)slot * NC + j - 1]) * H + i);
  x[(size_t)b * H + i] = v;
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
                              int* codes_snap, float* x, int M, hipStream_t s) {
  const dim3 grid((H + 255) / 256, M);
  if (bf16) hipLaunchKernelGGL(k_embed_codes<true>, grid, dim3(256), 0, s, cb, K, H, NC, slots, codes, codes_snap, x);
  else hipLaunchKernelGGL(k_embed_codes<false>, grid, dim3(256), 0, s, cb, K, H, NC, slots, codes, codes_snap, x);
  return hipGetLastError();
}

hipError_t launch_fast_input(bool bf16, const void* cb, const float* h, int K, int H, int NC, const int* slots,
                             const int* codes, int j, float* x, int M, hipStream_t s) {
  const dim3 grid((H + 255) / 256, M);
  if (bf16) hipLaunchKernelGGL(k_fast_input<true>, grid, dim3(256), 0, s, cb, h, K, H, NC, slots, codes, j, x);
  else hipLaunchKernelGGL(k_fast_input<false>, grid, dim3(256), 0, s, cb, h, K, H, NC, slots, codes, j, x);
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
