// gfx950 kernels of the batched multi-stream decode step (M <= 16 streams per launch).
//
// With several streams the per-frame work is still weight-bandwidth bound (each weight is read
// once per step and used M times), but the M products per weight no longer fit the scalar FMA
// budget.  k_mgemv maps them onto the matrix cores: 16 weight rows form the A operand of
// v_mfma_f32_16x16x32_bf16 (straight from HBM, 64 contiguous bytes per lane), the streams'
// activations form the 16-column B operand (staged in LDS in 128-wide K slices, split into
// bf16 hi + lo so the product keeps ~16 activation bits).  Inside a 32-wide MFMA step the
// k order is permuted identically for A and B, which lets each lane read contiguous weights.
// Small-N matrices split K over several blocks and a reduction applies the epilogue in a fixed
// split order (bitwise reproducible).
#include "kernels.h"

#include <limits.h>
#include <math.h>

namespace s2k {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int WAVE = 64;
constexpr int MB = 16;   // batch columns of one MFMA tile
constexpr int KS = 128;  // K per staged slice
constexpr int PD = 4;    // weight slices in flight per lane

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t a = __float_as_uint(f);
  a += 0x7fffu + ((a >> 16) & 1u);
  return a >> 16;
}

__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
  uint32_t* hp = reinterpret_cast<uint32_t*>(&h);
  uint32_t* lp = reinterpret_cast<uint32_t*>(&l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_bits(v[2 * i]), h1 = bf16_bits(v[2 * i + 1]);
    const float r0 = v[2 * i] - __uint_as_float(h0 << 16), r1 = v[2 * i + 1] - __uint_as_float(h1 << 16);
    hp[i] = h0 | (h1 << 16);
    lp[i] = bf16_bits(r0) | (bf16_bits(r1) << 16);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

template <bool BF16>
__device__ __forceinline__ float load_w(const void* p, size_t i) {
  if constexpr (BF16) return __uint_as_float(((uint32_t) static_cast<const uint16_t*>(p)[i]) << 16);
  else return static_cast<const float*>(p)[i];
}

}  // namespace

// grid = (ceil(N / 64), S); block = 4 wavefronts, wavefront w owns weight rows
// [64 bx + 16 w, +16) over the block's K range [K/S * by, K/S * (by + 1)).
template <int EPI>
__global__ __launch_bounds__(256) void k_mgemv(const MgemvArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[2][MB][KS + 4];
  __shared__ float bv_s[4][MB];
  __shared__ int bi_s[4][MB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 64 + w * 16;
  const int kspan = a.K / a.S;
  const int k0 = blockIdx.y * kspan;
  const int nsl = kspan / KS;
  const int row = min(n0 + i, a.N - 1);
  const uint16_t* wr = a.w + (size_t)row * a.K + k0 + 32 * g;

  u32x4 wb[PD][4];
  auto issue = [&](u32x4 (&d)[4], int sl) {
    const u32x4* p = reinterpret_cast<const u32x4*>(wr + sl * KS);
#pragma unroll
    for (int t = 0; t < 4; ++t) d[t] = __builtin_nontemporal_load(p + t);
  };
#pragma unroll
  for (int d = 0; d < PD; ++d)
    if (d < nsl) issue(wb[d], d);

  // X slice staging: thread t covers stream t / 16, k (t % 16) * 8 .. + 8 of the slice
  const int xj = tid >> 4, xk = (tid & 15) * 8;
  const float xsc = (xj < a.M && a.x_scale) ? a.x_scale[xj] : 1.0f;
  auto stage = [&](int sl, int buf) {
    f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
    const int k = k0 + sl * KS + xk;
    if (xj < a.M) {
      const float* src = a.x + (size_t)xj * a.ldx + k;
      v0 = *reinterpret_cast<const f32x4*>(src);
      v1 = *reinterpret_cast<const f32x4*>(src + 4);
      if (a.gain) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gain + k);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gain + k + 4);
        v0 = v0 * g0 * xsc;
        v1 = v1 * g1 * xsc;
      }
    }
    *reinterpret_cast<f32x4*>(&xs[buf][xj][xk]) = v0;
    *reinterpret_cast<f32x4*>(&xs[buf][xj][xk + 4]) = v1;
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsl; s0 += PD) {
#pragma unroll
    for (int d = 0; d < PD; ++d) {  // unrolled so that wb[d] is indexed statically
      const int sl = s0 + d;
      if (sl < nsl) {
        const int buf = sl & 1;
        stage(sl, buf);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // MFMA slot group g of step t holds k = 32 g + 8 t .. + 8 of this slice (same map for A and B)
          const float* xp = &xs[buf][i][32 * g + 8 * t];
          bf16x8 xh, xl;
          split8(xp, xh, xl);
          const bf16x8 wf = __builtin_bit_cast(bf16x8, wb[d][t]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xh, acc, 0, 0, 0);
        }
        if (sl + PD < nsl) issue(wb[d], sl + PD);
      }
    }
  }

  // lane holds D[row 4 g + r][stream i] for r = 0..3
  const int j = i;
  if constexpr (EPI == MG_ARGMAX) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * g + r;
      if (n < a.N && j < a.M) {
        a.out[(size_t)j * a.ldo + n] = acc[r];
        if (n >= a.am_lo && n < a.am_hi && acc[r] > bv) {
          bv = acc[r];
          bi = n;
        }
      }
    }
    // reduce over the 4 row groups (lanes j, j+16, j+32, j+48), then over the 4 wavefronts
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane < 16) {
      bv_s[w][lane] = bv;
      bi_s[w][lane] = bi;
    }
    __syncthreads();
    if (tid < MB) {
      float v = bv_s[0][tid];
      int ix = bi_s[0][tid];
      for (int ww = 1; ww < 4; ++ww)
        if (bv_s[ww][tid] > v || (bv_s[ww][tid] == v && bi_s[ww][tid] < ix)) {
          v = bv_s[ww][tid];
          ix = bi_s[ww][tid];
        }
      a.am_val[(size_t)blockIdx.x * MB + tid] = v;
      a.am_idx[(size_t)blockIdx.x * MB + tid] = ix;
    }
  } else if (a.S > 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * g + r;
      if (n < a.N && j < a.M) a.part[((size_t)blockIdx.y * a.M + j) * a.N + n] = acc[r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * g + r;
      if (j >= a.M || n >= a.N) continue;
      if constexpr (EPI == MG_STORE) a.out[(size_t)j * a.ldo + n] = acc[r];
      else if constexpr (EPI == MG_ADD) a.out[(size_t)j * a.ldo + n] += acc[r];
      else if constexpr (EPI == MG_SWIGLU) {
        if ((r & 1) == 0) a.out[(size_t)j * a.ldo + (n >> 1)] = acc[r] / (1.0f + expf(-acc[r])) * acc[r + 1];
      }
    }
  }
}

// Sum the K splits in split order and apply the epilogue.  grid = (ceil(N / 256), M).
template <int EPI>
__global__ __launch_bounds__(256) void k_mgemv_reduce(const MgemvArgs a) {
  const int j = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  float v = 0.f;
  for (int s = 0; s < a.S; ++s) v += a.part[((size_t)s * a.M + j) * a.N + n];
  if constexpr (EPI == MG_STORE) a.out[(size_t)j * a.ldo + n] = v;
  else if constexpr (EPI == MG_ADD) a.out[(size_t)j * a.ldo + n] += v;
  else if constexpr (EPI == MG_SWIGLU) {
    if ((n & 1) == 0) {
      float u = 0.f;
      for (int s = 0; s < a.S; ++s) u += a.part[((size_t)s * a.M + j) * a.N + n + 1];
      a.out[(size_t)j * a.ldo + (n >> 1)] = v / (1.0f + expf(-v)) * u;
    }
  }
}

int mgemv_blocks(int N) { return (N + 63) / 64; }

hipError_t launch_mgemv(const MgemvArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > MB || a.K % (KS * a.S) || (a.epi == MG_ARGMAX && a.S != 1)) return hipErrorInvalidValue;
  const dim3 grid(mgemv_blocks(a.N), a.S);
#define S2_MG(E)                                                                                      \
  case E:                                                                                             \
    hipLaunchKernelGGL(k_mgemv<E>, grid, dim3(256), 0, s, a);                                         \
    if (a.S > 1 && E != MG_ARGMAX) hipLaunchKernelGGL(k_mgemv_reduce<E>, dim3((a.N + 255) / 256, a.M), \
                                                      dim3(256), 0, s, a);                            \
    break;
  switch (a.epi) {
    S2_MG(MG_STORE)
    S2_MG(MG_ADD)
    S2_MG(MG_SWIGLU)
    S2_MG(MG_ARGMAX)
    default:
      return hipErrorInvalidValue;
  }
#undef S2_MG
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Batched finisher: one block row per stream (grid = (ceil(H / 256), M)).  Same modes as the
// single-stream finisher; per-stream state is addressed through slots[b].
template <bool BF16>
__global__ __launch_bounds__(256) void k_finish_b(const FinishBArgs f) {
  __shared__ float red[4];
  __shared__ int bidx[4];
  __shared__ int s_code;
  const int b = blockIdx.y, slot = f.slots[b];
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
  float v = -INFINITY;
  int i = INT_MAX;
  for (int blk = f.b0 + threadIdx.x; blk <= f.b1; blk += 256) {
    const float pv = f.am_val[(size_t)blk * MB + b];
    const int pi = f.am_idx[(size_t)blk * MB + b];
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
    s_code = (i == INT_MAX) ? 0 : i - f.lo;
  }
  __syncthreads();
  const int code = s_code;
  int* codes = f.codes + (size_t)slot * f.NC;
  const int e = blockIdx.x * 256 + threadIdx.x;
  float* x = f.x + (size_t)b * f.ldx;
  if (f.mode == FIN_FAST_NEXT) {
    if (e < f.H) x[e] = load_w<BF16>(f.codebook, ((size_t)f.j * f.K + code) * f.H + e);
  } else if (f.mode == FIN_FAST_LAST) {
    if (e < f.H) {
      float acc = 0.f;
      for (int k = 0; k < f.NC; ++k) {
        const int ck = (k == f.j) ? code : codes[k];
        acc += load_w<BF16>(f.codebook, ((size_t)k * f.K + ck) * f.H + e);
      }
      x[e] = acc;
    }
    if (blockIdx.x == 0 && threadIdx.x < f.NC)
      f.snap[(size_t)slot * f.NC + threadIdx.x] = (threadIdx.x == f.j) ? code : codes[threadIdx.x];
  } else if (f.mode == FIN_SLOW) {
    // h[slot] = RMSNorm of the stream's residual (the vector the Slow head saw); it is also
    // the input of the next frame's first Fast step
    if (e < f.H) {
      const float hv = f.x_res[(size_t)b * f.ldx + e] * f.scale[b] * f.gain[e];
      f.h[(size_t)slot * f.H + e] = hv;
      x[e] = hv;
      if (f.xf_slot) f.xf_slot[(size_t)slot * f.ld_xf_slot + e] = hv;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    codes[f.j] = code;
    if (f.mode == FIN_SLOW) f.pos[slot] += 1;
  }
}

hipError_t launch_finish_b(bool bf16, const FinishBArgs& f, int M, hipStream_t s) {
  const dim3 grid((f.H + 255) / 256, M);
  if (bf16) hipLaunchKernelGGL(k_finish_b<true>, grid, dim3(256), 0, s, f);
  else hipLaunchKernelGGL(k_finish_b<false>, grid, dim3(256), 0, s, f);
  return hipGetLastError();
}

// x[b] = h[slots[b]]: the Fast input of step 1 for every stream of the batch
__global__ __launch_bounds__(256) void k_gather_h(const float* h, const int* slots, int H, float* x, int ldx) {
  const int b = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e < H) x[(size_t)b * ldx + e] = h[(size_t)slots[b] * H + e];
}

hipError_t launch_gather_h(const float* h, const int* slots, int H, float* x, int ldx, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_gather_h, dim3((H + 255) / 256, M), dim3(256), 0, s, h, slots, H, x, ldx);
  return hipGetLastError();
}

}  // namespace s2k
