// gfx950 kernels of the batched multi-stream decode step (M <= 16 streams per launch).
//
// With several streams the per-frame work is still weight-bandwidth bound (each weight is read
// once per step and used M times), but the M products per weight no longer fit the scalar FMA
// budget.  k_mgemv maps them onto the matrix cores: 16 weight rows form the A operand of
// v_mfma_f32_16x16x32_bf16 (straight from HBM, 64 contiguous bytes per lane), the streams'
// activations form the 16-column B operand (each lane reads its 32 fp32 activations from the
// cache-resident input rows and splits them into bf16 hi + lo, so the product keeps ~16
// activation bits).  Inside a 32-wide MFMA step the k order is permuted identically for A and B,
// which lets each lane read contiguous weights and contiguous activations.  RMSNorm runs once per
// row in k_norm_rows, which also folds the split partials of the preceding residual projection
// in a fixed split order (bitwise reproducible).
#include "kernels.h"

#include <type_traits>

#include <limits.h>
#include <math.h>

#include <algorithm>

namespace s2k {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int WAVE = 64;
constexpr int MB = 16;   // batch columns of one MFMA tile
constexpr int KS = 128;  // K per slice (4 MFMA steps)
constexpr int KC = 512;               // K of one activation chunk task
constexpr int CS = KC / KS;           // slices per task (= weight slices in flight per lane)
constexpr int XROW = KC + 8;          // LDS row stride in bf16 (padded against bank conflicts)
// buffer resources: the fourth descriptor word of a raw (untyped) gfx9 buffer, and the nontemporal
// cache-policy bit of a buffer load
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

// two floats as one packed bf16 pair (a in the low half), one conversion instruction
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  typedef float f32v2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32v2{a, b}, bf16v2));
}

__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
  uint32_t* hp = reinterpret_cast<uint32_t*>(&h);
  uint32_t* lp = reinterpret_cast<uint32_t*>(&l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = bf16_pair(v[2 * i], v[2 * i + 1]);
    hp[i] = h;
    lp[i] = bf16_pair(v[2 * i] - __uint_as_float(h << 16), v[2 * i + 1] - __uint_as_float(h & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

template <bool BF16>
__device__ __forceinline__ float load_w(const void* p, size_t i) {
  if constexpr (BF16) return __uint_as_float(((uint32_t) static_cast<const uint16_t*>(p)[i]) << 16);
  else return static_cast<const float*>(p)[i];
}

// two fp32 values with at most 8 significant bits (int8 or E4M3 codes) as a bf16 pair, exactly
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// 16 consecutive 8-bit codes (int8, or OCP FP8 E4M3 decoded by the hardware conversion) as two
// bf16x8 MFMA operands: codes 0..7 and 8..15
template <int WF>
__device__ __forceinline__ void decode8(const u32x4 p, bf16x8& a, bf16x8& b) {
  uint32_t o[8];
  const uint32_t wd[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (WF == W_I8) {
      o[2 * q] = pack_bf16_exact((float)(int8_t)(wd[q] & 0xffu), (float)(int8_t)((wd[q] >> 8) & 0xffu));
      o[2 * q + 1] = pack_bf16_exact((float)(int8_t)((wd[q] >> 16) & 0xffu), (float)(int8_t)(wd[q] >> 24));
    } else {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[q], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[q], true);
      o[2 * q] = pack_bf16_exact(lo[0], lo[1]);
      o[2 * q + 1] = pack_bf16_exact(hi[0], hi[1]);
    }
  }
  a = __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
  b = __builtin_bit_cast(bf16x8, u32x4{o[4], o[5], o[6], o[7]});
}

// weight pieces of one 128-K slice as the four MFMA steps' A operands
template <int WF, int NP>
__device__ __forceinline__ void slice_operands(const u32x4 (&wb)[NP], bf16x8 (&wf)[4]) {
  if constexpr (WF == W_BF16) {
#pragma unroll
    for (int st = 0; st < 4; ++st) wf[st] = __builtin_bit_cast(bf16x8, wb[st]);
  } else {
    decode8<WF>(wb[0], wf[0], wf[1]);
    decode8<WF>(wb[1], wf[2], wf[3]);
  }
}

}  // namespace

int mgemv_tiles(int N) { return (N + 63) / 64; }
// row stride of the split partials [S][16][ldp]: N rounded up to whole 64-row tiles
__host__ __device__ __forceinline__ size_t mgemv_ldp(int N) { return (size_t)((N + 63) / 64) * 64; }

// LDS-only barrier: the fences are restricted to the local address space, so pending global
// loads (the weight stream) and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Weights come in the tiled layout of k_tile_weights (each load instruction of a wavefront reads
// 1 KB of contiguous memory; a row-major read of 16 rows would touch 64 separate lines).
// Work items are (64-row tile, K split) pairs, numbered split-major (item = split * tiles + tile);
// block b runs items [b * ipb, (b + 1) * ipb), each as K/S/512 chunk tasks of four 128-K slices.
// Wavefront w owns rows [64 tile + 16 w, +16).  Per task the block's 16 activation rows of the
// chunk go through LDS as bf16 hi + lo.  The pipeline is one task deep and free of conditional
// loads (clamped addresses): during task t each thread first loads its share of task t+1's
// activations, then, slice by slice, task t+1's weights, so waiting for the activations never
// drains the weight stream.
template <int EPI, int WF>
__global__ __launch_bounds__(256) void k_mgemv(const MgemvArgs a) {
  constexpr int NP = WF == W_BF16 ? 4 : 2;        // 16-byte weight pieces per lane and 128-K slice
  constexpr int BLK = WF == W_BF16 ? 4096 : 2048;  // bytes of one 16-row x 128-K block
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MB * XROW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int ntiles = (a.N + 63) / 64;
  const int it0 = blockIdx.x * a.ipb;
  const int it1 = min(it0 + a.ipb, ntiles * a.S);
  if (it0 >= it1) return;
  const int kspan = a.K / a.S, nch = kspan / KC;
  const int t0 = it0 * nch, t1 = it1 * nch;  // chunk tasks of this block

  // activation share of a thread: row xr_row, 32 columns from xr_col of the chunk
  const int xr_row = tid >> 4, xr_col = (tid & 15) * 32;
  const float* xrow = a.x + (size_t)min(xr_row, a.M - 1) * a.ldx + xr_col;
  const bool xlive = xr_row < a.M;
  auto task_k = [&](int t, int& tile) {  // absolute K start of task t, and its tile
    const int it = t / nch, ch = t - it * nch;
    const int split = it / ntiles;
    tile = it - split * ntiles;
    return split * kspan + ch * KC;
  };
  const int ksl = a.K / KS;
  // weights through a buffer resource (wave-uniform byte offset of slice k / 128 of the
  // wavefront's 16-row tile, constant lane offset), as in k_mgemv_s below
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int lane_off = lane * 16;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.w), (short)0, (int)((size_t)ntiles * 64 * a.K * (BLK / 2048)), kBufferWord3);
  auto wtile = [&](int tile, int k) { return ((tile * 4 + wu) * ksl + k / KS) * BLK; };
  auto wld = [&](int base, int piece) {
    return __builtin_amdgcn_raw_buffer_load_b128(wrs, lane_off, base + piece * 1024, kNonTemporal);
  };

  f32x4 xr[8];
  u32x4 wb[CS][NP];
  {
    int tile;
    const int k = task_k(t0, tile);
    const f32x4* q = reinterpret_cast<const f32x4*>(xrow + k);
#pragma unroll
    for (int u = 0; u < 8; ++u) xr[u] = q[u];
    const int wr = wtile(tile, k);
#pragma unroll
    for (int sl = 0; sl < CS; ++sl)
#pragma unroll
      for (int t = 0; t < NP; ++t) wb[sl][t] = wld(wr, sl * NP + t);
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // one task; with LOAD the next task's activations, then its weights slice by slice, are loaded
  // behind the MFMAs (the block's last task, run after the loop, loads nothing, so no weight is
  // read twice and the loop has no branch between the two forms)
  auto step = [&](int t, auto load_next) {
    constexpr bool LOAD = decltype(load_next)::value;
    // activations of task t -> LDS (hi, lo)
    lds_barrier();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float v[8];
      v[0] = xr[2 * u].x; v[1] = xr[2 * u].y; v[2] = xr[2 * u].z; v[3] = xr[2 * u].w;
      v[4] = xr[2 * u + 1].x; v[5] = xr[2 * u + 1].y; v[6] = xr[2 * u + 1].z; v[7] = xr[2 * u + 1].w;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = xlive ? v[e] : 0.f;
      bf16x8 hi, lo;
      split8(v, hi, lo);
      *reinterpret_cast<bf16x8*>(&xs[0][xr_row * XROW + xr_col + 8 * u]) = hi;
      *reinterpret_cast<bf16x8*>(&xs[1][xr_row * XROW + xr_col + 8 * u]) = lo;
    }
    lds_barrier();
    {
      int ntile;
      const int nk = task_k(LOAD ? t + 1 : t, ntile);
      if constexpr (LOAD) {
        const f32x4* q = reinterpret_cast<const f32x4*>(xrow + nk);
#pragma unroll
        for (int u = 0; u < 8; ++u) xr[u] = q[u];
      }
      const int nwr = wtile(ntile, nk);
#pragma unroll
      for (int sl = 0; sl < CS; ++sl) {
        bf16x8 wf[4];
        slice_operands<WF>(wb[sl], wf);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          // MFMA slot group g of step st holds k = 32 g + 8 st .. + 8 of the slice (same map for A and B)
          const int kl = sl * KS + 32 * g + 8 * st;
          const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&xs[0][i * XROW + kl]);
          const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&xs[1][i * XROW + kl]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[st], xl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[st], xh, acc, 0, 0, 0);
        }
        if constexpr (LOAD) {
          // keep the reload of wb[sl] after its last use (see k_mgemv_s)
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("" : "+a"(acc)::"memory");
#pragma unroll
          for (int st = 0; st < NP; ++st) wb[sl][st] = wld(nwr, sl * NP + st);
        }
      }
    }
    const int it = t / nch;
    if (t - it * nch == nch - 1) {
      // item done: lane holds D[row 4 g + r][stream i], r = 0..3
      const int split = it / ntiles, tile = it - split * ntiles;
      const int n0 = tile * 64 + w * 16 + 4 * g;
      if constexpr (WF != W_BF16) {  // 8-bit codes: the rows' scales (rows past N read zero padding)
        const f32x4 sc = *reinterpret_cast<const f32x4*>(a.wscale + n0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= sc[r];
      }
      if (EPI == MG_ARGMAX && a.S == 1) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + r;
          if (n < a.N && i < a.M) {
            a.out[(size_t)i * a.ldo + n] = acc[r];
            if (n >= a.am_lo && n < a.am_hi && acc[r] > bv) {
              bv = acc[r];
              bi = n;
            }
          }
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
          const float ov = __shfl_xor(bv, o, WAVE);
          const int oi = __shfl_xor(bi, o, WAVE);
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (g == 0) {
          a.am_val[(size_t)(tile * 4 + w) * MB + i] = bv;
          a.am_idx[(size_t)(tile * 4 + w) * MB + i] = bi;
        }
      } else if (a.S > 1 || EPI == MG_ADD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + r;
          if (n < a.N && i < a.M) a.part[((size_t)split * MB + i) * mgemv_ldp(a.N) + n] = acc[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + r;
          if (i >= a.M || n >= a.N) continue;
          if constexpr (EPI == MG_STORE) a.out[(size_t)i * a.ldo + n] = acc[r];
          else if constexpr (EPI == MG_SWIGLU) {
            if ((r & 1) == 0) a.out[(size_t)i * a.ldo + (n >> 1)] = acc[r] / (1.0f + expf(-acc[r])) * acc[r + 1];
          }
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  for (int t = t0; t < t1 - 1; ++t) step(t, std::true_type{});
  step(t1 - 1, std::false_type{});
}

// Split-K form for every launch whose K splits into 512-wide ranges (S = K / 512): each item is one
// (64-row tile, split) chunk, numbered split-major, so a block's consecutive items share their
// activation chunk and LDS is refilled only when the split changes (outside the inner loop).  The
// inner loop is straight-line: four slices of MFMA on the weight ring, the next item's weights
// loaded slice by slice, and an unconditional 16-byte store of the item's partial sums into
// part[split][16][ldp] (rows past M or N hold values nobody reads).
template <int WF>
__global__ __launch_bounds__(256) void k_mgemv_s(const MgemvArgs a) {
  constexpr int NP = WF == W_BF16 ? 4 : 2;        // 16-byte weight pieces per lane and 128-K slice
  constexpr int BLK = WF == W_BF16 ? 4096 : 2048;  // bytes of one 16-row x 128-K block
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MB * XROW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int ntiles = (a.N + 63) / 64;
  const int it0 = blockIdx.x * a.ipb;
  const int it1 = min(it0 + a.ipb, ntiles * a.S);
  if (it0 >= it1) return;
  const int ksl = a.K / KS;
  const size_t ldp = mgemv_ldp(a.N);
  // Weights are read through a buffer resource: the item's byte offset is wave-uniform (a scalar
  // register) and the lane's offset is constant, so the loop holds no 64-bit address arithmetic
  // that could compete with the weight ring for registers (a copy of a ring register forces a wait
  // for its load).  The resource's size bound covers the whole tiled matrix.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int lane_off = lane * 16;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.w), (short)0, (int)((size_t)ntiles * 64 * a.K * (BLK / 2048)), kBufferWord3);
  auto wtile = [&](int it) {
    const int split = it / ntiles, tile = it - split * ntiles;
    return ((tile * 4 + wu) * ksl + split * CS) * BLK;
  };
  auto wld = [&](int base, int piece) {
    return __builtin_amdgcn_raw_buffer_load_b128(wrs, lane_off, base + piece * 1024, kNonTemporal);
  };
  u32x4 wb[CS][NP];
  {
    const int wr = wtile(it0);
#pragma unroll
    for (int sl = 0; sl < CS; ++sl)
#pragma unroll
      for (int t = 0; t < NP; ++t) wb[sl][t] = wld(wr, sl * NP + t);
  }
  const int xr_row = tid >> 4, xr_col = (tid & 15) * 32;
  const int xr_m = min(xr_row, a.M - 1);
  const float* xrow = a.x + (size_t)xr_m * a.ldx + xr_col;
  const bool xlive = xr_row < a.M;
  float xsc = 1.f;  // RMSNorm row scale (same sum order in every consumer)
  if (a.ssq) {
    float tot = 0.f;
    for (int c = 0; c < a.nssq; ++c) tot += a.ssq[(size_t)xr_m * a.nssq + c];
    xsc = rsqrtf(tot / (float)a.K + a.eps);
  }
  int it = it0;
  while (true) {
    const int split = it / ntiles;
    const int run_end = min(it1, (split + 1) * ntiles);  // items of this split
    if (it != it0) lds_barrier();
    {
      const f32x4* q = reinterpret_cast<const f32x4*>(xrow + split * KC);
      const f32x4* gq = a.ssq ? reinterpret_cast<const f32x4*>(a.gain + split * KC + xr_col) : nullptr;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 u0 = q[2 * u], u1 = q[2 * u + 1];
        float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        if (a.ssq) {
          const f32x4 g0 = gq[2 * u], g1 = gq[2 * u + 1];
          const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * xsc * gv[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = xlive ? v[e] : 0.f;
        bf16x8 hi, lo;
        split8(v, hi, lo);
        *reinterpret_cast<bf16x8*>(&xs[0][xr_row * XROW + xr_col + 8 * u]) = hi;
        *reinterpret_cast<bf16x8*>(&xs[1][xr_row * XROW + xr_col + 8 * u]) = lo;
      }
    }
    lds_barrier();
    // one item; with LOAD the next item's weights are loaded slice by slice behind the MFMAs (the
    // block's last item loads nothing, so no weight is read twice)
    auto item = [&](auto load_next) {
      constexpr bool LOAD = decltype(load_next)::value;
      const int nwr = wtile(LOAD ? it + 1 : it);
      const int tile = it - split * ntiles;
      f32x4 sc = {1.f, 1.f, 1.f, 1.f};
      if constexpr (WF != W_BF16)  // 8-bit codes: the rows' scales (rows past N read zero padding)
        sc = *reinterpret_cast<const f32x4*>(a.wscale + tile * 64 + w * 16 + 4 * g);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < CS; ++sl) {
        bf16x8 wf[4];
        slice_operands<WF>(wb[sl], wf);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          // MFMA slot group g of step st holds k = 32 g + 8 st .. + 8 of the slice (same map for A and B)
          const int kl = sl * KS + 32 * g + 8 * st;
          const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&xs[0][i * XROW + kl]);
          const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&xs[1][i * XROW + kl]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[st], xl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[st], xh, acc, 0, 0, 0);
        }
        if constexpr (LOAD) {
          // keep the reload of wb[sl] after its last use, so it lands in the same registers: the
          // empty statement takes the accumulator (so the slice's MFMAs come first) and orders
          // memory (so no reload moves above it)
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("" : "+a"(acc)::"memory");
#pragma unroll
          for (int st = 0; st < NP; ++st) wb[sl][st] = wld(nwr, sl * NP + st);
        }
      }
      if constexpr (WF != W_BF16)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= sc[r];
      // lane holds D[row 4 g + r][stream i] of the item's tile
      *reinterpret_cast<f32x4*>(a.part + ((size_t)split * MB + i) * ldp + tile * 64 + w * 16 + 4 * g) = acc;
    };
    // the loop itself has no branch (a branch between the two item forms inside it would make
    // the compiler copy the weight ring at the join and wait for its loads); the block's last item
    // runs after it, once its split's activations are staged
    const int loop_end = min(run_end, it1 - 1);
    for (; it < loop_end; ++it) item(std::true_type{});
    if (it == it1 - 1 && it < run_end) {
      item(std::false_type{});
      break;
    }
  }
}

// Tiled copy of a row-major bf16 matrix [N][K] (K a multiple of 128) for k_mgemv: rows are padded
// with zeros to a multiple of 64; the 16-row x 128-K block (16-row tile t, slice s) is 4 KB at
// ((t * K / 128 + s) * 4) * 512 elements, and inside it MFMA step st of lane l = i + 16 g holds the
// 8 elements W[16 t + i][128 s + 32 g + 8 st ...] at (st * 64 + l) * 8.
__global__ __launch_bounds__(256) void k_tile_weights(const uint16_t* src, uint16_t* dst, int N, int K,
                                                      size_t units) {
  const int ksl = K / KS;
  for (size_t o = blockIdx.x * (size_t)256 + threadIdx.x; o < units; o += (size_t)gridDim.x * 256) {
    const int lane = (int)(o & 63), st = (int)((o >> 6) & 3);
    const size_t rest = o >> 8;
    const int sl = (int)(rest % ksl);
    const size_t t16 = rest / ksl;
    const size_t n = t16 * 16 + (lane & 15);
    const int k = sl * KS + 32 * (lane >> 4) + 8 * st;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < (size_t)N) v = *reinterpret_cast<const u32x4*>(src + n * K + k);
    *reinterpret_cast<u32x4*>(dst + o * 8) = v;
  }
}

size_t tiled_weight_elems(int N, int K) { return (size_t)mgemv_tiles(N) * 64 * K; }

// 8-bit codes: 16-byte piece o of the tiled copy holds the codes W[16 t + i][128 s + 32 g + 16 h ..
// + 16] for lane l = i + 16 g (o = ((t * K / 128 + s) * 2 + h) * 64 + l): MFMA steps 2h and 2h + 1
__global__ __launch_bounds__(256) void k_tile_weights8(const uint8_t* src, uint8_t* dst, int N, int K,
                                                       size_t units) {
  const int ksl = K / KS;
  for (size_t o = blockIdx.x * (size_t)256 + threadIdx.x; o < units; o += (size_t)gridDim.x * 256) {
    const int lane = (int)(o & 63), h = (int)((o >> 6) & 1);
    const size_t rest = o >> 7;
    const int sl = (int)(rest % ksl);
    const size_t t16 = rest / ksl;
    const size_t n = t16 * 16 + (lane & 15);
    const int k = sl * KS + 32 * (lane >> 4) + 16 * h;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < (size_t)N) v = *reinterpret_cast<const u32x4*>(src + n * K + k);
    *reinterpret_cast<u32x4*>(dst + o * 16) = v;
  }
}

hipError_t launch_tile_weights8(const uint8_t* src, uint8_t* dst, int N, int K, hipStream_t s) {
  if (K % KS) return hipErrorInvalidValue;
  const size_t units = tiled_weight_elems(N, K) / 16;
  hipLaunchKernelGGL(k_tile_weights8, dim3((unsigned)std::min<size_t>((units + 255) / 256, 65536)), dim3(256), 0, s,
                     src, dst, N, K, units);
  return hipGetLastError();
}

hipError_t launch_tile_weights(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t s) {
  if (K % KS) return hipErrorInvalidValue;
  const size_t units = tiled_weight_elems(N, K) / 8;
  hipLaunchKernelGGL(k_tile_weights, dim3((unsigned)std::min<size_t>((units + 255) / 256, 65536)), dim3(256), 0, s,
                     src, dst, N, K, units);
  return hipGetLastError();
}

// Fold pending split partials of an MG_ADD launch into the residual rows (split order), then
// RMSNorm: xn[j] = x[j] / sqrt(mean(x[j]^2) + eps) * gain.  One 1024-thread block per batch row;
// the partial loads are issued eight at a time, the second pass re-reads the thread's own
// (cache-resident) elements.
__global__ __launch_bounds__(1024) void k_norm_rows(NormRowsArgs a) {
  __shared__ float red[16];
  const int j = blockIdx.x;
  float* x = a.x + (size_t)j * a.ldx;
  const size_t ldp = mgemv_ldp(a.H), pstride = (size_t)MB * ldp;
  float ss = 0.f;
  for (int e = threadIdx.x; e < a.H; e += 1024) {
    float t = x[e];
    const float* p = a.part + (size_t)j * ldp + e;
    int s = 0;
    for (; s + 8 <= a.S; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(s + u) * pstride];
#pragma unroll
      for (int u = 0; u < 8; ++u) t += v[u];
    }
    for (; s < a.S; ++s) t += p[s * pstride];
    if (a.S > 0) x[e] = t;
    ss = fmaf(t, t, ss);
  }
  if (!a.xn) return;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += red[w];
  const float scale = rsqrtf(tot / (float)a.H + a.eps);
  float* xn = a.xn + (size_t)j * a.ldx;
  for (int e = threadIdx.x; e < a.H; e += 1024) xn[e] = x[e] * scale * a.gain[e];
}

// acc + p[0] + p[st] + ... + p[(S - 1) st], added in split order; the first 24 loads all go out
// before the first add (one memory round trip for every split count of the model's shapes)
__device__ __forceinline__ float add_splits(float acc, const float* p, size_t st, int S) {
  constexpr int CAP = 24;
  float v[CAP];
#pragma unroll
  for (int u = 0; u < CAP; ++u) v[u] = u < S ? p[u * st] : 0.f;
#pragma unroll
  for (int u = 0; u < CAP; ++u)
    if (u < S) acc += v[u];
  for (int u = CAP; u < S; ++u) acc += p[u * st];
  return acc;
}

__global__ __launch_bounds__(256) void k_fold_rows(const FoldArgs f) {
  __shared__ float red[4];
  const int j = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  float t = 0.f;
  if (e < f.H) {
    float* x = f.x + (size_t)j * f.ldx;
    t = x[e];
    const float* p = f.part + (size_t)j * mgemv_ldp(f.H) + e;
    t = add_splits(t, p, (size_t)MB * mgemv_ldp(f.H), f.S);
    if (f.S > 0) x[e] = t;
  }
  float ss = t * t;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) f.ssq[(size_t)j * gridDim.x + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

int fold_chunks(int H) { return (H + 255) / 256; }

hipError_t launch_fold_rows(const FoldArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_fold_rows, dim3(fold_chunks(a.H), a.M), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_rows(const NormRowsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_norm_rows, dim3(a.M), dim3(1024), 0, s, a);
  return hipGetLastError();
}

// Sum the K splits in split order and apply the epilogue.  grid = (ceil(N / 256), M).
// MG_ARGMAX: logits plus the per-16-row-group maxima over [am_lo, am_hi).
template <int EPI>
__global__ __launch_bounds__(256) void k_mgemv_reduce(const MgemvArgs a) {
  const int j = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool live = n < a.N;
  const size_t ldp = mgemv_ldp(a.N);
  float v = 0.f;
  if (live) v = add_splits(0.f, a.part + (size_t)j * ldp + n, (size_t)MB * ldp, a.S);
  if constexpr (EPI == MG_STORE) {
    if (live) a.out[(size_t)j * a.ldo + n] = v;
  } else if constexpr (EPI == MG_SWIGLU) {
    // row n + 1 (the up half of the pair) is the next lane's sum
    const float u = __shfl_down(v, 1, WAVE);
    if (live && (n & 1) == 0) a.out[(size_t)j * a.ldo + (n >> 1)] = v / (1.0f + expf(-v)) * u;
  } else if constexpr (EPI == MG_ARGMAX) {
    if (live) a.out[(size_t)j * a.ldo + n] = v;
    float bv = (live && n >= a.am_lo && n < a.am_hi) ? v : -INFINITY;
    int bi = (live && n >= a.am_lo && n < a.am_hi) ? n : INT_MAX;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ov = __shfl_xor(bv, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((n & 15) == 0 && n < a.N) {
      a.am_val[(size_t)(n >> 4) * MB + j] = bv;
      a.am_idx[(size_t)(n >> 4) * MB + j] = bi;
    }
  }
}

hipError_t launch_mgemv(const MgemvArgs& a, hipStream_t s) {
  const int items = mgemv_tiles(a.N) * a.S;
  if (a.M < 1 || a.M > MB || a.S < 1 || a.K % a.S || (a.K / a.S) % KC || a.ipb < 1)
    return hipErrorInvalidValue;
  const dim3 grid((items + a.ipb - 1) / a.ipb);
  const bool split_form = a.S == a.K / KC;  // one 512-wide chunk per item: k_mgemv_s
  if (a.ssq && !split_form) return hipErrorInvalidValue;  // the input norm lives in k_mgemv_s only
  const size_t esz = a.w_fmt == W_BF16 ? 2 : 1;
  if (tiled_weight_elems(a.N, a.K) * esz > (size_t)INT_MAX) return hipErrorInvalidValue;  // buffer-resource range
  if (a.w_fmt != W_BF16 && (a.w_fmt != W_I8 && a.w_fmt != W_F8 || !a.wscale)) return hipErrorInvalidValue;
#define S2_MGW(E, WF)                                                                                  \
  if (split_form) hipLaunchKernelGGL(k_mgemv_s<WF>, grid, dim3(256), 0, s, a);                         \
  else hipLaunchKernelGGL((k_mgemv<E, WF>), grid, dim3(256), 0, s, a);
#define S2_MG(E)                                                                                      \
  case E:                                                                                             \
    if (a.w_fmt == W_BF16) { S2_MGW(E, W_BF16) }                                                      \
    else if (a.w_fmt == W_I8) { S2_MGW(E, W_I8) }                                                     \
    else { S2_MGW(E, W_F8) }                                                                          \
    if ((a.S > 1 || split_form) && E != MG_ADD)                                                       \
      hipLaunchKernelGGL(k_mgemv_reduce<E>, dim3((a.N + 255) / 256, a.M), dim3(256), 0, s, a);        \
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
#undef S2_MGW
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
    // the stop id is a text id, below every semantic id, so it also wins a tie
    if (f.mode == FIN_SLOW && f.eos_at >= 0 && f.logits[(size_t)b * f.ld_logits + f.eos_at] >= v) s_code = -1;
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
        // c0 is -1 once the stream picked its stop id: the gather stays in bounds, the result is unused
        const int ck = min(max((k == f.j) ? code : codes[k], 0), f.K - 1);
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
      const float hv = f.x_res[(size_t)b * f.ldx + e];  // already RMS-normalised with the final gain
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
