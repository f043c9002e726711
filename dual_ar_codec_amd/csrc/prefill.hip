// gfx950 kernels of the prompt prefill (many positions at once).
//
// Prefill runs every Slow layer on P prompt positions, so its projections are real dense
// contractions: C[P][N] = A[P][K] . W[N][K]^T with P up to a few thousand.  They run on the
// matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Every activation matrix is held
// as two bf16 planes, hi = bf16(x) and lo = bf16(x - hi), written once by the kernel that
// produces it (the RMSNorm + split row kernel, the prefill attention, the SwiGLU epilogue); both
// planes multiply the bf16 weights, so the product carries ~16 bits of the activation instead of 8
// (the weights are bf16 already, exactly).  Epilogues store, add the residual or form SwiGLU pairs.
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace s2k {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int WAVE = 64;

// bf16 of f rounded to nearest even, by gfx950's conversion instruction
__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats as one packed bf16 pair (a in the low half), one conversion instruction
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  typedef float f32v2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32v2{a, b}, bf16v2));
}

// IEEE fp16 bits of f, rounded to nearest even
__device__ __forceinline__ uint32_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// two floats as one packed fp16 pair (a in the low half), one conversion instruction, nearest even
__device__ __forceinline__ uint32_t f16_pair(float a, float b) {
  typedef float f32v2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16v2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32v2{a, b}, f16v2));
}

// The fp16 prefill mode writes each activation once as fp16; a value that fp16 cannot hold (beyond
// 65504 in magnitude after rounding, or not a number) raises the caller's range flag, which the
// host turns into an error.  The stored bits are the rounded value (infinity for such a value).
__device__ __forceinline__ uint16_t f16_checked(float y, int* range_flag) {
  const uint32_t h = f16_bits(y);
  if ((h & 0x7c00u) == 0x7c00u) *range_flag = 1;  // exponent all ones: infinity or NaN
  return (uint16_t)h;
}

// eight bf16 (one u32x4) as eight fp16, each rounded to nearest even: exact for magnitudes from
// 2^-17 to 65504 (bf16 keeps 8 significant bits, fp16 11, and its subnormals reach 2^-24)
__device__ __forceinline__ u32x4 bf16x8_to_f16(const u32x4 p) {
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = f16_pair(__uint_as_float(p[q] << 16), __uint_as_float(p[q] & 0xffff0000u));
  return u32x4{o[0], o[1], o[2], o[3]};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// eight 8-bit weight codes (int8, or OCP FP8 E4M3 through the hardware conversion) as eight bf16
// (or, F16, eight fp16), exactly (a code has at most 8 significant bits)
template <int WF, bool F16 = false>
__device__ __forceinline__ u32x4 widen8(const u32x2 p) {
  uint32_t o[4];
  const uint32_t wd[2] = {p.x, p.y};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float f[4];
    if constexpr (WF == W_I8) {
#pragma unroll
      for (int b = 0; b < 4; ++b) f[b] = (float)(int8_t)((wd[q] >> (8 * b)) & 0xffu);
    } else {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[q], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[q], true);
      f[0] = lo[0];
      f[1] = lo[1];
      f[2] = hi[0];
      f[3] = hi[1];
    }
    if constexpr (F16) {  // an int8 code or an E4M3 value is exact in fp16 as well
      o[2 * q] = f16_pair(f[0], f[1]);
      o[2 * q + 1] = f16_pair(f[2], f[3]);
    } else {
      o[2 * q] = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
      o[2 * q + 1] = (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xffff0000u);
    }
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// MFMA GEMM.  The activations arrive split into bf16 hi and lo planes (k_norm_split, the prefill
// attention and the SwiGLU epilogue write them), so the stage loaders only copy.  Block = 4 wavefronts in a 2 x 2 grid; wavefront (wm, wn) owns rows
// [wm BM/2, (wm+1) BM/2) and columns [64 wn, 64 wn + 64) of the block tile.
template <int BM, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs g) {
  constexpr int BN = 128, BK = 32, LS = BK + 8;  // LDS row stride (bf16): 80 bytes
  constexpr int TM = BM / 2 / 16;                 // 16-row MFMA tiles per wavefront
  constexpr int TN = 4;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LS];   // activation, bf16 hi
  __shared__ __attribute__((aligned(16))) uint16_t Al[2][BM * LS];   // activation, bf16 lo
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LS];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nk = g.K / BK;

  // global -> register staging of one K step (32 bf16 = 64 bytes per row and plane)
  // A: BM 128 -> thread t copies 16 bf16 of row t/2 at k (t%2)*16 from each plane; BM 64 -> 8 of row t/4
  constexpr int AE = BM == 128 ? 16 : 8;
  const int a_row = BM == 128 ? tid >> 1 : tid >> 2;
  const int a_k = BM == 128 ? (tid & 1) * 16 : (tid & 3) * 8;
  const int a_m = min(m0 + a_row, g.M - 1);
  const uint16_t* ah_src = g.a_hi + (size_t)a_m * g.lda + a_k;
  const uint16_t* al_src = g.a_lo + (size_t)a_m * g.lda + a_k;
  // W: thread t loads 32 bytes of row t/2 at k (t%2)*16
  const int w_row = tid >> 1, w_k = (tid & 1) * 16;
  const uint16_t* w_src = static_cast<const uint16_t*>(g.w) + (size_t)(n0 + w_row) * g.K + w_k;

  u32x4 ahr[AE / 8], alr[AE / 8];
  u32x4 wr[2];
  auto load = [&](int kt) {
    const int k = kt * BK;
#pragma unroll
    for (int i = 0; i < AE / 8; ++i) {
      ahr[i] = *reinterpret_cast<const u32x4*>(ah_src + k + 8 * i);
      alr[i] = *reinterpret_cast<const u32x4*>(al_src + k + 8 * i);
    }
    wr[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w_src + k));
    wr[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w_src + k + 8));
  };
  auto stash = [&](int kt, int buf) {
    (void)kt;
#pragma unroll
    for (int i = 0; i < AE / 8; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][a_row * LS + a_k + 8 * i]) = ahr[i];
      *reinterpret_cast<u32x4*>(&Al[buf][a_row * LS + a_k + 8 * i]) = alr[i];
    }
    uint16_t* wd = &Ws[buf][w_row * LS + w_k];
    *reinterpret_cast<u32x4*>(wd) = wr[0];
    *reinterpret_cast<u32x4*>(wd + 8) = wr[1];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  stash(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    bf16x8 af[TM], afl[TM], bfr[TN];
    const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * (BM / 2) + i * 16 + fr) * LS + fk]);
      afl[i] = *reinterpret_cast<const bf16x8*>(&Al[buf][(wm * (BM / 2) + i * 16 + fr) * LS + fk]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(&Ws[buf][(wn * 64 + j * 16 + fr) * LS + fk]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afl[i], bfr[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    if (kt + 1 < nk) stash(kt + 1, buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4 (lane/16) + r, column lane % 16 of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + r;
        const float v = acc[i][j][r];
        if constexpr (EPI == GEMM_SWIGLU) {
          const float up = __shfl_xor(v, 1, WAVE);  // columns 2i (gate) and 2i+1 (up) sit in adjacent lanes
          if (m < g.M && (n & 1) == 0) {
            const float y = v / (1.0f + expf(-v)) * up;
            const uint32_t h = bf16_bits(y);
            g.c_hi[(size_t)m * g.ldc + (n >> 1)] = (uint16_t)h;
            g.c_lo[(size_t)m * g.ldc + (n >> 1)] = (uint16_t)bf16_bits(y - __uint_as_float(h << 16));
          }
        } else if (m < g.M) {
          if constexpr (EPI == GEMM_ADD) g.c[(size_t)m * g.ldc + n] += v;
          else g.c[(size_t)m * g.ldc + n] = v;
        }
      }
    }
}

// Larger-tile variant for long prompts: NW wavefronts (WM x WN) per block, BK = 64 per stage,
// LDS double-buffered plus two register staging sets, so a stage's global loads are issued two
// stages before its compute.  Tiles are numbered with M fastest, and the blocks of one XCD
// (block ids round-robin over the 8 XCDs) take a contiguous range of tiles, so the blocks that
// share a weight column sit on one XCD and reuse it from that XCD's L2.
// F16: the activations are one IEEE fp16 plane (g.a_hi), the weights are converted to fp16 when
// staged, and every product is one v_mfma_f32_16x16x32_f16; the SwiGLU epilogue writes fp16.
template <int BM, int BN, int NW, int WM, int EPI, int WF = W_BF16, bool F16 = false, int BK = 64>
__global__ __launch_bounds__(NW * 64) void k_gemm2(const GemmArgs g) {
  // WF: bf16 weights, or 8-bit codes loaded 8 bytes per lane, widened to bf16 (fp16) when staged in
  // LDS and scaled per output column (weight row) in the epilogue
  using WR = typename std::conditional<WF == W_BF16, u32x4, u32x2>::type;
  // LDS row stride (16-bit elements): BK 64: 64 + 16.  Measured on the 1200-position prefill: 64 (no
  // pad) 31.1 ms, 72 26.5 ms, 80 25.9 ms; 80 fills the 160 KB of LDS exactly with the 128 x 256
  // tiles.  BK 32: 32 + 8 (rows 20 words apart: the 16 rows a fragment read touches hit distinct banks).
  constexpr int NT = NW * 64, WN = NW / WM, LS = BK == 64 ? BK + 16 : BK + 8;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  // coalesced stage loads: one load instruction of a wavefront covers RPI rows x BK elements (LPR
  // lanes per row, 16 bytes each) of an activation plane or of the weights
  constexpr int LPR = BK / 8, RPI = WAVE / LPR;
  constexpr int AI = BM / (RPI * NW);                 // load instructions per thread per stage and A plane
  constexpr int WI = BN / (RPI * NW);                 // W load instructions per thread per stage
  constexpr int NPL = F16 ? 1 : 2;                    // activation planes
  constexpr int STAGE = (NPL * BM + BN) * LS;         // 16-bit elements: A hi (or fp16), A lo, W
  static_assert(AI >= 1 && WI >= 1, "tile too small for the loaders");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int mt = (g.M + BM - 1) / BM, ntiles = mt * (g.N / BN);
  int tile, ks = 0;
  if (g.split > 1) {  // split K: block b takes slice b % split of tile b / split
    tile = (int)blockIdx.x / g.split;
    ks = (int)blockIdx.x % g.split;
  } else {
    const int xcd = blockIdx.x & 7, per = ntiles >> 3, rem = ntiles & 7;
    tile = xcd * per + min(xcd, rem) + (int)(blockIdx.x >> 3);
  }
  const int m0 = (tile % mt) * BM, n0 = (tile / mt) * BN;
  const int nk = g.K / BK / max(g.split, 1), kbeg = ks * nk;  // this block's stages
  (void)NT;

  // A rows of this thread: a_row0 + RPI i, columns 8 (lane % LPR) .. + 7 of the stage, both planes
  const int r_k = (lane % LPR) * 8;
  const int a_row0 = wv * (BM / NW) + lane / LPR;
  size_t a_off[AI];  // row offsets into A (rows past M repeat the last row)
#pragma unroll
  for (int i = 0; i < AI; ++i) a_off[i] = (size_t)min(m0 + a_row0 + RPI * i, g.M - 1) * g.lda + r_k;
  // W rows: w_row0 + RPI i
  const int w_row0 = wv * (BN / NW) + lane / LPR;
  const size_t w_off = (size_t)(n0 + w_row0) * g.K + r_k;  // element (= byte for 8-bit codes) offset

  u32x4 ah0[AI], al0[AI], ah1[AI], al1[AI];
  WR wr0[WI], wr1[WI];
  auto load = [&](int kt, u32x4 (&ah)[AI], u32x4 (&al)[AI], WR (&wr)[WI]) {
    const int k = (kbeg + min(kt, nk - 1)) * BK;  // past the end: reload the last stage (never computed)
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      ah[i] = *reinterpret_cast<const u32x4*>(g.a_hi + a_off[i] + k);
      if constexpr (!F16) al[i] = *reinterpret_cast<const u32x4*>(g.a_lo + a_off[i] + k);
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      if constexpr (WF == W_BF16)
        wr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.w) + w_off + (size_t)RPI * i * g.K + k));
      else
        wr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(g.w) + w_off + (size_t)RPI * i * g.K + k));
    }
  };
  auto stash = [&](int st, const u32x4 (&ah)[AI], const u32x4 (&al)[AI], const WR (&wr)[WI]) {
    uint16_t* sh = lds + st * STAGE;
    uint16_t* sl = sh + BM * LS;
    uint16_t* sw = sh + NPL * BM * LS;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      *reinterpret_cast<u32x4*>(sh + (a_row0 + RPI * i) * LS + r_k) = ah[i];
      if constexpr (!F16) *reinterpret_cast<u32x4*>(sl + (a_row0 + RPI * i) * LS + r_k) = al[i];
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      u32x4 v;
      if constexpr (WF != W_BF16) v = widen8<WF, F16>(wr[i]);
      else if constexpr (F16) v = bf16x8_to_f16(wr[i]);
      else v = wr[i];
      *reinterpret_cast<u32x4*>(sw + (w_row0 + RPI * i) * LS + r_k) = v;
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  auto compute = [&](int st) {
    const uint16_t* ah = lds + st * STAGE;
    const uint16_t* al = ah + BM * LS;
    const uint16_t* ws = ah + NPL * BM * LS;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      if constexpr (F16) {
        f16x8 bfr[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[j] = *reinterpret_cast<const f16x8*>(ws + (wn * (BN / WN) + j * 16 + fr) * LS + ks * 32 + fk);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const f16x8 af = *reinterpret_cast<const f16x8*>(ah + (wm * (BM / WM) + i * 16 + fr) * LS + ks * 32 + fk);
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bfr[j], acc[i][j], 0, 0, 0);
        }
      } else {
        bf16x8 bfr[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(ws + (wn * (BN / WN) + j * 16 + fr) * LS + ks * 32 + fk);
#pragma unroll
        for (int i = 0; i < TM; ++i) {  // one A row tile at a time keeps few fragments live
          const int r = (wm * (BM / WM) + i * 16 + fr) * LS + ks * 32 + fk;
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(ah + r);
          const bf16x8 afl = *reinterpret_cast<const bf16x8*>(al + r);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afl, bfr[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  load(0, ah0, al0, wr0);
  load(1, ah1, al1, wr1);
  stash(0, ah0, al0, wr0);
  load(2, ah0, al0, wr0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    compute(0);               // stage kt
    stash(1, ah1, al1, wr1);  // stage kt + 1
    load(kt + 3, ah1, al1, wr1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    compute(1);               // stage kt + 1
    stash(0, ah0, al0, wr0);  // stage kt + 2
    load(kt + 4, ah0, al0, wr0);
    __syncthreads();
  }

  if constexpr (WF != W_BF16) {  // 8-bit codes: scale each column by its weight row's scale
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float sc = g.wscale[n0 + wn * (BN / WN) + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] *= sc;
    }
  }
  // epilogue: lane holds rows 4 (lane/16) + r, column lane % 16 of each 16 x 16 tile
  if (g.split > 1) {  // the slice's partial sums; k_gemm_split_reduce adds the slices and applies EPI
    float* part = g.part + (size_t)ks * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
          if (m < g.M) part[(size_t)m * g.N + n] = acc[i][j][r];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * (BN / WN) + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / WM) + i * 16 + (lane >> 4) * 4 + r;
        const float v = acc[i][j][r];
        if constexpr (EPI == GEMM_SWIGLU) {
          const float up = __shfl_xor(v, 1, WAVE);  // columns 2i (gate) and 2i+1 (up) sit in adjacent lanes
          if (m < g.M && (n & 1) == 0) {
            const float y = v / (1.0f + expf(-v)) * up;
            if constexpr (F16) {
              g.c_hi[(size_t)m * g.ldc + (n >> 1)] = f16_checked(y, g.range_flag);
            } else {
              const uint32_t h = bf16_bits(y);
              g.c_hi[(size_t)m * g.ldc + (n >> 1)] = (uint16_t)h;
              g.c_lo[(size_t)m * g.ldc + (n >> 1)] = (uint16_t)bf16_bits(y - __uint_as_float(h << 16));
            }
          }
        } else if (m < g.M) {
          if constexpr (EPI == GEMM_ADD) g.c[(size_t)m * g.ldc + n] += v;
          else g.c[(size_t)m * g.ldc + n] = v;
        }
      }
    }
}

// Sum of the K slices of a split GEMM, in slice order, and the GEMM's epilogue.  Thread (m, e):
// column e (GEMM_STORE, GEMM_ADD) or the SwiGLU pair (2e, 2e + 1) of row m.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_split_reduce(const GemmArgs g) {
  const int m = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const size_t slice = (size_t)g.M * g.N;
  const float* p = g.part + (size_t)m * g.N;
  if constexpr (EPI == GEMM_SWIGLU) {
    if (2 * e + 1 >= g.N) return;
    float gt = 0.f, up = 0.f;
    for (int k = 0; k < g.split; ++k) {
      gt += p[k * slice + 2 * e];
      up += p[k * slice + 2 * e + 1];
    }
    const float y = gt / (1.0f + expf(-gt)) * up;
    if (g.a_f16) {  // the fp16 mode: the down product reads one fp16 plane
      g.c_hi[(size_t)m * g.ldc + e] = f16_checked(y, g.range_flag);
      return;
    }
    const uint32_t h = bf16_bits(y);
    g.c_hi[(size_t)m * g.ldc + e] = (uint16_t)h;
    g.c_lo[(size_t)m * g.ldc + e] = (uint16_t)bf16_bits(y - __uint_as_float(h << 16));
  } else {
    if (e >= g.N) return;
    float v = 0.f;
    for (int k = 0; k < g.split; ++k) v += p[k * slice + e];
    if constexpr (EPI == GEMM_ADD) g.c[(size_t)m * g.ldc + e] += v;
    else g.c[(size_t)m * g.ldc + e] = v;
  }
}

// K slices for a GEMM whose tiles alone would leave the CUs idle (prompts of up to 512 rows): the
// fewest of 2, 4 or 8 that give at least two blocks per CU, each slice a whole number of 64-wide
// stages.  Full-shape prefill, unsplit -> split: 64 rows 13.9 -> 6.0 ms, 200 rows 14.6 -> 10.1,
// 512 rows 18.0 -> 16.1; at 1200 rows splitting the O and down products cost 1.5 ms.
static int gemm_splits(const GemmArgs& g, int ntiles) {
  if (!g.part || g.M > 512) return 1;
  int S = 1;
  while (S < 8 && ntiles * S < 2 * device_cus() && (g.K / 64) % (2 * S) == 0 &&
         (size_t)2 * S * g.M * g.N <= g.part_floats)
    S *= 2;
  return S;
}

template <int BM, int BN, int EPI, int NW = 8, int BK = 64>
static hipError_t gemm2_launch(GemmArgs g, hipStream_t s) {
  const int ntiles = (g.M + BM - 1) / BM * (g.N / BN);
  g.split = gemm_splits(g, ntiles);
  const dim3 grid(ntiles * g.split), block(NW * 64);
  if (g.a_f16) {
    if (g.w_fmt == W_I8) hipLaunchKernelGGL((k_gemm2<BM, BN, NW, 2, EPI, W_I8, true, BK>), grid, block, 0, s, g);
    else if (g.w_fmt == W_F8) hipLaunchKernelGGL((k_gemm2<BM, BN, NW, 2, EPI, W_F8, true, BK>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((k_gemm2<BM, BN, NW, 2, EPI, W_BF16, true, BK>), grid, block, 0, s, g);
  } else if (g.w_fmt == W_I8) {
    hipLaunchKernelGGL((k_gemm2<BM, BN, NW, 2, EPI, W_I8, false, BK>), grid, block, 0, s, g);
  } else if (g.w_fmt == W_F8) {
    hipLaunchKernelGGL((k_gemm2<BM, BN, NW, 2, EPI, W_F8, false, BK>), grid, block, 0, s, g);
  } else {
    hipLaunchKernelGGL((k_gemm2<BM, BN, NW, 2, EPI, W_BF16, false, BK>), grid, block, 0, s, g);
  }
  if (g.split > 1) {
    const int cols = EPI == GEMM_SWIGLU ? g.N / 2 : g.N;
    hipLaunchKernelGGL(k_gemm_split_reduce<EPI>, dim3((cols + 255) / 256, g.M), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.N % 128 || g.K % 32 || g.M < 1) return hipErrorInvalidValue;
  if (g.w_fmt != W_BF16 && (g.K % 64 || !g.wscale)) return hipErrorInvalidValue;  // 8-bit: k_gemm2 only
  // the 8-wavefront kernel for every prompt length (rows past M repeat the last row and are not
  // stored): at 64..200 rows it ran the full-shape prefill in 14-15 ms against 25-30 ms for the
  // 4-wavefront kernel, which remains for K not divisible by 64
  if (g.epi == GEMM_SWIGLU ? (!g.c_hi || (!g.a_f16 && !g.c_lo)) : !g.c) return hipErrorInvalidValue;
  if (g.a_f16 && (g.K % 64 || !g.range_flag)) return hipErrorInvalidValue;  // fp16: k_gemm2 only
  if (g.K % 64 == 0) {
    // Measured at P = 1200 on the full shape (copy-only stage loaders): the wide gate/up + SwiGLU
    // product runs best on 128 x 256 tiles (64 x 128 per wavefront; its store and add forms would
    // spill), the other shapes on 64 x 256 tiles, both with 8 wavefronts.
    if (g.epi == GEMM_SWIGLU && g.N % 256 == 0 && g.N >= 16384) return gemm2_launch<128, 256, GEMM_SWIGLU>(g, s);
    // fp16 (one activation plane, a smaller LDS stage): QKV on 128 x 256 tiles and the residual
    // products on 128 x 128 (1200 rows: 19.4-19.6 ms each against 20.4 ms on 64 x 256)
    // (8-bit weights keep 64 x 256 for QKV: their 128 x 256 form spills)
    if (g.a_f16 && g.epi == GEMM_STORE && g.N % 256 == 0 && g.w_fmt == W_BF16)
      return gemm2_launch<128, 256, GEMM_STORE>(g, s);
    if (g.a_f16 && g.epi == GEMM_ADD) return gemm2_launch<128, 128, GEMM_ADD>(g, s);
    if (g.N % 256 == 0) {
      if (g.epi == GEMM_STORE) return gemm2_launch<64, 256, GEMM_STORE>(g, s);
      if (g.epi == GEMM_ADD) return gemm2_launch<64, 256, GEMM_ADD>(g, s);
      return gemm2_launch<64, 256, GEMM_SWIGLU>(g, s);
    }
    if (g.epi == GEMM_STORE) return gemm2_launch<128, 128, GEMM_STORE>(g, s);
    if (g.epi == GEMM_ADD) return gemm2_launch<128, 128, GEMM_ADD>(g, s);
    return gemm2_launch<128, 128, GEMM_SWIGLU>(g, s);
  }
  const bool small = (long)((g.M + 127) / 128) * (g.N / 128) < 2L * device_cus();
  const int BM = small ? 64 : 128;
  const dim3 grid(g.N / 128, (g.M + BM - 1) / BM);
#define S2_GEMM(B, E) hipLaunchKernelGGL((k_gemm<B, E>), grid, dim3(256), 0, s, g)
  if (small) {
    if (g.epi == GEMM_STORE) S2_GEMM(64, GEMM_STORE);
    else if (g.epi == GEMM_ADD) S2_GEMM(64, GEMM_ADD);
    else S2_GEMM(64, GEMM_SWIGLU);
  } else {
    if (g.epi == GEMM_STORE) S2_GEMM(128, GEMM_STORE);
    else if (g.epi == GEMM_ADD) S2_GEMM(128, GEMM_ADD);
    else S2_GEMM(128, GEMM_SWIGLU);
  }
#undef S2_GEMM
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// RMSNorm of a row and its bf16 split: hi = bf16(y), lo = bf16(y - hi) with y = x * (scale * gain),
// scale = 1 / sqrt(mean(x^2) + eps).  One block per row; the GEMMs read the two planes (lo ==
// nullptr: the fp16 mode, one plane of fp16(y)).
__global__ __launch_bounds__(256) void k_norm_split(const float* x, int ld, int H, float eps, const float* gain,
                                                    uint16_t* hi, uint16_t* lo, int ldo, int* range_flag) {
  __shared__ float red[4];
  const float* r = x + (size_t)blockIdx.x * ld;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += 256) ss = fmaf(r[k], r[k], ss);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float scale = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  uint16_t* oh = hi + (size_t)blockIdx.x * ldo;
  if (!lo) {
    for (int k = threadIdx.x; k < H; k += 256) oh[k] = f16_checked(r[k] * (scale * gain[k]), range_flag);
    return;
  }
  uint16_t* ol = lo + (size_t)blockIdx.x * ldo;
  for (int k = threadIdx.x; k < H; k += 256) {
    const float y = r[k] * (scale * gain[k]);
    const uint32_t h = bf16_bits(y);
    oh[k] = (uint16_t)h;
    ol[k] = (uint16_t)bf16_bits(y - __uint_as_float(h << 16));
  }
}

hipError_t launch_norm_split(const float* x, int ld, int H, float eps, const float* gain, uint16_t* hi, uint16_t* lo,
                             int ldo, int M, int* range_flag, hipStream_t s) {
  if (!lo && !range_flag) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_norm_split, dim3(M), dim3(256), 0, s, x, ld, H, eps, gain, hi, lo, ldo, range_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Append the keys and values of prompt rows to the paged cache: per (row, KV head) one
// wavefront applies the per-head RMSNorm and RoPE to k at position pos0 + row.
template <int D, bool KB, bool VB>
__global__ __launch_bounds__(64) void k_prefill_append(const PrefillKvArgs a) {
  constexpr int PER = D / WAVE;
  const int g = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
  const int pos = a.pos0 + row;
  const float* qkv = a.qkv + (size_t)row * a.ld;
  float kv[PER], vv[PER], ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    kv[i] = qkv[(size_t)(a.Hq + g) * D + lane + i * WAVE];
    vv[i] = qkv[(size_t)(a.Hq + a.Hkv + g) * D + lane + i * WAVE];
    ss = fmaf(kv[i], kv[i], ss);
  }
  const float rk = rsqrtf(wave_sum(ss) / (float)D + a.eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) kv[i] = kv[i] * rk * a.k_norm[lane + i * WAVE];
  const float* crow = a.rope_cos + (size_t)pos * (D / 2);
  const float* srow = a.rope_sin + (size_t)pos * (D / 2);
  if constexpr (D == 128) {
    const float cs = crow[lane], sn = srow[lane];
    const float x0 = kv[0], x1 = kv[1];
    kv[0] = x0 * cs - x1 * sn;
    kv[1] = x1 * cs + x0 * sn;
  } else {
    const int i = lane & 31;
    const float cs = crow[i], sn = srow[i];
    const float partner = __shfl_xor(kv[0], 32, WAVE);
    kv[0] = lane < 32 ? kv[0] * cs - partner * sn : kv[0] * cs + partner * sn;
  }
  const int page = a.block_table[pos / a.page_size];
  const size_t off = (((size_t)page * a.Hkv + g) * a.page_size + pos % a.page_size) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + i * WAVE;
    if constexpr (KB) {
      uint32_t ku = __float_as_uint(kv[i]);
      ku += 0x7fffu + ((ku >> 16) & 1u);
      static_cast<uint16_t*>(a.k_cache)[off + d] = (uint16_t)(ku >> 16);
    } else {
      static_cast<float*>(a.k_cache)[off + d] = kv[i];
    }
    if constexpr (VB) {
      uint32_t vu = __float_as_uint(vv[i]);
      vu += 0x7fffu + ((vu >> 16) & 1u);
      static_cast<uint16_t*>(a.v_cache)[off + d] = (uint16_t)(vu >> 16);
    } else {
      static_cast<float*>(a.v_cache)[off + d] = vv[i];
    }
  }
}

hipError_t launch_prefill_append(const PrefillKvArgs& a, int rows, hipStream_t s) {
  const dim3 grid(a.Hkv, rows);
#define S2_APP(DD)                                                                                     \
  if (a.D == DD) {                                                                                     \
    if (a.k_bf16 && a.v_bf16) hipLaunchKernelGGL((k_prefill_append<DD, true, true>), grid, dim3(64), 0, s, a); \
    else if (a.k_bf16) hipLaunchKernelGGL((k_prefill_append<DD, true, false>), grid, dim3(64), 0, s, a);    \
    else if (a.v_bf16) hipLaunchKernelGGL((k_prefill_append<DD, false, true>), grid, dim3(64), 0, s, a);    \
    else hipLaunchKernelGGL((k_prefill_append<DD, false, false>), grid, dim3(64), 0, s, a);                 \
    return hipGetLastError();                                                                          \
  }
  S2_APP(128) S2_APP(64)
#undef S2_APP
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------
// Causal attention of a block of prompt rows on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with every fp32 operand split as x = hi + lo (two bf16): each product takes hi*hi + hi*lo +
// lo*hi, so scores and weighted sums keep about 16 bits of every input (the lo*lo term and the
// split's own rounding are below 2^-15 of the product).  A workgroup of G wavefronts serves one
// (16-row block, KV group, key split); wavefront w is q head g G + w.  Per tile of 64 cached keys,
// staged in LDS as bf16 hi / lo planes (K as [key][dim], V transposed to [dim][key]) and shared
// by the G heads, a wavefront forms S^T = K Q^T: lane (i, c) (i = lane % 16, c = lane / 16) holds
// A = K[key][8 dims], B = Q[row i][the same 8 dims], and the result puts the scores of row i
// against keys 16 kt + 4 c + r in st[kt][r].  For P V the contraction over 32 keys takes, in lane
// (i, c), the keys 32 m + 4 c + r and 32 m + 16 + 4 c + r (r < 4): exactly the scores that lane
// already holds, with V read from the transposed planes 8 bytes at a time.  The running softmax
// (max, sum) is per query row; the 16-row x 16-dimension output tiles are rescaled with the row
// factors fetched from the lanes that own those rows.  Keys and values must already be cached.
constexpr int PA_QR = 16, PA_KT = 64;  // query rows per row tile (one wavefront), keys per tile
constexpr int PA_MAXT = 8;              // most tiles per workgroup (longer key ranges are split)
// row tiles per workgroup: the workgroup's G x RT wavefronts share each staged key/value tile, so a
// tile is read from the cache once per RT x 16 query rows (at most 8 wavefronts per workgroup)
__host__ __device__ constexpr int pa_row_tiles(int G) { return G >= 8 ? 1 : 2; }

// key splits of row block rb of qr rows (tiles of its causal key range over tps, at least 1)
__host__ __device__ inline int pa_splits(int rb, int rows, int pos0, int tps, int qr) {
  const int tiles = (pos0 + min(rb * qr + qr, rows) + PA_KT - 1) / PA_KT;
  return tps > 0 ? (tiles + tps - 1) / tps : 1;
}

// (the last row block has the longest key range whatever the row-block height)
int prefill_attn_splits(int rows, int pos0, int tps) { return pa_splits((rows + PA_QR - 1) / PA_QR - 1, rows, pos0, tps, PA_QR); }

// two bf16 halves (element 0 low) of hi and lo of four fp32 values
__device__ __forceinline__ void split4(const float (&x)[4], uint2& hi, uint2& lo) {
  const uint32_t h01 = bf16_pair(x[0], x[1]), h23 = bf16_pair(x[2], x[3]);
  hi = uint2{h01, h23};
  lo = uint2{bf16_pair(x[0] - __uint_as_float(h01 << 16), x[1] - __uint_as_float(h01 & 0xffff0000u)),
             bf16_pair(x[2] - __uint_as_float(h23 << 16), x[3] - __uint_as_float(h23 & 0xffff0000u))};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint2 a, uint2 b) {
  return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// four fp32 values as two packed fp16 pairs (element 0 low), rounded to nearest even
__device__ __forceinline__ uint2 f16x4_bits(const float (&x)[4]) { return uint2{f16_pair(x[0], x[1]), f16_pair(x[2], x[3])}; }

__device__ __forceinline__ f16x8 as_f16x8(uint2 a, uint2 b) {
  return __builtin_bit_cast(f16x8, u32x4{a.x, a.y, b.x, b.y});
}

// e^x as 2^(x log2 e) on the hardware base-2 exponential (0 at x = -inf): the softmax weights'
// exponentials, a large share of the attention's vector work
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// F16 (the fp16 prefill, out_lo == nullptr): q, the staged keys and values and the softmax weights are
// rounded once to fp16 and every product is one v_mfma_f32_16x16x32_f16; K and V take one LDS plane.
// The fp16 form fits 128 VGPRs (two spilled), so two workgroups of 8 wavefronts share a CU: 1200-position
// prefill 18.1 -> 17.7 ms against its natural 130 VGPRs at one workgroup per CU.
template <int D, int G, bool KB, bool VB, bool F16>
__global__ __launch_bounds__(64 * G * pa_row_tiles(G), F16 && G >= 4 ? 4 : 1) void k_prefill_attn(const PrefillAttnArgs a) {
  constexpr int RT = pa_row_tiles(G), QR = PA_QR * RT, KT = PA_KT, NT = 64 * G * RT, NDS = D / 32, NDT = D / 16;
  constexpr int KS = D + 8;    // 16-bit row stride of the K planes [key][dim]
  constexpr int VS = KT + 12;  // 16-bit row stride of the transposed V planes [dim][key]
  __shared__ __attribute__((aligned(16))) uint16_t kh[KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t kl[F16 ? 8 : KT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vh[D * VS];
  __shared__ __attribute__((aligned(16))) uint16_t vl[F16 ? 8 : D * VS];
  __shared__ int rowoff[PA_MAXT * KT];
  const int g = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int i = lane & 15, c = lane >> 4;
  const int h = g * G + w % G, rt = w / G;  // q head and row tile of this wavefront
  // workgroup -> (row block, key split): the workgroups walk the row blocks from the last (the most
  // keys) down, each row block taking its splits of at most tps tiles in order
  int rb = (a.rows + QR - 1) / QR - 1, sp = blockIdx.x, nsp;
  while (true) {
    nsp = pa_splits(rb, a.rows, a.pos0, a.tps, QR);
    if (sp < nsp || rb == 0) break;
    sp -= nsp;
    --rb;
  }
  if (sp >= nsp) return;  // (a grid larger than the split count)
  const int row0 = rb * QR;
  const int nrows = min(QR, a.rows - row0);
  const int last_pos = a.pos0 + row0 + nrows - 1;  // largest position of the block
  // keys [j_begin, j_end) of this split, at most PA_MAXT tiles
  const int j_begin = sp * a.tps * KT;
  const int j_end = min((sp + 1) * a.tps * KT, last_pos + 1);
  // cache offsets of every key of the split: one page-table round trip
  for (int t = tid; t < j_end - j_begin; t += NT) {
    const int jj = j_begin + t;
    const int page = a.block_table[jj / a.page_size];
    rowoff[t] = (int)((((size_t)page * a.Hkv + g) * a.page_size + jj % a.page_size) * D);
  }

  // q of row i (lanes (i, 0..3) share it): per-head RMSNorm, RoPE, scale; lane (i, c) keeps the
  // dimensions 32 ds + 8 c + r as the bf16 hi / lo operands qh[ds], ql[ds]
  // this wavefront's 16 rows of the block (the last block's second row tile may hold none: its q
  // row is clamped into the prompt and it writes nothing)
  const int wrow0 = row0 + PA_QR * rt, wrows = min(PA_QR, a.rows - wrow0);
  const int qrow = min(wrow0 + min(i, max(wrows, 1) - 1), a.rows - 1);
  const int rpos = a.pos0 + qrow;
  bf16x8 qh[NDS], ql[NDS];
  f16x8 qf[NDS];
  {
    float q[NDS][8];
    const float* qp = a.qkv + (size_t)qrow * a.ld + h * D + 8 * c;
    float ss = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(qp + 32 * ds);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(qp + 32 * ds + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        q[ds][r] = v[r];
        ss = fmaf(v[r], v[r], ss);
      }
    }
    ss += __shfl_xor(ss, 16, WAVE);
    ss += __shfl_xor(ss, 32, WAVE);
    const float rq = rsqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int r = 0; r < 8; ++r) q[ds][r] = q[ds][r] * rq * a.q_norm[32 * ds + 8 * c + r];
    // rotate-half pairs (d, d + D/2) sit in the same lane: chunks ds and ds + NDS/2
    const float* crow = a.rope_cos + (size_t)rpos * (D / 2);
    const float* srow = a.rope_sin + (size_t)rpos * (D / 2);
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int d = 32 * ds + 8 * c + r;
        const float cs = crow[d], sn = srow[d];
        const float x0 = q[ds][r], x1 = q[ds + NDS / 2][r];
        q[ds][r] = (x0 * cs - x1 * sn) * a.scale;
        q[ds + NDS / 2][r] = (x1 * cs + x0 * sn) * a.scale;
      }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if constexpr (F16) {
        qf[ds] = as_f16x8(f16x4_bits({q[ds][0], q[ds][1], q[ds][2], q[ds][3]}),
                          f16x4_bits({q[ds][4], q[ds][5], q[ds][6], q[ds][7]}));
      } else {
        uint2 h0, l0, h1, l1;
        split4({q[ds][0], q[ds][1], q[ds][2], q[ds][3]}, h0, l0);
        split4({q[ds][4], q[ds][5], q[ds][6], q[ds][7]}, h1, l1);
        qh[ds] = as_bf16x8(h0, h1);
        ql[ds] = as_bf16x8(l0, l1);
      }
    }
  }

  float m_i = -INFINITY, l_i = 0.f;  // softmax state of row i
  f32x4 o[NDT];                       // o[t][r] = O[row 4 c + r][dim 16 t + i]
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const uint16_t* kb = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vb = static_cast<const uint16_t*>(a.v_cache);
  // A tile is staged as blocks of 4 keys x 4 dimensions: a thread loads its blocks' rows (every load
  // of a batch issued before the first is used; keys past the tile's end read the last key, in
  // bounds, and are zeroed after the loads), splits them, and writes K rows and transposed V rows
  constexpr int NBLK = (KT / 4) * (D / 4);
  constexpr int NB = (NBLK + NT - 1) / NT, NBB = NB < 2 ? NB : 2;
  static_assert(NB % NBB == 0, "staging batches must divide evenly");
  for (int j0 = j_begin; j0 < j_end; j0 += KT) {
    const int nk = min(KT, j_end - j0);
    __syncthreads();  // the previous tile is no longer read (and, first, the offsets are in LDS)
#pragma unroll
    for (int u0 = 0; u0 < NB; u0 += NBB) {
      f32x4 kr[NBB][4], vr[NBB][4];
#pragma unroll
      for (int u = 0; u < NBB; ++u) {
        const int bb = tid + (u0 + u) * NT;
        if (NBLK % NT == 0 || bb < NBLK) {
          const int kg = bb / (D / 4), dg = bb % (D / 4);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const size_t off = (size_t)rowoff[j0 - j_begin + min(4 * kg + x, nk - 1)] + 4 * dg;
            if constexpr (KB) {
              const uint2 k2 = *reinterpret_cast<const uint2*>(kb + off);
              kr[u][x] = f32x4{__uint_as_float(k2.x << 16), __uint_as_float(k2.x & 0xffff0000u),
                               __uint_as_float(k2.y << 16), __uint_as_float(k2.y & 0xffff0000u)};
            } else {
              kr[u][x] = *reinterpret_cast<const f32x4*>(kc + off);
            }
            if constexpr (VB) {
              const uint2 v2 = *reinterpret_cast<const uint2*>(vb + off);
              vr[u][x] = f32x4{__uint_as_float(v2.x << 16), __uint_as_float(v2.x & 0xffff0000u),
                               __uint_as_float(v2.y << 16), __uint_as_float(v2.y & 0xffff0000u)};
            } else {
              vr[u][x] = *reinterpret_cast<const f32x4*>(vc + off);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NBB; ++u) {
        const int bb = tid + (u0 + u) * NT;
        if (NBLK % NT == 0 || bb < NBLK) {
          const int kg = bb / (D / 4), dg = bb % (D / 4);
          float kx[4][4], vx[4][4];  // [key x][dim y]; keys past the tile stay finite and weightless
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const bool live = 4 * kg + x < nk;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              kx[x][y] = live ? kr[u][x][y] : 0.f;
              vx[x][y] = live ? vr[u][x][y] : 0.f;
            }
          }
          if constexpr (F16) {
#pragma unroll
            for (int x = 0; x < 4; ++x) *reinterpret_cast<uint2*>(&kh[(4 * kg + x) * KS + 4 * dg]) = f16x4_bits(kx[x]);
#pragma unroll
            for (int y = 0; y < 4; ++y)
              *reinterpret_cast<uint2*>(&vh[(4 * dg + y) * VS + 4 * (kg ^ ((dg >> 2) & 3))]) =
                  f16x4_bits({vx[0][y], vx[1][y], vx[2][y], vx[3][y]});
            continue;
          }
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            uint2 hh, ll;
            split4(kx[x], hh, ll);
            *reinterpret_cast<uint2*>(&kh[(4 * kg + x) * KS + 4 * dg]) = hh;
            *reinterpret_cast<uint2*>(&kl[(4 * kg + x) * KS + 4 * dg]) = ll;
          }
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            uint2 hh, ll;
            split4({vx[0][y], vx[1][y], vx[2][y], vx[3][y]}, hh, ll);
            *reinterpret_cast<uint2*>(&vh[(4 * dg + y) * VS + 4 * (kg ^ ((dg >> 2) & 3))]) = hh;
            *reinterpret_cast<uint2*>(&vl[(4 * dg + y) * VS + 4 * (kg ^ ((dg >> 2) & 3))]) = ll;
          }
        }
      }
    }
    __syncthreads();

    // S^T = K Q^T: st[kt][r] = score of row i against key 16 kt + 4 c + r
    f32x4 st[KT / 16];
#pragma unroll
    for (int kt = 0; kt < KT / 16; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < KT / 16; ++kt) {
        const int ko = (kt * 16 + i) * KS + 32 * ds + 8 * c;
        if constexpr (F16) {
          st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const f16x8*>(&kh[ko]), qf[ds], st[kt], 0, 0, 0);
          continue;
        }
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&kh[ko]);
        const bf16x8 kb8 = *reinterpret_cast<const bf16x8*>(&kl[ko]);
        st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[ds], st[kt], 0, 0, 0);
        st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb8, qh[ds], st[kt], 0, 0, 0);
        st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[ds], st[kt], 0, 0, 0);
      }
    // causal mask and online softmax of row i over this tile (lane (i, c) holds keys 16 kt + 4 c + r);
    // a whole tile at or below every row of the wavefront needs no mask
    float mx = -INFINITY;
    if (nk == KT && j0 + KT - 1 <= a.pos0 + wrow0) {
#pragma unroll
      for (int kt = 0; kt < KT / 16; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kt][r]);
    } else {
#pragma unroll
      for (int kt = 0; kt < KT / 16; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jl = kt * 16 + 4 * c + r;
          const float v = (jl < nk && j0 + jl <= rpos) ? st[kt][r] : -INFINITY;
          st[kt][r] = v;
          mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    // A row's first key split always holds key 0 <= rpos, so m is finite from its first tile on; in
    // a later split a row may have no key yet (m still -inf), and then every weight is 0
    const float m_new = fmaxf(m_i, mx);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float corr = exp_hw(m_i - m_ref);
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT / 16; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp_hw(st[kt][r] - m_ref);
        st[kt][r] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 16, WAVE);
    ps += __shfl_xor(ps, 32, WAVE);
    l_i = l_i * corr + ps;
    m_i = m_new;
    float cr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * c + r, WAVE);
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[t][r] *= cr[r];
    // O += P V over 32-key blocks m: lane (i, c) contracts keys 32 m + 4 c + r and 32 m + 16 + 4 c + r
#pragma unroll
    for (int m = 0; m < KT / 32; ++m) {
      if constexpr (F16) {
        const f16x8 pf = as_f16x8(f16x4_bits({st[2 * m][0], st[2 * m][1], st[2 * m][2], st[2 * m][3]}),
                                  f16x4_bits({st[2 * m + 1][0], st[2 * m + 1][1], st[2 * m + 1][2], st[2 * m + 1][3]}));
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const int vo = (16 * t + i) * VS + 32 * m + 4 * (c ^ (t & 3));
          const f16x8 vf = as_f16x8(*reinterpret_cast<const uint2*>(&vh[vo]), *reinterpret_cast<const uint2*>(&vh[vo + 16]));
          o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf, o[t], 0, 0, 0);
        }
        continue;
      }
      uint2 p0h, p0l, p1h, p1l;
      split4({st[2 * m][0], st[2 * m][1], st[2 * m][2], st[2 * m][3]}, p0h, p0l);
      split4({st[2 * m + 1][0], st[2 * m + 1][1], st[2 * m + 1][2], st[2 * m + 1][3]}, p1h, p1l);
      const bf16x8 pa = as_bf16x8(p0h, p1h), pb = as_bf16x8(p0l, p1l);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const int vo = (16 * t + i) * VS + 32 * m + 4 * (c ^ (t & 3));
        const bf16x8 va = as_bf16x8(*reinterpret_cast<const uint2*>(&vh[vo]), *reinterpret_cast<const uint2*>(&vh[vo + 16]));
        const bf16x8 vb8 = as_bf16x8(*reinterpret_cast<const uint2*>(&vl[vo]), *reinterpret_cast<const uint2*>(&vl[vo + 16]));
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, va, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb8, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, va, o[t], 0, 0, 0);
      }
    }
  }
  if (nsp > 1) {  // a split's unnormalised output and row state, merged by k_prefill_attn_combine
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wrow0 + 4 * c + r;
      if (row - wrow0 < wrows) {
        float* po = a.part_o + (((size_t)sp * a.rows + row) * a.Hq + h) * D + i;
#pragma unroll
        for (int t = 0; t < NDT; ++t) po[16 * t] = o[t][r];
      }
    }
    if (c == 0 && i < wrows) {
      float* pml = a.part_ml + (((size_t)sp * a.rows + wrow0 + i) * a.Hq + h) * 2;
      pml[0] = m_i;
      pml[1] = l_i;
    }
    return;
  }
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) inv[r] = 1.0f / __shfl(l_i, 4 * c + r, WAVE);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = wrow0 + 4 * c + r;
    if (row - wrow0 < wrows) {
      uint16_t* oh = a.out_hi + (size_t)row * a.ld_out + h * D + i;
      if (!a.out_lo) {
#pragma unroll
        for (int t = 0; t < NDT; ++t) oh[16 * t] = f16_checked(o[t][r] * inv[r], a.range_flag);
        continue;
      }
      uint16_t* ol = a.out_lo + (size_t)row * a.ld_out + h * D + i;
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const float y = o[t][r] * inv[r];
        const uint32_t hb = bf16_bits(y);
        oh[16 * t] = (uint16_t)hb;
        ol[16 * t] = (uint16_t)bf16_bits(y - __uint_as_float(hb << 16));
      }
    }
  }
}

// Merge the key splits of the row blocks that have several, in split order: per row and q head,
// M = max m_s, L = sum e^(m_s - M) l_s, y = sum e^(m_s - M) o_s / L, written as the bf16 planes.
// grid = (16-row tiles, Hq), 4 wavefronts of 4 rows each; lane holds dimensions lane + 64 u.  A
// row's loads for up to 8 splits are all issued before the first is used (longer ranges loop).
template <int D>
__global__ __launch_bounds__(256) void k_prefill_attn_combine(const PrefillAttnArgs a) {
  constexpr int PER = D / 64, SB = 8;
  const int rb = blockIdx.x, h = blockIdx.y, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int qr = PA_QR * pa_row_tiles(a.Hq / a.Hkv);  // rows of the attention's row blocks
  const int nsp = pa_splits(rb * PA_QR / qr, a.rows, a.pos0, a.tps, qr);
  if (nsp == 1) return;  // written by the attention kernel
  const int row0 = rb * PA_QR, nrows = min(PA_QR, a.rows - row0);
  for (int ri = wv; ri < nrows; ri += 4) {
    const int row = row0 + ri;
    float M = -INFINITY, L = 0.f, acc[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] = 0.f;
    for (int s0 = 0; s0 < nsp; s0 += SB) {
      float m[SB], l[SB], o[SB][PER];
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const size_t base = ((size_t)min(s0 + q, nsp - 1) * a.rows + row) * a.Hq + h;  // in bounds
        m[q] = a.part_ml[base * 2];
        l[q] = a.part_ml[base * 2 + 1];
#pragma unroll
        for (int u = 0; u < PER; ++u) o[q][u] = a.part_o[base * D + lane + 64 * u];
      }
      // running merge in split order (a split with no key of this row: m = -inf, weight 0)
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        if (s0 + q >= nsp) break;
        const float Mn = fmaxf(M, m[q]);
        const float ca = expf(M - Mn), cb = expf(m[q] - Mn);  // M = -inf only before the first split
        L = L * ca + l[q] * cb;
#pragma unroll
        for (int u = 0; u < PER; ++u) acc[u] = acc[u] * ca + o[q][u] * cb;
        M = Mn;
      }
    }
    const float inv = 1.0f / L;
    uint16_t* oh = a.out_hi + (size_t)row * a.ld_out + h * D;
    if (!a.out_lo) {
#pragma unroll
      for (int u = 0; u < PER; ++u) oh[lane + 64 * u] = f16_checked(acc[u] * inv, a.range_flag);
      continue;
    }
    uint16_t* ol = a.out_lo + (size_t)row * a.ld_out + h * D;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const float y = acc[u] * inv;
      const uint32_t hb = bf16_bits(y);
      oh[lane + 64 * u] = (uint16_t)hb;
      ol[lane + 64 * u] = (uint16_t)bf16_bits(y - __uint_as_float(hb << 16));
    }
  }
}

template <int D, int G, bool F16>
static void launch_pa_kernel(const PrefillAttnArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(64 * G * pa_row_tiles(G));
  if (a.k_bf16 && a.v_bf16) hipLaunchKernelGGL((k_prefill_attn<D, G, true, true, F16>), grid, block, 0, s, a);
  else if (a.k_bf16) hipLaunchKernelGGL((k_prefill_attn<D, G, true, false, F16>), grid, block, 0, s, a);
  else if (a.v_bf16) hipLaunchKernelGGL((k_prefill_attn<D, G, false, true, F16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_prefill_attn<D, G, false, false, F16>), grid, block, 0, s, a);
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.Hkv < 1 || a.Hq % a.Hkv) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv, qr = PA_QR * pa_row_tiles(G);
  const int nb = (a.rows + qr - 1) / qr, nb16 = (a.rows + PA_QR - 1) / PA_QR;
  if (a.tps < 1 || a.tps > PA_MAXT || a.rows < 1) return hipErrorInvalidValue;
  if (!a.out_hi || (!a.out_lo && !a.range_flag)) return hipErrorInvalidValue;
  int blocks = 0;
  for (int rb = 0; rb < nb; ++rb) blocks += pa_splits(rb, a.rows, a.pos0, a.tps, qr);
  if (blocks > nb && (!a.part_o || !a.part_ml)) return hipErrorInvalidValue;
  const dim3 grid(blocks, a.Hkv);
  // some row block has several splits: the attention, then the merge
#define S2_PA(DD, GG)                                                                     \
  if (a.D == DD && G == GG) {                                                             \
    if (a.out_lo) launch_pa_kernel<DD, GG, false>(a, grid, s);                            \
    else launch_pa_kernel<DD, GG, true>(a, grid, s);                                      \
    hipError_t e = hipGetLastError();                                                     \
    if (e != hipSuccess || blocks == nb) return e;                                        \
    hipLaunchKernelGGL(k_prefill_attn_combine<DD>, dim3(nb16, a.Hq), dim3(256), 0, s, a); \
    return hipGetLastError();                                                             \
  }
  S2_PA(64, 1) S2_PA(64, 2) S2_PA(64, 4) S2_PA(64, 8)
  S2_PA(128, 1) S2_PA(128, 2) S2_PA(128, 4) S2_PA(128, 8)
#undef S2_PA
  return hipErrorInvalidValue;
}

// Prompt embeddings of rows [p0, p0 + rows): text rows take embed[token]; masked rows take the
// sum of their ten codebook rows (fp32, codebook order).
template <bool BF16>
__global__ __launch_bounds__(256) void k_embed_rows(const void* emb, const void* cb, int K, int H, int NC,
                                                    const int* tokens, const uint8_t* mask, const int* codes, int p0,
                                                    float* x, int ldx) {
  const int row = blockIdx.y, p = p0 + row;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= H) return;
  auto ld = [&](const void* base, size_t i) -> float {
    if constexpr (BF16) return __uint_as_float(((uint32_t) static_cast<const uint16_t*>(base)[i]) << 16);
    else return static_cast<const float*>(base)[i];
  };
  float acc = 0.f;
  if (mask != nullptr && mask[p]) {
    for (int k = 0; k < NC; ++k) acc += ld(cb, ((size_t)k * K + codes[(size_t)p * NC + k]) * H + e);
  } else {
    acc = ld(emb, (size_t)tokens[p] * H + e);
  }
  x[(size_t)row * ldx + e] = acc;
}

hipError_t launch_embed_rows(bool bf16, const void* emb, const void* cb, int K, int H, int NC, const int* tokens,
                             const uint8_t* mask, const int* codes, int p0, int rows, float* x, int ldx,
                             hipStream_t s) {
  const dim3 grid((H + 255) / 256, rows);
  if (bf16) hipLaunchKernelGGL(k_embed_rows<true>, grid, dim3(256), 0, s, emb, cb, K, H, NC, tokens, mask, codes, p0, x, ldx);
  else hipLaunchKernelGGL(k_embed_rows<false>, grid, dim3(256), 0, s, emb, cb, K, H, NC, tokens, mask, codes, p0, x, ldx);
  return hipGetLastError();
}

}  // namespace s2k
