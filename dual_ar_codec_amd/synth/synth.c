/*
 * Seeded synthetic inputs for the Dual-AR decode step: weights, prompt token
 * ids and VQ codes.  This file holds no arithmetic of the model itself; it only
 * draws numbers.  Both the CPU oracle and the HIP path receive the arrays it
 * writes, so the two sides always see bit-identical inputs.
 *
 * Every value is a pure function of (seed, stream, index):
 *   - SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014) supplies 64-bit words: the i-th output of a
 *     SplitMix64 sequence whose state starts at key(seed, stream);
 *   - uniforms in [0,1) take the top 53 bits;
 *   - normals use the Box-Muller transform (Box & Muller, 1958) on the pair of
 *     uniforms (2m, 2m+1): element 2m takes the cosine branch, 2m+1 the sine;
 *   - bounded integers in [0, n) use Lemire's multiply-shift on the top 32 bits
 *     (Lemire, "Fast random integer generation in an interval", 2019).
 * Thread count never changes a value (each element is computed from its index).
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GOLDEN + mix64(stream + GOLDEN));
}

/* i-th SplitMix64 output of the sequence keyed by (seed, stream). */
uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t i) {
  return mix64(stream_key(seed, stream) + (i + 1) * GOLDEN);
}

static inline double unit53(uint64_t u) { return (double)(u >> 11) * 0x1.0p-53; }

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7fffu + lsb) >> 16);
}

/* Both members of Box-Muller pair m (elements 2m and 2m+1). */
static inline void normal_pair(uint64_t key, uint64_t m, double* a, double* b) {
  double u1 = unit53(mix64(key + (2 * m + 1) * GOLDEN));
  double u2 = unit53(mix64(key + (2 * m + 2) * GOLDEN));
  double r = sqrt(-2.0 * log(1.0 - u1));
  double t = 6.283185307179586476925286766559 * u2;
  *a = r * cos(t);
  *b = r * sin(t);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double scale, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < (n + 1) / 2; ++m) {
    double a, b;
    normal_pair(key, (uint64_t)m, &a, &b);
    out[2 * m] = (float)(scale * a);
    if (2 * m + 1 < n) out[2 * m + 1] = (float)(scale * b);
  }
}

/* The normal value is rounded to fp32 first, then to bf16 (round to nearest even). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double scale, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < (n + 1) / 2; ++m) {
    double a, b;
    normal_pair(key, (uint64_t)m, &a, &b);
    out[2 * m] = f32_to_bf16_rne((float)(scale * a));
    if (2 * m + 1 < n) out[2 * m + 1] = f32_to_bf16_rne((float)(scale * b));
  }
}

void synth_uniform_f32(uint64_t seed, uint64_t stream, int64_t n, double lo, double hi, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(lo + (hi - lo) * unit53(mix64(key + ((uint64_t)i + 1) * GOLDEN)));
}

void synth_uniform_bf16(uint64_t seed, uint64_t stream, int64_t n, double lo, double hi, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)(lo + (hi - lo) * unit53(mix64(key + ((uint64_t)i + 1) * GOLDEN))));
}

/* Integers uniform on [lo, hi). */
void synth_uniform_int(uint64_t seed, uint64_t stream, int64_t n, int32_t lo, int32_t hi, int32_t* out) {
  uint64_t key = stream_key(seed, stream);
  uint64_t range = (uint64_t)((int64_t)hi - (int64_t)lo);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t u32 = mix64(key + ((uint64_t)i + 1) * GOLDEN) >> 32;
    out[i] = (int32_t)((int64_t)lo + (int64_t)((u32 * range) >> 32));
  }
}

/* Seeded permutation of [0, n) (Fisher-Yates driven by the same stream). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t u32 = mix64(key + ((uint64_t)(n - 1 - i) + 1) * GOLDEN) >> 32;
    int32_t j = (int32_t)((u32 * (uint64_t)(i + 1)) >> 32);
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

void synth_fill_f32(int64_t n, float v, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = v;
}

void synth_fill_bf16(int64_t n, float v, uint16_t* out) {
  uint16_t b = f32_to_bf16_rne(v);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = b;
}
