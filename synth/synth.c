/*
 * Seeded, counter-based generator of synthetic decode-attention inputs.
 *
 * This file draws random numbers and lays them out; it contains none of the
 * attention method's arithmetic.  Every value is a pure function of
 * (seed, stream, logical index), never of the physical page layout or of the
 * number of threads, so the same inputs come out whatever the pool
 * permutation or the OpenMP thread count.
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used in counter mode: the
 * i-th draw of a stream is the SplitMix64 finaliser applied to
 * key + (i + 1) * 0x9E3779B97F4A7C15, where key identifies (seed, stream).
 * Normals: Box-Muller (cosine branch) from two uniform draws, in double.
 * Storage type: bf16 bit patterns, rounded to nearest-even from fp32 after the
 * double is rounded to fp32.
 *
 * Built with gcc as a plain shared library and called through ctypes.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of stream `stream` under `seed`. */
uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return sm64_mix(sm64_mix(seed + SM64_GAMMA) ^ sm64_mix(stream * 0xD1B54A32D192ED03ULL + 1));
}

static inline uint64_t draw(uint64_t key, uint64_t idx) {
  return sm64_mix(key + (idx + 1) * SM64_GAMMA);
}

/* Uniform in the open interval (0, 1), 53 bits. */
static inline double unif(uint64_t key, uint64_t idx) {
  return ((double)(draw(key, idx) >> 11) + 0.5) * 0x1p-53;
}

static inline double normal(uint64_t key, uint64_t idx) {
  const double u1 = unif(key, 2 * idx);
  const double u2 = unif(key, 2 * idx + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) /* inf or nan: keep class */
    return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t synth_bf16_from_double(double x) { return f32_to_bf16_rne((float)x); }

void synth_uniform(uint64_t key, uint64_t idx0, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unif(key, idx0 + (uint64_t)i);
}

void synth_normal_f64(uint64_t key, uint64_t idx0, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = normal(key, idx0 + (uint64_t)i);
}

void synth_normal_bf16(uint64_t key, uint64_t idx0, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)normal(key, idx0 + (uint64_t)i));
}

void synth_raw_u64(uint64_t key, uint64_t idx0, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, idx0 + (uint64_t)i);
}

/*
 * Fill the tokens [t0, t1) of sequence b into a plain paged pool
 * pool[num_pool_pages][hkv][page][d] (bf16 bits), through page_row (the
 * sequence's logical->physical page map).  Value of (b, t, g, c):
 *     bf16(scale[g*d + c] * N(key, ((b * 2^24 + t) * hkv + g) * d + c))
 * scale may be NULL (all ones).
 */
void synth_fill_pool_seq(uint64_t key, int32_t b, int64_t t0, int64_t t1, int32_t hkv, int32_t d,
                         int32_t page, const int32_t* page_row, const double* scale,
                         uint16_t* pool) {
#pragma omp parallel for schedule(static)
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t phys = page_row[t / page];
    const int64_t slot = t % page;
    for (int32_t g = 0; g < hkv; ++g) {
      uint16_t* dst = pool + (((phys * hkv + g) * page + slot) * d);
      const uint64_t base = (((uint64_t)b << 24) + (uint64_t)t) * (uint64_t)hkv + (uint64_t)g;
      for (int32_t c = 0; c < d; ++c) {
        double v = normal(key, base * (uint64_t)d + (uint64_t)c);
        if (scale) v *= scale[g * d + c];
        dst[c] = f32_to_bf16_rne((float)v);
      }
    }
  }
}

/*
 * Same value rule as synth_fill_pool_seq, written token-major into
 * out[n][hkv][d] for tokens t0 .. t0+n-1 of sequence b (used for the K/V of
 * tokens appended during decode).
 */
void synth_fill_tokens(uint64_t key, int32_t b, int64_t t0, int64_t n, int32_t hkv, int32_t d,
                       const double* scale, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = t0 + i;
    for (int32_t g = 0; g < hkv; ++g) {
      const uint64_t base = (((uint64_t)b << 24) + (uint64_t)t) * (uint64_t)hkv + (uint64_t)g;
      uint16_t* dst = out + (i * hkv + g) * d;
      for (int32_t c = 0; c < d; ++c) {
        double v = normal(key, base * (uint64_t)d + (uint64_t)c);
        if (scale) v *= scale[g * d + c];
        dst[c] = f32_to_bf16_rne((float)v);
      }
    }
  }
}
