/*
 * Seeded synthetic inputs for the Llama decoder step: weights, norm gains, token ids, pre-filled KV
 * rows and per-row context lengths.  This file holds no step of the decoder's arithmetic; it only
 * draws numbers.  Both the GPU path's harness and the CPU oracle's tests read what it writes.
 *
 * Generator: the counter-based draw published with bend-ml-llama (main.bend, "Sampling" section,
 * `hash32` and `uniform`): hash32 is Chris Wellons' lowbias32 (public domain), and draw n of a seed
 * is the top 24 bits of hash32(hash32(seed) + n).  Nothing is carried between draws, so any slice
 * of any tensor can be regenerated on its own (the large pre-filled caches are made in pieces).
 *
 * Normal draws use Box-Muller in double precision on draws 2i and 2i+1; the result is rounded to
 * F32 once, then (for bf16 tensors) to bf16 with round-to-nearest-even on the F32 bits.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see synth/build.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 2146121005u; /* 0x7feb352d */
  x ^= x >> 15;
  x *= 2221713035u; /* 0x846ca68b */
  x ^= x >> 16;
  return x;
}

/* top 24 bits of draw n */
static inline uint32_t draw24(uint32_t hseed, uint32_t n) { return lowbias32(hseed + n) >> 8; }

uint32_t synth_hash32(uint32_t x) { return lowbias32(x); }

/* draw n of a seed as an F32 in [0, 1): exact (24 bits times 2^-24) */
float synth_uniform(uint32_t seed, uint32_t n) {
  return (float)draw24(lowbias32(seed), n) * 5.9604644775390625e-8f;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* standard normals z[2p], z[2p+1] from draws 2p and 2p+1 (Box-Muller, double precision) */
static inline void normal_pair(uint32_t hseed, uint64_t p, double *z0, double *z1) {
  double u1 = (double)draw24(hseed, (uint32_t)(2 * p)) * (1.0 / 16777216.0);
  double u2 = (double)draw24(hseed, (uint32_t)(2 * p + 1)) * (1.0 / 16777216.0);
  double r = sqrt(-2.0 * log(1.0 - u1)); /* 1 - u1 is in (0, 1] */
  double th = 6.283185307179586 * u2;
  *z0 = r * cos(th);
  *z1 = r * sin(th);
}

/* F32(mean + std * z[i]) for i in [start, start + n): pairs are computed once, both halves kept */
static void normal_span(uint32_t seed, uint64_t start, uint64_t n, double mean, double std, float *outf,
                        uint16_t *outbf) {
  uint32_t hs = lowbias32(seed);
  uint64_t p0 = start >> 1, p1 = (start + n + 1) >> 1;
#pragma omp parallel for schedule(static)
  for (int64_t p = (int64_t)p0; p < (int64_t)p1; ++p) {
    double z[2];
    normal_pair(hs, (uint64_t)p, &z[0], &z[1]);
    for (int h = 0; h < 2; ++h) {
      uint64_t i = 2 * (uint64_t)p + (uint64_t)h;
      if (i < start || i >= start + n) continue;
      float v = (float)(mean + std * z[h]);
      if (outf) outf[i - start] = v;
      else outbf[i - start] = f32_to_bf16_rne(v);
    }
  }
}

/* out[k] = F32(mean + std * z[start + k]), k < n */
void synth_normal_f32(uint32_t seed, uint64_t start, uint64_t n, double mean, double std, float *out) {
  normal_span(seed, start, n, mean, std, out, 0);
}

/* the same values rounded F32 -> bf16 (RNE), stored as the upper 16 bits of the F32 */
void synth_normal_bf16(uint32_t seed, uint64_t start, uint64_t n, double mean, double std, uint16_t *out) {
  normal_span(seed, start, n, mean, std, 0, out);
}

/* uniform token ids in [0, vocab): (draw24 * vocab) >> 24, integer only */
void synth_tokens(uint32_t seed, uint64_t start, uint64_t n, uint32_t vocab, int32_t *out) {
  uint32_t hs = lowbias32(seed);
  for (uint64_t k = 0; k < n; ++k)
    out[k] = (int32_t)(((uint64_t)draw24(hs, (uint32_t)(start + k)) * vocab) >> 24);
}

/* uniform integers in [lo, hi]: lo + (draw24 * (hi - lo + 1)) >> 24 */
void synth_int_range(uint32_t seed, uint64_t start, uint64_t n, int32_t lo, int32_t hi, int32_t *out) {
  uint32_t hs = lowbias32(seed);
  uint64_t span = (uint64_t)(hi - lo) + 1u;
  for (uint64_t k = 0; k < n; ++k) out[k] = lo + (int32_t)(((uint64_t)draw24(hs, (uint32_t)(start + k)) * span) >> 24);
}

/*
 * Integer-exact uniform fill for pre-filled cache rows: x = (int)(draw24 - 2^23) * step, one F32
 * multiply of an exactly representable integer by an F32 constant, so every platform produces the
 * same bits; then (bf16 caches) RNE to bf16.  step = amplitude * 2^-23, rounded to F32 by the caller.
 */
void synth_uniform_kv_f32(uint32_t seed, uint64_t start, uint64_t n, float step, float *out) {
  uint32_t hs = lowbias32(seed);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) {
    int32_t iv = (int32_t)draw24(hs, (uint32_t)(start + (uint64_t)k)) - 8388608;
    out[k] = (float)iv * step;
  }
}

void synth_uniform_kv_bf16(uint32_t seed, uint64_t start, uint64_t n, float step, uint16_t *out) {
  uint32_t hs = lowbias32(seed);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) {
    int32_t iv = (int32_t)draw24(hs, (uint32_t)(start + (uint64_t)k)) - 8388608;
    out[k] = f32_to_bf16_rne((float)iv * step);
  }
}
