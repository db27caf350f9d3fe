/*
 * Seeded synthetic inputs shared by the oracle and the GPU path.
 *
 * This file holds no attention or layout arithmetic: it only turns
 * (seed, stream, element index) into numbers.  Both sides of every parity
 * check consume the bytes written here.
 *
 * Generator: counter-based SplitMix64.  SplitMix64 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; constants as
 * in Vigna's public-domain splitmix64.c) advances a 64-bit state by the
 * golden-ratio increment 0x9E3779B97F4A7C15 and returns mix64(state).  Here the
 * k-th output of a stream is evaluated directly from its counter:
 *
 *     base(seed, stream) = mix64(seed * GAMMA + stream)
 *     word(seed, stream, k) = mix64(base + (k + 1) * GAMMA)
 *
 * so that any slice of a stream can be produced independently and in
 * parallel.  With base = s this is exactly the SplitMix64 sequence started
 * from state s.
 *
 * Normals: Box-Muller (Box and Muller, 1958).  Element e uses words 2*(e/2)
 * and 2*(e/2)+1 as u1, u2 in (0, 1]; element e is r*cos(t) when e is even
 * and r*sin(t) when odd, with r = sqrt(-2 ln u1), t = 2 pi u2.
 *
 * Rounding: value * scale is computed in double, rounded to fp32 by the C
 * conversion (round to nearest even), and for bf16 the fp32 bits are rounded
 * to the upper 16 bits with round-to-nearest-even.
 *
 * Uniform integers in [lo, hi]: lo + floor(u * (hi - lo + 1)) with
 * u = (word >> 11) * 2^-53 in [0, 1).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64(seed * GAMMA + stream);
}

static inline uint64_t word_at(uint64_t base, uint64_t k) {
  return mix64(base + (k + 1) * GAMMA);
}

/* Uniform in (0, 1]: never zero, so log() below is finite. */
static inline double unit_open0(uint64_t w) {
  return (double)((w >> 11) + 1) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t base, uint64_t e) {
  const uint64_t pair = e >> 1;
  const double u1 = unit_open0(word_at(base, 2 * pair));
  const double u2 = unit_open0(word_at(base, 2 * pair + 1));
  const double r = sqrt(-2.0 * log(u1));
  const double t = 6.283185307179586476925286766559 * u2;
  return (e & 1) ? r * sin(t) : r * cos(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  const uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb;
  return (uint16_t)(b >> 16);
}

/* Raw SplitMix64 words k = offset .. offset+count-1 of (seed, stream). */
void synth_words(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count,
                 uint64_t* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = word_at(base, offset + (uint64_t)i);
}

/* Plain SplitMix64 sequence from an explicit state (for checking the mixer
 * against published output values). */
void synth_splitmix64_sequence(uint64_t state, int64_t count, uint64_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = word_at(state, (uint64_t)i);
}

void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count,
                      double scale, double* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = normal_at(base, offset + (uint64_t)i) * scale;
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count,
                      double scale, float* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = (float)(normal_at(base, offset + (uint64_t)i) * scale);
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count,
                       double scale, uint16_t* out) {
  const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = f32_to_bf16_rne((float)(normal_at(base, offset + (uint64_t)i) * scale));
}

void synth_uniform_int(uint64_t seed, uint64_t stream, uint64_t offset, int64_t count,
                       int64_t lo, int64_t hi, int64_t* out) {
  const uint64_t base = stream_base(seed, stream);
  const double span = (double)(hi - lo + 1);
  for (int64_t i = 0; i < count; ++i) {
    const double u = (double)(word_at(base, offset + (uint64_t)i) >> 11) * (1.0 / 9007199254740992.0);
    int64_t v = lo + (int64_t)floor(u * span);
    if (v > hi) v = hi;
    out[i] = v;
  }
}
