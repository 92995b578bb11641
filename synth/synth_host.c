/*
 * Seeded synthetic inputs (host side).
 *
 * This module only draws numbers; it holds none of the decode step's
 * arithmetic.  Both the oracle (through the test harness) and the GPU path
 * (through synth_dev.hip, a device copy of the same integer recipe) take their
 * inputs from it, so the two sides see bit-identical weights, caches, states
 * and tokens.
 *
 * Recipe, per tensor named `name` drawn with seed `seed`:
 *   key      = seed XOR FNV-1a-64(name)             (FNV-1a: Fowler/Noll/Vo)
 *   w_i      = SplitMix64 output for counter i      (Steele, Lea, Flood 2014)
 *   s_i      = sum of the four 16-bit fields of w_i  (integer, 0..262140)
 *   z_i      = (float)(s_i - 131070) * scale        (one IEEE fp32 multiply)
 * The sum of four uniforms (Irwin-Hall, n = 4) has mean 131070 and standard
 * deviation sqrt(4 * (65536^2 - 1) / 12); `scale` = sigma / that deviation is
 * rounded to fp32 by the caller and passed in, so host and device evaluate the
 * same single rounding.  bf16 outputs round z_i to nearest-even.
 * Integers in [0, hi) take the high 32 bits of w_i times hi, shifted down 32.
 */
#include <stdint.h>
#include <stddef.h>

static inline uint64_t sm64(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline float irwin_hall4(uint64_t w, float scale) {
  int32_t s = (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
              (int32_t)((w >> 32) & 0xFFFF) + (int32_t)((w >> 48) & 0xFFFF);
  float f = (float)(s - 131070); /* exact: |s - 131070| < 2^24 */
  return f * scale;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  uint32_t u = v.u;
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t synth_key(uint64_t seed, const char* name) {
  uint64_t h = 0xCBF29CE484222325ull;
  for (const unsigned char* p = (const unsigned char*)name; *p; ++p) {
    h ^= *p;
    h *= 0x100000001B3ull;
  }
  return seed ^ h;
}

void synth_normal_bf16(uint64_t key, float scale, uint16_t* out, int64_t n, int64_t offset) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(irwin_hall4(sm64(key, (uint64_t)(offset + i)), scale));
}

void synth_normal_f32(uint64_t key, float scale, float* out, int64_t n, int64_t offset) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = irwin_hall4(sm64(key, (uint64_t)(offset + i)), scale);
}

void synth_uniform_i32(uint64_t key, int32_t hi, int32_t* out, int64_t n, int64_t offset) {
  for (int64_t i = 0; i < n; ++i) {
    uint64_t w = sm64(key, (uint64_t)(offset + i));
    out[i] = (int32_t)(((w >> 32) * (uint64_t)(uint32_t)hi) >> 32);
  }
}

void synth_fill_u16(uint16_t value, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = value;
}
