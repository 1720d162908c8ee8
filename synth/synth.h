/* synth.h - seeded synthetic inputs shared by the HIP library's tests, the
 * oracle's tests and the benchmark.
 *
 * This module holds no arithmetic of the optimizer method. It only turns a
 * (seed, stream, tensor, step, element) counter into reproducible bit
 * patterns, identically on the host and on the device, so that the oracle
 * and the GPU path can each build the same inputs without one handing data
 * to the other.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: output i
 * of a stream with key k is mix(k + (i + 1) * gamma).
 *
 * Normal variates: Irwin-Hall sum of twelve independent 32-bit uniforms
 * minus its mean, which has unit variance and a support of +-6 sigma. The sum
 * is an exact 64-bit integer, so the value is bit-identical on every platform;
 * only the final scaling by sigma (one double multiply) and the roundings to
 * fp32 and then bf16 (round-to-nearest-even both) are floating point.
 *
 * Compiled only by hipcc (host and device passes).
 */
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

#define SYN_FN __host__ __device__ static inline

#define SYN_GAMMA 0x9E3779B97F4A7C15ull

SYN_FN uint64_t syn_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Output i of the counter-based stream keyed by `key`. */
SYN_FN uint64_t syn_at(uint64_t key, uint64_t i) { return syn_mix(key + (i + 1) * SYN_GAMMA); }

/* Key of one (seed, stream, tensor, step) stream. Each field passes through the
 * bijective mixer before the next one is folded in. */
SYN_FN uint64_t syn_key(uint64_t seed, uint64_t stream, uint64_t tensor, uint64_t step) {
  uint64_t k = syn_mix(seed + SYN_GAMMA);
  k = syn_mix(k ^ (stream + 0x632BE59BD9B4E019ull));
  k = syn_mix(k ^ (tensor + 0x8CB92BA72F3D8DD7ull));
  k = syn_mix(k ^ (step + 0xC2B2AE3D27D4EB4Full));
  return k;
}

/* Irwin-Hall(12) standard normal approximation for element i, as an exact
 * multiple of 2^-32 returned in double. */
SYN_FN double syn_std_normal(uint64_t key, uint64_t i) {
  int64_t acc = 0;
  for (int r = 0; r < 6; ++r) {
    uint64_t u = syn_at(key, 6 * i + (uint64_t)r);
    acc += (int64_t)(u & 0xFFFFFFFFull) + (int64_t)(u >> 32);
  }
  acc -= (int64_t)6 << 32;
  return (double)acc * 0x1p-32;
}

SYN_FN uint32_t syn_f32_bits(float f) {
  union { float f; uint32_t u; } c; c.f = f; return c.u;
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs). */
SYN_FN uint16_t syn_bf16_rne(float f) {
  uint32_t b = syn_f32_bits(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* bf16 bit pattern of sigma * N(0,1) for element i; with probability
 * `outlier_p` (decided by a second stream) the value is multiplied by
 * `outlier_scale` before rounding. */
SYN_FN uint16_t syn_bf16_normal(uint64_t key, uint64_t okey, uint64_t i, double sigma,
                                double outlier_p, double outlier_scale) {
  double x = syn_std_normal(key, i) * sigma;
  if (outlier_p > 0.0) {
    double u = (double)(syn_at(okey, i) >> 11) * 0x1p-53;
    if (u < outlier_p) x = x * outlier_scale;
  }
  return syn_bf16_rne((float)x);
}

/* Uniform 16-bit pattern for element i: four elements per 64-bit output. */
SYN_FN uint16_t syn_u16_uniform(uint64_t key, uint64_t i) {
  uint64_t u = syn_at(key, i >> 2);
  return (uint16_t)(u >> (16 * (i & 3)));
}
