// dev_common.h - gfx950 device helpers: residual split/join on packed
// 16-bit pairs, the uint16 moment codec, and 16-lane DPP reductions.
//
// Data layout convention: 16-bit streams are handled as 32-bit words holding
// two consecutive elements, the even element in the low half.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ps.h"

namespace ps {

// Global (HBM) address space: accesses through it compile to global_* rather
// than flat_* instructions (no LDS aperture check, uniform-base addressing).
#define GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_perm_b32 byte selectors. perm(s0, s1, sel) picks bytes of the 64-bit
// value {s0:s1} (s1 = bytes 0..3, s0 = bytes 4..7).
constexpr uint32_t kSelLoHalves = 0x05040100u;  // {s0.lo16, s1.lo16}
constexpr uint32_t kSelHiHalves = 0x07060302u;  // {s0.hi16, s1.hi16}

__device__ __forceinline__ uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// ---------------------------------------------------------------------------
// XCD-aware work order. MI355X dispatches consecutive workgroups round-robin
// over its 8 XCDs, each with its own L2 and address-translation caches, so in
// index order every XCD touches every page of the range in flight. This
// bijection on [0, gridDim.x) instead gives each XCD runs of CHUNK
// consecutive work items (chunk c of XCD x is items (8c + x)·CHUNK ...); the
// items past the last whole round of 8 chunks keep their own index.
// ---------------------------------------------------------------------------
constexpr uint32_t kXcdCount = 8;
constexpr uint32_t kXcdChunk = 2048;   // (N)AdamW step: 2048 items of 512 elements

template <uint32_t CHUNK = kXcdChunk>
__device__ __forceinline__ uint32_t xcd_item(uint32_t wg, uint32_t n_wg) {
  constexpr uint32_t kRound = kXcdCount * CHUNK;
  if (wg >= n_wg / kRound * kRound) return wg;
  const uint32_t x = wg % kXcdCount, l = wg / kXcdCount;
  return (l / CHUNK) * kRound + x * CHUNK + l % CHUNK;
}

// ---------------------------------------------------------------------------
// Residual split / join [KAHAN]: fp32 bits = hi << 16 | lo (TRUNC), or the
// round-to-nearest-away variant whose join subtracts the carry back out.
// ---------------------------------------------------------------------------

// Join the even (which = 0) or odd (which = 1) element of a packed pair.
template <int MODE>
__device__ __forceinline__ uint32_t join_pair_elem(uint32_t hi2, uint32_t lo2, int which) {
  uint32_t w = perm(hi2, lo2, which ? kSelHiHalves : kSelLoHalves);
  if (MODE == PS_SPLIT_NEAREST_AWAY) w -= (w & 0x8000u) << 1;  // hi -= lo >> 15 (mod 2^16)
  return w;
}

// Split two fp32 words into packed hi and lo pairs.
template <int MODE>
__device__ __forceinline__ void split_pair(uint32_t w_even, uint32_t w_odd, uint32_t& hi2, uint32_t& lo2) {
  lo2 = perm(w_odd, w_even, kSelLoHalves);
  if (MODE == PS_SPLIT_NEAREST_AWAY) {
    w_even += 0x8000u;
    w_odd += 0x8000u;
  }
  hi2 = perm(w_odd, w_even, kSelHiHalves);
}

// ---------------------------------------------------------------------------
// Stochastic rounding without a residual (split mode STOCHASTIC): random 16
// bits per element from a SplitMix64 stream (Steele, Lea, Flood, OOPSLA
// 2014) keyed on (seed, update number, tensor index).
// ---------------------------------------------------------------------------
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Start of the stream of tensor `tid` at update `step`.
__device__ __forceinline__ uint64_t sr_stream(uint64_t seed, uint32_t step, uint32_t tid) {
  return splitmix64_mix(seed ^ splitmix64_mix(((uint64_t)step << 32) | tid));
}

// Random bits of elements e .. e+7 (e a multiple of 8): outputs e/4 and
// e/4 + 1 of the stream, element e + j taking bits 16*(j % 4) of output
// e/4 + j/4.
__device__ __forceinline__ void sr_bits8(uint64_t s, int64_t e, uint64_t* w2) {
  const uint64_t x = s + ((uint64_t)(e >> 2) + 1) * kGolden;
  w2[0] = splitmix64_mix(x);
  w2[1] = splitmix64_mix(x + kGolden);
}

// bf16 pair of two fp32 words rounded stochastically with the random 16-bit
// values r0 and r1: the upper halves of bits + r.
__device__ __forceinline__ uint32_t sr_pair(uint32_t w_even, uint32_t w_odd, uint32_t r0, uint32_t r1) {
  return perm(w_odd + r1, w_even + r0, kSelHiHalves);
}

// bf16 pair -> two fp32 values.
__device__ __forceinline__ float bf16_lo(uint32_t g2) { return __uint_as_float(g2 << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t g2) { return __uint_as_float(g2 & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Moment codec [NADAM second post]: 1/4-power companding, per-block scale.
// D(h) = ((h*K)^2)^2 with K = fp32(1/Q).
// ---------------------------------------------------------------------------

constexpr float kK15 = 3.05185094e-05f;  // fp32(1/32767) = 0x38000100
constexpr float kK16 = 1.52590219e-05f;  // fp32(1/65535) = 0x37800080
constexpr float kMagic = 8388608.0f;     // 2^23

// Decoder offsets: a code c arrives as the float 2^23 + c, and
// fma(2^23 + c, K, -(2^23 + bias) * K) is (c - bias) * K rounded once, i.e.
// exactly the product k * K, because both offsets are fp32 numbers:
// (2^23 + 2^15) * K15 = 2^8 + 2^0 + 2^-7 + 2^-15 and 2^23 * K16 = 2^7 + 2^-9.
constexpr float kDecOffS = -(256.0f + 1.0f + 0x1p-7f + 0x1p-15f);
constexpr float kDecOffU = -(128.0f + 0x1p-9f);
static_assert((8388608.0 + 32768.0) * (double)kK15 == -(double)kDecOffS, "signed decoder offset is not exact");
static_assert(8388608.0 * (double)kK16 == -(double)kDecOffU, "unsigned decoder offset is not exact");

__device__ __forceinline__ float dmag(float h, float K) {
  float a = h * K;
  float t = a * a;
  return t * t;
}

// Code value as float, exactly: (2^23 | c) as float is 2^23 + c.
__device__ __forceinline__ float code_lo_f(uint32_t c2) { return __uint_as_float(perm(0x4B000000u, c2, 0x07060100u)); }
__device__ __forceinline__ float code_hi_f(uint32_t c2) { return __uint_as_float(perm(0x4B000000u, c2, 0x07060302u)); }

// Signed decode of one code given as (2^23 + c): sign(k) * D(|k|) * s, k = c - 32768.
__device__ __forceinline__ float dec_signed(float magic_c, float s) {
  float t = __builtin_fmaf(magic_c, kK15, kDecOffS);  // k * K15, one rounding
  // t*|t| squares the magnitude and keeps the sign, so sign(k) * D(|k|) * s
  // comes out of the same three roundings with no separate sign step.
  t = t * __builtin_fabsf(t);
  t = t * __builtin_fabsf(t);
  return t * s;
}

__device__ __forceinline__ float dec_unsigned(float magic_c, float s) {
  const float a = __builtin_fmaf(magic_c, kK16, kDecOffU);  // k * K16, one rounding
  const float t = a * a;
  return (t * t) * s;
}

// Code magnitude of x in [0, 1 + 2^-23] given y ~ x^(1/4) (a few ulp): the
// nearest code k0 = rint(y*Q) is exact except next to a half-way point, so
// only the boundary on y's side of k0 is tested, with D evaluated exactly as
// the definition does. Equal to the definition whenever |y*Q - (x^(1/4))*Q|
// stays well below 1/2 code.
// The result is biased: 0x4B000000 + k (the bit pattern of 2^23 + k, less
// or more one), so its low 16 bits are k and bits 16..23 are zero; callers
// that keep only the low half need no unbiasing.
template <int Q>
__device__ __forceinline__ uint32_t code_mag_biased(float x, float y) {
  constexpr float K = (Q == 32767) ? kK15 : kK16;
  const float q = (float)Q;
  float z = __builtin_fmaf(y, q, kMagic);  // 2^23 + rint(y*Q)
  float kf = z - kMagic;
  // y*Q - k0, exact; +0 when equal (never -0), so its sign bit is "below k0"
  float dl = __builtin_fmaf(y, q, -kf);
  float T = dmag(kf + __builtin_copysignf(0.5f, dl), K);
  return __float_as_uint(z) - (__float_as_uint(dl) >> 31) + (x >= T ? 1u : 0u);
}

template <int Q>
__device__ __forceinline__ uint32_t code_mag(float x, float y) {
  return code_mag_biased<Q>(x, y) - 0x4B000000u;
}

// Two 16-bit codes (low halves of their words) packed as one word, even
// element in the low half.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t even, uint32_t odd) { return perm(odd, even, kSelLoHalves); }

__device__ __forceinline__ float fast_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

// Correctly rounded sqrt for v == 0 or v >= 2^-96 (finite): the hardware
// square root is within one ulp, and the exact residuals v - s'*s of its two
// neighbours (one fma each, normal-range results) decide which of the three
// candidates is the rounded root. For 0 < v < 2^-96 use __builtin_sqrtf.
__device__ __forceinline__ float sqrt_rn_fast(float v) {
  float s = __builtin_amdgcn_sqrtf(v);
  float sm = __uint_as_float(__float_as_uint(s) - 1u);
  float sp = __uint_as_float(__float_as_uint(s) + 1u);
  float rm = __builtin_fmaf(-sm, s, v);
  float rp = __builtin_fmaf(-sp, s, v);
  s = rm <= 0.0f ? sm : s;
  s = rp > 0.0f ? sp : s;
  return s;
}

// Signed code of m given inv = 1/scale (0 for a flushed block), in the low
// 16 bits of the result (the upper bits are not zero: pack with pack_lo16).
__device__ __forceinline__ uint32_t enc_signed_lo16(float m, float inv) {
  float x = __builtin_fabsf(m) * inv;
  uint32_t k = code_mag_biased<32767>(x, fast_sqrt(fast_sqrt(x)));
  // 32768 - k for m < 0 (k = 0 for -0), else 32768 + k: negate k by the sign
  // mask; the bias is a multiple of 2^16 and leaves the low half alone
  const uint32_t neg = (uint32_t)((int32_t)__float_as_uint(m) >> 31);
  return 32768u + ((k ^ neg) - neg);
}

__device__ __forceinline__ uint32_t enc_signed(float m, float inv) { return enc_signed_lo16(m, inv) & 0xFFFFu; }

// Unsigned code of v >= 0 given inv = 1/scale and y ~ (v*inv)^(1/4), in the
// low 16 bits of the result (pack with pack_lo16).
__device__ __forceinline__ uint32_t enc_unsigned_y_lo16(float v, float inv, float y) {
  return code_mag_biased<65535>(v * inv, y);
}

__device__ __forceinline__ uint32_t enc_unsigned(float v, float inv) {
  float x = __builtin_fabsf(v) * inv;
  return code_mag<65535>(x, fast_sqrt(fast_sqrt(x)));
}

// ---------------------------------------------------------------------------
// 16-lane (one DPP row) butterfly max: every lane of the row gets the max.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float x) {
  x = __builtin_fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = __builtin_fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = __builtin_fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = __builtin_fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}

// Max over the 32 lanes of a row pair (rows 0-1 and rows 2-3 of the wave):
// the row butterfly, then one exchange of the two rows (v_permlane16_swap
// hands each row the other row's values).
__device__ __forceinline__ float row32_max(float x) {
  x = row16_max(x);
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// The same maxima on the bit patterns of non-negative floats (their unsigned
// order is the float order): the max folds into one DPP instruction per step
// and needs no NaN quieting.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t row32_max_u32(uint32_t x) {
  x = __builtin_elementwise_max(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = __builtin_elementwise_max(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = __builtin_elementwise_max(x, dpp_u32<0x141>(x));  // row_half_mirror
  x = __builtin_elementwise_max(x, dpp_u32<0x140>(x));  // row_mirror
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return __builtin_elementwise_max((uint32_t)p[0], (uint32_t)p[1]);
}

// Block scale from the block max: blocks below the smallest normal are
// flushed to 0 so 1/scale never overflows; inv is 0 for them.
__device__ __forceinline__ void block_scale(float mx, float& s, float& inv) {
  bool keep = mx >= 0x1p-126f;
  s = keep ? mx : 0.0f;
  inv = keep ? 1.0f / mx : 0.0f;
}

// ---------------------------------------------------------------------------
// f24 moment storage [NADAM third post]: the upper three bytes of the fp32
// word, rounded to nearest (ties to even), packed little-endian at 3 bytes
// per value. Eight values occupy six 32-bit words.
// ---------------------------------------------------------------------------

// fp32 word rounded to its upper 24 bits (low byte zero).
__device__ __forceinline__ uint32_t f24_round(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7Fu + ((u >> 8) & 1u)) & 0xFFFFFF00u;
}

// Four values from three packed words (bytes 0..11).
__device__ __forceinline__ void f24_unpack4(uint32_t a, uint32_t b, uint32_t c, float* x) {
  x[0] = __uint_as_float(a << 8);                        // bytes 0..2
  x[1] = __uint_as_float(perm(b, a, 0x0504030Cu));       // bytes 3..5
  x[2] = __uint_as_float(perm(c, b, 0x0403020Cu));       // bytes 6..8
  x[3] = __uint_as_float(c & 0xFFFFFF00u);               // bytes 9..11
}

// Three packed words from four rounded words t[0..3] (low bytes zero).
__device__ __forceinline__ void f24_pack4(const uint32_t* t, uint32_t& a, uint32_t& b, uint32_t& c) {
  a = perm(t[1], t[0], 0x05030201u);
  b = perm(t[2], t[1], 0x06050302u);
  c = perm(t[3], t[2], 0x07060503u);
}

}  // namespace ps
