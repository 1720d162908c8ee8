// k_elementwise.hip - standalone residual split/join [KAHAN, copy_kahan_
// docstring] and moment encode/decode [NADAM second post] kernels.
//
// split/join: one lane handles 8 consecutive elements (one 16-byte access of
// 16-bit data, two of fp32). encode: each wave takes 4 blocks of 256, 16
// lanes per block, 16 elements per lane, DPP row max. decode: 8 elements per
// lane, one scale per lane (8 divides 256). Every launch has one unit of work
// per lane (the grid covers the array; the loops run once), so workgroups
// dispatched in index order sweep the arrays front to back: that measured
// 15-25% faster than a grid of 8 workgroups per CU striding over them.
// Loads and the 16-bit stores carry the non-temporal hint (each byte is
// touched once); the fp32 stores stay plain, which measured faster for them.
#include "dev_common.h"
#include "ps_internal.h"

namespace ps {
namespace {

constexpr int kThreads = 256;
// Each XCD takes runs of 256 consecutive workgroups (512K elements; the
// encoder's workgroups cover twice as many, so half as many of them): 2-6%
// faster than plain index order on 2^30 elements, runs of 512 to 2048 slower.
constexpr uint32_t kEwXcdChunk = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void ld_f8(const float* p, int64_t e, int64_t n, float* d) {
  if (e + 8 <= n) {
    const f32x4 a = __builtin_nontemporal_load((const GLOBAL f32x4*)(p + e));
    const f32x4 b = __builtin_nontemporal_load((const GLOBAL f32x4*)(p + e + 4));
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
  } else {
    for (int j = 0; j < 8; ++j) d[j] = (e + j < n) ? p[e + j] : 0.0f;
  }
}

__device__ __forceinline__ void st_f8(float* p, int64_t e, int64_t n, const float* s) {
  if (e + 8 <= n) {
    *reinterpret_cast<float4*>(p + e) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(p + e + 4) = make_float4(s[4], s[5], s[6], s[7]);
  } else {
    for (int j = 0; j < 8; ++j)
      if (e + j < n) p[e + j] = s[j];
  }
}

__device__ __forceinline__ void ld_h8(const uint16_t* p, int64_t e, int64_t n, uint32_t fill, uint32_t* d) {
  if (e + 8 <= n) {
    const u32x4 v = __builtin_nontemporal_load((const GLOBAL u32x4*)(p + e));
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else {
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = (e + 2 * j < n) ? p[e + 2 * j] : (fill & 0xFFFFu);
      uint32_t hi = (e + 2 * j + 1 < n) ? p[e + 2 * j + 1] : (fill >> 16);
      d[j] = lo | (hi << 16);
    }
  }
}

__device__ __forceinline__ void st_h8(uint16_t* p, int64_t e, int64_t n, const uint32_t* s) {
  if (e + 8 <= n) {
    __builtin_nontemporal_store(u32x4{s[0], s[1], s[2], s[3]}, (GLOBAL u32x4*)(p + e));
  } else {
    for (int j = 0; j < 8; ++j)
      if (e + j < n) p[e + j] = (uint16_t)(s[j >> 1] >> (16 * (j & 1)));
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_split(const float* __restrict__ w, uint16_t* __restrict__ hi,
                                                    uint16_t* __restrict__ lo, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * 8;
  for (int64_t e = ((int64_t)xcd_item<kEwXcdChunk>(blockIdx.x, gridDim.x) * kThreads + threadIdx.x) * 8; e < n; e += stride) {
    float f[8];
    uint32_t h[4], l[4];
    ld_f8(w, e, n, f);
#pragma unroll
    for (int j = 0; j < 4; ++j) split_pair<MODE>(__float_as_uint(f[2 * j]), __float_as_uint(f[2 * j + 1]), h[j], l[j]);
    st_h8(hi, e, n, h);
    st_h8(lo, e, n, l);
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_join(const uint16_t* __restrict__ hi, const uint16_t* __restrict__ lo,
                                                   float* __restrict__ w, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * 8;
  for (int64_t e = ((int64_t)xcd_item<kEwXcdChunk>(blockIdx.x, gridDim.x) * kThreads + threadIdx.x) * 8; e < n; e += stride) {
    uint32_t h[4], l[4];
    float f[8];
    ld_h8(hi, e, n, 0u, h);
    ld_h8(lo, e, n, 0u, l);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(join_pair_elem<MODE>(h[j], l[j], 0));
      f[2 * j + 1] = __uint_as_float(join_pair_elem<MODE>(h[j], l[j], 1));
    }
    st_f8(w, e, n, f);
  }
}

// Encode: wave = 4 blocks of 256, 16 lanes per block, 16 elements per lane.
template <int KIND>
__global__ __launch_bounds__(kThreads) void k_encode(const float* __restrict__ x, uint16_t* __restrict__ code,
                                                     float* __restrict__ scale, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int b = lane >> 4, r = lane & 15;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(xcd_item<kEwXcdChunk / 2>(blockIdx.x, gridDim.x) * (kThreads / 64) + (threadIdx.x >> 6));
  const uint32_t n_waves = gridDim.x * (kThreads / 64);
  const int64_t n_items = (n + kItemElems - 1) / kItemElems;
  for (int64_t item = wave; item < n_items; item += n_waves) {
    const int64_t elem0 = item * kItemElems;
    const int64_t blk = (elem0 >> 8) + b;
    const int64_t ea = elem0 + b * kBlock + r * 8, eb = ea + 128;
    float v[16];
    ld_f8(x, ea, n, v);
    ld_f8(x, eb, n, v + 8);
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[j]));
    float s, inv;
    block_scale(row16_max(mx), s, inv);
    uint32_t c[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t c0 = KIND == PS_MOMENT_SIGNED ? enc_signed(v[2 * w], inv) : enc_unsigned(v[2 * w], inv);
      uint32_t c1 = KIND == PS_MOMENT_SIGNED ? enc_signed(v[2 * w + 1], inv) : enc_unsigned(v[2 * w + 1], inv);
      c[w] = c0 | (c1 << 16);
    }
    st_h8(code, ea, n, c);
    st_h8(code, eb, n, c + 4);
    if (r == 0 && blk * kBlock < n) scale[blk] = s;
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void k_decode(const uint16_t* __restrict__ code, const float* __restrict__ scale,
                                                     float* __restrict__ x, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * 8;
  for (int64_t e = ((int64_t)xcd_item<kEwXcdChunk>(blockIdx.x, gridDim.x) * kThreads + threadIdx.x) * 8; e < n; e += stride) {
    uint32_t c[4];
    float f[8];
    ld_h8(code, e, n, KIND == PS_MOMENT_SIGNED ? 0x80008000u : 0u, c);
    const float s = scale[e >> 8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (KIND == PS_MOMENT_SIGNED) {
        f[2 * j] = dec_signed(code_lo_f(c[j]), s);
        f[2 * j + 1] = dec_signed(code_hi_f(c[j]), s);
      } else {
        f[2 * j] = dec_unsigned(code_lo_f(c[j]), s);
        f[2 * j + 1] = dec_unsigned(code_hi_f(c[j]), s);
      }
    }
    st_f8(x, e, n, f);
  }
}

// Workgroups covering n elements at units_per_block each (at most 2^31 - 1,
// which covers every n the ABI accepts; the kernels' loops handle any rest).
uint32_t grid_for(int64_t units_per_block, int64_t n) {
  int64_t g = (n + units_per_block - 1) / units_per_block;
  if (g > 0x7FFFFFFF) g = 0x7FFFFFFF;
  if (g < 1) g = 1;
  return (uint32_t)g;
}

}  // namespace

ps_status launch_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, int mode, hipStream_t s) {
  dim3 grid(grid_for(kThreads * 8, n));
  if (mode == PS_SPLIT_TRUNC)
    hipLaunchKernelGGL(k_split<PS_SPLIT_TRUNC>, grid, dim3(kThreads), 0, s, w, hi, lo, n);
  else
    hipLaunchKernelGGL(k_split<PS_SPLIT_NEAREST_AWAY>, grid, dim3(kThreads), 0, s, w, hi, lo, n);
  return hip_check(hipGetLastError(), "k_split launch");
}

ps_status launch_join(const uint16_t* hi, const uint16_t* lo, float* w, int64_t n, int mode, hipStream_t s) {
  dim3 grid(grid_for(kThreads * 8, n));
  if (mode == PS_SPLIT_TRUNC)
    hipLaunchKernelGGL(k_join<PS_SPLIT_TRUNC>, grid, dim3(kThreads), 0, s, hi, lo, w, n);
  else
    hipLaunchKernelGGL(k_join<PS_SPLIT_NEAREST_AWAY>, grid, dim3(kThreads), 0, s, hi, lo, w, n);
  return hip_check(hipGetLastError(), "k_join launch");
}

ps_status launch_encode(const float* x, uint16_t* code, float* scale, int64_t n, int kind, hipStream_t s) {
  dim3 grid(grid_for((int64_t)kItemElems * (kThreads / 64), n));
  if (kind == PS_MOMENT_SIGNED)
    hipLaunchKernelGGL(k_encode<PS_MOMENT_SIGNED>, grid, dim3(kThreads), 0, s, x, code, scale, n);
  else
    hipLaunchKernelGGL(k_encode<PS_MOMENT_UNSIGNED>, grid, dim3(kThreads), 0, s, x, code, scale, n);
  return hip_check(hipGetLastError(), "k_encode launch");
}

ps_status launch_decode(const uint16_t* code, const float* scale, float* x, int64_t n, int kind, hipStream_t s) {
  dim3 grid(grid_for(kThreads * 8, n));
  if (kind == PS_MOMENT_SIGNED)
    hipLaunchKernelGGL(k_decode<PS_MOMENT_SIGNED>, grid, dim3(kThreads), 0, s, code, scale, x, n);
  else
    hipLaunchKernelGGL(k_decode<PS_MOMENT_UNSIGNED>, grid, dim3(kThreads), 0, s, code, scale, x, n);
  return hip_check(hipGetLastError(), "k_decode launch");
}

}  // namespace ps
