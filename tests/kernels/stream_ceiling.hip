// stream_ceiling.hip - streaming kernels with the fused (N)AdamW step's memory
// access pattern and no optimizer arithmetic, run by bench.py over the same
// state arrays as the step: the practical HBM ceiling for that pattern on the
// GPU at hand, next to the 8 TB/s peak. Built into tests/kernels/libps_probe.so.
//
// Pattern (as k_adam_step): one 512-element item (two 256-element blocks) per
// 64-lane workgroup, a block's 32 lanes each taking 8 consecutive elements;
// 16-byte non-temporal loads of the five 16-bit streams (weight hi and lo,
// gradient, m and v codes) and the item's block scales of both moments;
// 16-byte non-temporal stores of four streams (hi, lo, m, v) and the scales;
// the same XCD-aware item order (runs of 2048 items per XCD). The stored
// words are xor combinations of the loaded ones, so nothing is elided.
//   mode 0: the step's mix, 18 B per element + 16 B per block
//   mode 1: the five streams and scale reads only (10 B per element + 8 B
//           per block); a word is stored only if an impossible value appears
//   mode 2: the stochastic-rounding step's mix (no residual stream: reads of
//           hi, g, m and v codes, writes of hi, m, v; 14 B per element + 16 B
//           per block)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../precision_state_amd/csrc/dev_common.h"

namespace {

using ps::u32x4;

__device__ __forceinline__ u32x4 ld(const uint16_t* p) {
  return __builtin_nontemporal_load((const GLOBAL u32x4*)p);
}
__device__ __forceinline__ void st(uint16_t* p, u32x4 v) { __builtin_nontemporal_store(v, (GLOBAL u32x4*)p); }

template <int MODE>
__global__ __launch_bounds__(64) void k_ceiling(uint16_t* hi, uint16_t* lo, const uint16_t* g, uint16_t* mc,
                                                uint16_t* vc, float* ms, float* vs, uint32_t* sink) {
  const uint32_t item = ps::xcd_item<>(blockIdx.x, gridDim.x);
  const uint32_t lane = threadIdx.x, b = lane >> 5, r = lane & 31;
  const size_t e = (size_t)item * 512 + b * 256 + r * 8;
  const size_t blk = (size_t)item * 2 + b;
  const u32x4 vh = ld(hi + e), vl = MODE == 2 ? u32x4{0u, 0u, 0u, 0u} : ld(lo + e), vg = ld(g + e),
              vm = ld(mc + e), vv = ld(vc + e);
  const float sm = ((const GLOBAL float*)ms)[blk], sv = ((const GLOBAL float*)vs)[blk];
  if (MODE == 0 || MODE == 2) {
    st(hi + e, vh ^ vg);
    if (MODE == 0) st(lo + e, vl ^ vg);
    st(mc + e, vm ^ vg);
    st(vc + e, vv ^ vg);
    if (r == 0) {
      ((GLOBAL float*)ms)[blk] = sm;
      ((GLOBAL float*)vs)[blk] = sv;
    }
  } else {
    const u32x4 x = vh ^ vl ^ vg ^ vm ^ vv;
    const uint32_t y = x.x ^ x.y ^ x.z ^ x.w ^ __float_as_uint(sm) ^ __float_as_uint(sv);
    if (y == 0x9E3779B9u && e == 0) sink[0] = y;
  }
}

// ---- the standalone elementwise kernels' access patterns, no arithmetic ----
// Same grids, XCD-aware order, lane layouts and cache hints as k_split, k_join,
// k_encode and k_decode over full tiles (n a multiple of 4096); stored words
// are xor or byte-permute combinations of the loaded ones.
//   kind 0 (split): 32 B of fp32 read per lane, 16 B to each of two 16-bit streams
//   kind 1 (join): 16 B from each of two 16-bit streams, 32 B of fp32 written (plain stores)
//   kind 2 (encode): 64 B of fp32 read per lane (runs at +0 and +128 elements of a
//           256-block, 16 lanes per block), 32 B of codes written, one scale per block
//   kind 3 (decode): 16 B of codes and a scale read per lane, 32 B of fp32 written (plain)
constexpr int kEwT = 256;
__device__ __forceinline__ u32x4 ldw(const void* p) { return __builtin_nontemporal_load((const GLOBAL u32x4*)p); }
__device__ __forceinline__ void stw(void* p, u32x4 v) { __builtin_nontemporal_store(v, (GLOBAL u32x4*)p); }
__device__ __forceinline__ void stw_plain(void* p, u32x4 v) { *(GLOBAL u32x4*)p = v; }

__global__ __launch_bounds__(kEwT) void k_ew_split(const float* w, uint16_t* hi, uint16_t* lo) {
  const size_t e = ((size_t)ps::xcd_item<256>(blockIdx.x, gridDim.x) * kEwT + threadIdx.x) * 8;
  const u32x4 a = ldw(w + e), b = ldw(w + e + 4);
  stw(hi + e, u32x4{__builtin_amdgcn_perm(a.y, a.x, 0x07060302u), __builtin_amdgcn_perm(a.w, a.z, 0x07060302u),
                    __builtin_amdgcn_perm(b.y, b.x, 0x07060302u), __builtin_amdgcn_perm(b.w, b.z, 0x07060302u)});
  stw(lo + e, u32x4{__builtin_amdgcn_perm(a.y, a.x, 0x05040100u), __builtin_amdgcn_perm(a.w, a.z, 0x05040100u),
                    __builtin_amdgcn_perm(b.y, b.x, 0x05040100u), __builtin_amdgcn_perm(b.w, b.z, 0x05040100u)});
}
__global__ __launch_bounds__(kEwT) void k_ew_join(const uint16_t* hi, const uint16_t* lo, float* w) {
  const size_t e = ((size_t)ps::xcd_item<256>(blockIdx.x, gridDim.x) * kEwT + threadIdx.x) * 8;
  const u32x4 h = ldw(hi + e), l = ldw(lo + e);
  stw_plain(w + e, u32x4{__builtin_amdgcn_perm(h.x, l.x, 0x05040100u), __builtin_amdgcn_perm(h.x, l.x, 0x07060302u),
                         __builtin_amdgcn_perm(h.y, l.y, 0x05040100u), __builtin_amdgcn_perm(h.y, l.y, 0x07060302u)});
  stw_plain(w + e + 4, u32x4{__builtin_amdgcn_perm(h.z, l.z, 0x05040100u), __builtin_amdgcn_perm(h.z, l.z, 0x07060302u),
                             __builtin_amdgcn_perm(h.w, l.w, 0x05040100u), __builtin_amdgcn_perm(h.w, l.w, 0x07060302u)});
}
__global__ __launch_bounds__(kEwT) void k_ew_encode(const float* x, uint16_t* code, float* scale) {
  const int lane = threadIdx.x & 63, b = lane >> 4, r = lane & 15;
  const size_t item = (size_t)ps::xcd_item<128>(blockIdx.x, gridDim.x) * (kEwT / 64) + (threadIdx.x >> 6);
  const size_t elem0 = item * 1024, blk = (elem0 >> 8) + b;
  const size_t ea = elem0 + b * 256 + r * 8, eb = ea + 128;
  const u32x4 a0 = ldw(x + ea), a1 = ldw(x + ea + 4), b0 = ldw(x + eb), b1 = ldw(x + eb + 4);
  stw(code + ea, a0 ^ a1);
  stw(code + eb, b0 ^ b1);
  if (r == 0) ((GLOBAL uint32_t*)scale)[blk] = a0.x ^ b1.w;
}
__global__ __launch_bounds__(kEwT) void k_ew_decode(const uint16_t* code, const float* scale, float* x) {
  const size_t e = ((size_t)ps::xcd_item<256>(blockIdx.x, gridDim.x) * kEwT + threadIdx.x) * 8;
  const u32x4 c = ldw(code + e);
  const uint32_t s = ((const GLOBAL uint32_t*)scale)[e >> 8];
  stw_plain(x + e, u32x4{c.x ^ s, c.y, c.z, c.w});
  stw_plain(x + e + 4, u32x4{c.x, c.y ^ s, c.z, c.w});
}

}  // namespace

// in0/in1/out0/out1 per kind: split (w, -, hi, lo); join (hi, lo, w, -);
// encode (x, -, code, scale); decode (code, scale, x, -). n a multiple of 4096.
extern "C" int probe_ew_ceiling(int kind, const void* in0, const void* in1, void* out0, void* out1, int64_t n,
                                hipStream_t s) {
  if (n <= 0 || n % 4096 != 0 || n / 2048 > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  const dim3 g8((uint32_t)(n / (kEwT * 8))), genc((uint32_t)(n / 4096));
  if (kind == 0)
    hipLaunchKernelGGL(k_ew_split, g8, dim3(kEwT), 0, s, (const float*)in0, (uint16_t*)out0, (uint16_t*)out1);
  else if (kind == 1)
    hipLaunchKernelGGL(k_ew_join, g8, dim3(kEwT), 0, s, (const uint16_t*)in0, (const uint16_t*)in1, (float*)out0);
  else if (kind == 2)
    hipLaunchKernelGGL(k_ew_encode, genc, dim3(kEwT), 0, s, (const float*)in0, (uint16_t*)out0, (float*)out1);
  else if (kind == 3)
    hipLaunchKernelGGL(k_ew_decode, g8, dim3(kEwT), 0, s, (const uint16_t*)in0, (const float*)in1, (float*)out0);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

extern "C" int probe_stream_ceiling(int mode, uint16_t* hi, uint16_t* lo, const uint16_t* g, uint16_t* mc,
                                    uint16_t* vc, float* ms, float* vs, uint32_t* sink, uint32_t n_items,
                                    hipStream_t s) {
  if (n_items == 0) return 0;
  if (mode == 0)
    hipLaunchKernelGGL(k_ceiling<0>, dim3(n_items), dim3(64), 0, s, hi, lo, g, mc, vc, ms, vs, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(k_ceiling<1>, dim3(n_items), dim3(64), 0, s, hi, lo, g, mc, vc, ms, vs, sink);
  else if (mode == 2)
    hipLaunchKernelGGL(k_ceiling<2>, dim3(n_items), dim3(64), 0, s, hi, lo, g, mc, vc, ms, vs, sink);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
