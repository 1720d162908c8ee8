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

}  // namespace

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
