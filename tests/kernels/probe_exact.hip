// probe_exact.hip - test-only kernels that evaluate the library's device
// arithmetic helpers (precision_state_amd/csrc/dev_common.h) over whole input
// ranges, for the exhaustive exactness tests in tests/test_gpu_exhaustive.py.
// Built into tests/kernels/libps_probe.so; the library itself never loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../precision_state_amd/csrc/dev_common.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kGrid = 65536;

// sqrt_rn_fast of the fp32 bit patterns first .. first + n - 1.
__global__ __launch_bounds__(kThreads) void k_sqrt_fast(uint32_t first, uint32_t n, uint32_t* out) {
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += kGrid * kThreads)
    out[i] = __float_as_uint(ps::sqrt_rn_fast(__uint_as_float(first + i)));
}

// The unsigned (exp_avg_sq) code of v at block scale s, as the fused step
// forms it: inv from the block scale, y = sqrt(sqrt(v) * sqrt(inv)) with the
// correctly rounded sqrt(v) (the library root for 0 < v < 2^-96, as the step
// chooses for such a wave).
__device__ __forceinline__ uint32_t fused_vcode(float v, float inv) {
  const float rv = (v == 0.0f || v >= 0x1p-96f) ? ps::sqrt_rn_fast(v) : __builtin_sqrtf(v);
  return ps::enc_unsigned_y_lo16(v, inv, ps::fast_sqrt(rv * ps::fast_sqrt(inv))) & 0xFFFFu;
}

// Every fp32 v in [0, s]: the fused step's code against the standalone
// encoder's (ps_encode_moments) code of the same v. counters[0] = number of
// differences, counters[1..16] = the first differing bit patterns.
__global__ __launch_bounds__(kThreads) void k_fused_vcode_diff(float s, uint32_t* counters) {
  float sc, inv;
  ps::block_scale(s, sc, inv);
  const uint32_t n = __float_as_uint(s) + 1u;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += kGrid * kThreads) {
    const float v = __uint_as_float(i);
    if (fused_vcode(v, inv) != ps::enc_unsigned(v, inv)) {
      const uint32_t k = atomicAdd(&counters[0], 1u);
      if (k < 16) counters[1 + k] = i;
    }
  }
}

// The fused step's codes of given values at block scale s.
__global__ __launch_bounds__(kThreads) void k_fused_vcode(float s, const float* v, uint32_t* out, uint32_t n) {
  float sc, inv;
  ps::block_scale(s, sc, inv);
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += kGrid * kThreads) out[i] = fused_vcode(v[i], inv);
}

uint32_t grid_for(uint32_t n) {
  const uint32_t g = (n + kThreads - 1) / kThreads;
  return g < kGrid ? (g ? g : 1) : kGrid;
}

}  // namespace

extern "C" {

int probe_sqrt_fast(uint32_t first, uint32_t n, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_sqrt_fast, dim3(grid_for(n)), dim3(kThreads), 0, s, first, n, out);
  return (int)hipGetLastError();
}

int probe_fused_vcode_diff(float scale, uint32_t* counters, hipStream_t s) {
  if (!(scale >= 0x1p-126f) || !(scale <= 3.4e38f)) return -1;   // a kept block scale: normal and finite
  hipLaunchKernelGGL(k_fused_vcode_diff, dim3(kGrid), dim3(kThreads), 0, s, scale, counters);
  return (int)hipGetLastError();
}

int probe_fused_vcode(float scale, const float* v, uint32_t* out, uint32_t n, hipStream_t s) {
  if (!(scale >= 0x1p-126f) || !(scale <= 3.4e38f)) return -1;
  hipLaunchKernelGGL(k_fused_vcode, dim3(grid_for(n)), dim3(kThreads), 0, s, scale, v, out, n);
  return (int)hipGetLastError();
}

}  // extern "C"
