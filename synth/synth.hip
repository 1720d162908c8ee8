/* synth.hip - host and device fill routines for the seeded synthetic inputs
 * defined in synth.h. Both sides evaluate the same inline functions, so a
 * buffer filled on the device is bit-identical to one filled on the host.
 *
 * Element `start + j` of a stream is written to out[j], so any slice of a
 * tensor can be regenerated on its own.
 */
#include "synth.h"

#define SYN_OUTLIER_STREAM_OFFSET 0x100ull

extern "C" {

void syn_host_fill_bf16_normal(uint16_t* out, int64_t start, int64_t n, uint64_t seed, uint64_t stream,
                               uint64_t tensor, uint64_t step, double sigma, double outlier_p,
                               double outlier_scale) {
  uint64_t key = syn_key(seed, stream, tensor, step);
  uint64_t okey = syn_key(seed, stream + SYN_OUTLIER_STREAM_OFFSET, tensor, step);
  for (int64_t j = 0; j < n; ++j)
    out[j] = syn_bf16_normal(key, okey, (uint64_t)(start + j), sigma, outlier_p, outlier_scale);
}

void syn_host_fill_u16_uniform(uint16_t* out, int64_t start, int64_t n, uint64_t seed, uint64_t stream,
                               uint64_t tensor, uint64_t step) {
  uint64_t key = syn_key(seed, stream, tensor, step);
  for (int64_t j = 0; j < n; ++j) out[j] = syn_u16_uniform(key, (uint64_t)(start + j));
}

}  // extern "C"

__global__ void syn_k_bf16_normal(uint16_t* __restrict__ out, int64_t start, int64_t n, uint64_t key,
                                  uint64_t okey, double sigma, double outlier_p, double outlier_scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = syn_bf16_normal(key, okey, (uint64_t)(start + j), sigma, outlier_p, outlier_scale);
}

__global__ void syn_k_u16_uniform(uint16_t* __restrict__ out, int64_t start, int64_t n, uint64_t key) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = syn_u16_uniform(key, (uint64_t)(start + j));
}

static int syn_grid(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

extern "C" {

/* Device fills: `out` is device memory, launched on `stream_handle`
 * (a hipStream_t). Return 0 or the hipError_t of the launch. */
int syn_dev_fill_bf16_normal(uint16_t* out, int64_t start, int64_t n, uint64_t seed, uint64_t stream,
                             uint64_t tensor, uint64_t step, double sigma, double outlier_p,
                             double outlier_scale, void* stream_handle) {
  if (n <= 0) return 0;
  uint64_t key = syn_key(seed, stream, tensor, step);
  uint64_t okey = syn_key(seed, stream + SYN_OUTLIER_STREAM_OFFSET, tensor, step);
  hipLaunchKernelGGL(syn_k_bf16_normal, dim3(syn_grid(n)), dim3(256), 0, (hipStream_t)stream_handle, out,
                     start, n, key, okey, sigma, outlier_p, outlier_scale);
  return (int)hipGetLastError();
}

int syn_dev_fill_u16_uniform(uint16_t* out, int64_t start, int64_t n, uint64_t seed, uint64_t stream,
                             uint64_t tensor, uint64_t step, void* stream_handle) {
  if (n <= 0) return 0;
  uint64_t key = syn_key(seed, stream, tensor, step);
  hipLaunchKernelGGL(syn_k_u16_uniform, dim3(syn_grid(n)), dim3(256), 0, (hipStream_t)stream_handle, out,
                     start, n, key);
  return (int)hipGetLastError();
}

}  // extern "C"
