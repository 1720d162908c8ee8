// ps_noalloc.hip - ps_factored_step_noalloc: the factored step for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The plan image and the workspace of the call live in `scratch`, a fixed
// array in each GPU's memory that the library holds for the life of the
// process. In host code `scratch` is only a host-side handle: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the launches receive. The plan image
// reaches the array through kernel arguments (k_fill_words), so the call
// makes no copy from host memory and allocates nothing. The kernels are the
// ones ps_factored_step launches.
#include <mutex>
#include <unordered_map>

#include "ps_internal.h"

namespace ps {
namespace {

static_assert(PS_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must be a multiple of 256 bytes");

static __device__ __align__(256) unsigned char scratch[PS_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::unordered_map<int, char*> g_scratch_ptr;   // device -> address of that device's scratch

// Device address of the current device's scratch (looked up on the first
// call on each device).
ps_status scratch_ptr(char** out) {
  int dev = 0;
  if (ps_status st = hip_check(hipGetDevice(&dev), "hipGetDevice")) return st;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return PS_OK;
  }
  void* p = nullptr;
  if (ps_status st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return st;
  if (!p || !is_aligned(p, 256)) return fail(PS_ERR_HIP, "scratch has no 256-byte aligned device address");
  g_scratch_ptr[dev] = (char*)p;
  *out = (char*)p;
  return PS_OK;
}

// Words carried per fill launch (just under 2 KiB of kernel arguments).
constexpr uint32_t kFillWords = 496;

struct FillArgs {
  uint32_t* dst;
  uint32_t n;
  uint32_t pad;
  uint32_t w[kFillWords];
};

__global__ __launch_bounds__(256) void k_fill_words(FillArgs a) {
  for (uint32_t i = threadIdx.x; i < a.n; i += 256) a.dst[i] = a.w[i];
}

// Copies `bytes` (a multiple of 4) from host memory to dst through the
// arguments of successive fill launches on s.
ps_status fill_from_args(char* dst, const unsigned char* src, size_t bytes, hipStream_t s) {
  FillArgs a;
  a.pad = 0;
  for (size_t off = 0; off < bytes; off += 4 * (size_t)kFillWords) {
    const size_t chunk = bytes - off < 4 * (size_t)kFillWords ? bytes - off : 4 * (size_t)kFillWords;
    a.dst = (uint32_t*)(dst + off);
    a.n = (uint32_t)(chunk / 4);
    memcpy(a.w, src + off, chunk);
    hipLaunchKernelGGL(k_fill_words, dim3(1), dim3(256), 0, s, a);
    if (ps_status st = hip_check(hipGetLastError(), "k_fill_words launch")) return st;
  }
  return PS_OK;
}

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace
}  // namespace ps

using namespace ps;

extern "C" ps_status ps_factored_step_noalloc(const ps_tensor* tensors, int32_t n_tensors,
                                              const ps_factored_hparams* hp, int64_t step, ps_stream_t stream) {
  thread_local FactoredCall c;
  // validation and sizes first: a rejected call makes no HIP call
  if (ps_status s = factored_prepare(tensors, n_tensors, hp, step, nullptr, c)) return s;
  if (c.empty) return PS_OK;
  const size_t head = up256(c.image.size());
  if (head + c.ws_bytes > (size_t)PS_NOALLOC_SCRATCH_BYTES)
    return fail(PS_ERR_WORKSPACE, "the call needs %zu bytes of scratch (plan %zu + workspace %zu); the library holds %zu",
                head + c.ws_bytes, head, c.ws_bytes, (size_t)PS_NOALLOC_SCRATCH_BYTES);
  char* base = nullptr;
  if (ps_status s = scratch_ptr(&base)) return s;
  if (ps_status s = factored_prepare(tensors, n_tensors, hp, step, base + head, c)) return s;
  if (c.image.size() % 4 != 0) return fail(PS_ERR_INVALID_ARG, "plan image of %zu bytes", c.image.size());
  hipStream_t s = (hipStream_t)stream;
  if (ps_status st = fill_from_args(base, c.image.data(), c.image.size(), s)) return st;
  factored_bind(c, base);
  return launch_factored(c.plan, c.sc, hp->split_mode, s);
}
