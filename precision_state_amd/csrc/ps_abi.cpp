// ps_abi.cpp - extern "C" entry points of libps.so: argument validation (all
// on the host, before any HIP call), the device tensor-table cache, and
// dispatch to the kernels.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ps_internal.h"

namespace ps {

namespace {
thread_local char g_err[512] = "";

bool finite(double x) { return std::isfinite(x); }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
}  // namespace

ps_status fail(ps_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

ps_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return PS_OK;
  return fail(PS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------

bool is_finite(double x) { return std::isfinite(x); }
bool is_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

namespace {

ps_status check_hparams(const ps_hparams* hp) {
  if (!hp) return fail(PS_ERR_INVALID_ARG, "hparams is NULL");
  if (hp->algo != PS_ALGO_ADAM && hp->algo != PS_ALGO_NADAM) return fail(PS_ERR_INVALID_ARG, "unknown algo %d", hp->algo);
  if (hp->split_mode != PS_SPLIT_TRUNC && hp->split_mode != PS_SPLIT_NEAREST_AWAY &&
      hp->split_mode != PS_SPLIT_STOCHASTIC)
    return fail(PS_ERR_INVALID_ARG, "unknown split_mode %d", hp->split_mode);
  if (!finite(hp->lr) || hp->lr < 0) return fail(PS_ERR_INVALID_ARG, "lr must be finite and >= 0");
  if (!finite(hp->beta1) || hp->beta1 < 0 || hp->beta1 >= 1) return fail(PS_ERR_INVALID_ARG, "beta1 must be in [0, 1)");
  if (!finite(hp->beta2) || hp->beta2 < 0 || hp->beta2 >= 1) return fail(PS_ERR_INVALID_ARG, "beta2 must be in [0, 1)");
  if (!finite(hp->eps) || !(hp->eps > 0) || !((float)hp->eps > 0.0f))
    return fail(PS_ERR_INVALID_ARG, "eps must be finite and > 0 once rounded to fp32");
  if (!finite(hp->weight_decay) || hp->weight_decay < 0)
    return fail(PS_ERR_INVALID_ARG, "weight_decay must be finite and >= 0");
  if (!finite(hp->momentum_decay) || hp->momentum_decay < 0)
    return fail(PS_ERR_INVALID_ARG, "momentum_decay must be finite and >= 0");
  return PS_OK;
}

constexpr int64_t kMaxNumel = int64_t(1) << 40;

ps_status check_array(const void* p, const char* what, int i, uintptr_t align) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "tensor %d: %s is NULL", i, what);
  if (!aligned(p, align)) return fail(PS_ERR_ALIGNMENT, "tensor %d: %s is not %d-byte aligned", i, what, (int)align);
  return PS_OK;
}

// Validates the records and builds the active lists (tensors with numel > 0
// and a gradient) with their work-item prefix ends: default formats in recs,
// tensors with storage flags in xrecs.
ps_status build_active(const ps_tensor* t, int32_t n, bool residual, std::vector<DevTensor>& recs,
                       std::vector<uint32_t>& ends, std::vector<DevTensorEx>& xrecs, std::vector<uint32_t>& xends) {
  if (n < 0) return fail(PS_ERR_INVALID_ARG, "n_tensors < 0");
  if (n > 0 && !t) return fail(PS_ERR_INVALID_ARG, "tensors is NULL");
  uint64_t items = 0, xitems = 0;
  const uint32_t known = PS_TENSOR_FP32_MOMENTS | PS_TENSOR_FP32_PARAM | PS_TENSOR_F24_MOMENTS;
  for (int32_t i = 0; i < n; ++i) {
    const ps_tensor& x = t[i];
    if (x.numel < 0 || x.numel > kMaxNumel) return fail(PS_ERR_SHAPE, "tensor %d: numel %lld out of range", i, (long long)x.numel);
    if ((x.flags & ~known) || x.reserved) return fail(PS_ERR_INVALID_ARG, "tensor %d: unknown flags", i);
    if ((x.flags & PS_TENSOR_FP32_MOMENTS) && (x.flags & PS_TENSOR_F24_MOMENTS))
      return fail(PS_ERR_INVALID_ARG, "tensor %d: FP32_MOMENTS and F24_MOMENTS are exclusive", i);
    if (x.numel == 0 || x.grad == nullptr) continue;
    const bool no_scales = x.flags & (PS_TENSOR_FP32_MOMENTS | PS_TENSOR_F24_MOMENTS);
    const bool fpp = x.flags & PS_TENSOR_FP32_PARAM;
    ps_status s;
    if ((s = check_array(x.w_hi, "w_hi", i, 16)) || (s = check_array(x.grad, "grad", i, 16)) ||
        (s = check_array(x.m_code, "m_code", i, 16)) || (s = check_array(x.v_code, "v_code", i, 16)))
      return s;
    if (!fpp && residual && (s = check_array(x.w_lo, "w_lo", i, 16))) return s;
    if (!no_scales && ((s = check_array(x.m_scale, "m_scale", i, 4)) || (s = check_array(x.v_scale, "v_scale", i, 4))))
      return s;
    const uint64_t nit = (uint64_t)((x.numel + kStepItemElems - 1) / kStepItemElems);
    if (x.flags) {
      xitems += nit;
      if (xitems > 0x7FFFFFFFull) return fail(PS_ERR_SHAPE, "tensor list too large (more than 2^31 - 1 work items)");
      xrecs.push_back(DevTensorEx{x.w_hi, x.w_lo, x.grad, x.m_code, x.m_scale, x.v_code, x.v_scale, x.numel, x.flags,
                                  (uint32_t)i});
      xends.push_back((uint32_t)xitems);
    } else {
      items += nit;
      if (items > 0x7FFFFFFFull) return fail(PS_ERR_SHAPE, "tensor list too large (more than 2^31 - 1 work items)");
      recs.push_back(DevTensor{x.w_hi, x.w_lo, x.grad, x.m_code, x.m_scale, x.v_code, x.v_scale, x.numel, (uint32_t)i, 0});
      ends.push_back((uint32_t)items);
    }
  }
  return PS_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// device blob cache (blob_cache.h): HIP backend
// ---------------------------------------------------------------------------

int HipBlobBackend::alloc_chunk(size_t bytes, char** d, char** h) {
  if (hipMalloc((void**)d, bytes) != hipSuccess) return fail(PS_ERR_NO_MEMORY, "device table allocation failed");
  if (hipHostMalloc((void**)h, bytes, hipHostMallocDefault) != hipSuccess) {
    (void)hipFree(*d);
    return fail(PS_ERR_NO_MEMORY, "pinned table staging allocation failed");
  }
  return PS_OK;
}

void HipBlobBackend::free_chunk(char* d, char* h) {
  if (d) (void)hipFree(d);
  if (h) (void)hipHostFree(h);
}

int HipBlobBackend::create_event(hipEvent_t* e) {
  return hip_check(hipEventCreateWithFlags(e, hipEventDisableTiming), "hipEventCreate");
}

void HipBlobBackend::destroy_event(hipEvent_t e) {
  if (e) (void)hipEventDestroy(e);
}

int HipBlobBackend::upload(char* d, const char* h, size_t bytes, hipStream_t s, hipEvent_t e) {
  if (ps_status st = hip_check(hipMemcpyAsync(d, h, bytes, hipMemcpyHostToDevice, s), "table upload")) return st;
  return hip_check(hipEventRecord(e, s), "hipEventRecord");
}

bool HipBlobBackend::event_done(hipEvent_t e) { return hipEventQuery(e) == hipSuccess; }

int HipBlobBackend::stream_wait(hipStream_t s, hipEvent_t e) {
  return hip_check(hipStreamWaitEvent(s, e, 0), "hipStreamWaitEvent");
}

int HipBlobBackend::device_sync() { return hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize"); }

void HipBlobBackend::sync_stream(hipStream_t s) { (void)hipStreamSynchronize(s); }

// Up to 16384 blobs or 64 MiB of arena per device, grown 1 MiB at a time.
// The cache lives until the process ends.
TableCache& table_cache() {
  static HipBlobBackend* backend = new HipBlobBackend;
  static TableCache* cache = new TableCache(*backend, BlobLimits{16384, size_t(64) << 20, size_t(1) << 20});
  return *cache;
}

ps_status device_blob(const void* data, size_t bytes, hipStream_t s, const void** dptr, TableLease& lease) {
  int dev = 0;
  if (ps_status st = hip_check(hipGetDevice(&dev), "hipGetDevice")) return st;
  return table_cache().get(dev, data, bytes, s, dptr, lease);
}

namespace {

ps_status get_table(const std::vector<DevTensor>& recs, const std::vector<uint32_t>& ends, hipStream_t s,
                    TablePtr* out, TableLease& lease) {
  const size_t rb = recs.size() * sizeof(DevTensor), eb = ends.size() * sizeof(uint32_t);
  std::vector<unsigned char> blob(rb + eb);
  memcpy(blob.data(), recs.data(), rb);
  memcpy(blob.data() + rb, ends.data(), eb);
  const void* d = nullptr;
  if (ps_status st = device_blob(blob.data(), blob.size(), s, &d, lease)) return st;
  *out = TablePtr{(const DevTensor*)d, (const uint32_t*)((const char*)d + rb), (int32_t)recs.size()};
  return PS_OK;
}

ps_status check_elementwise(int64_t n, std::initializer_list<std::pair<const void*, const char*>> arrays,
                            std::initializer_list<std::pair<const void*, const char*>> scales) {
  if (n < 0 || n > kMaxNumel) return fail(PS_ERR_SHAPE, "n = %lld out of range", (long long)n);
  if (n == 0) return PS_OK;
  for (auto& a : arrays) {
    if (!a.first) return fail(PS_ERR_INVALID_ARG, "%s is NULL", a.second);
    if (!aligned(a.first, 16)) return fail(PS_ERR_ALIGNMENT, "%s is not 16-byte aligned", a.second);
  }
  for (auto& a : scales) {
    if (!a.first) return fail(PS_ERR_INVALID_ARG, "%s is NULL", a.second);
    if (!aligned(a.first, 4)) return fail(PS_ERR_ALIGNMENT, "%s is not 4-byte aligned", a.second);
  }
  return PS_OK;
}

}  // namespace
}  // namespace ps

using namespace ps;

extern "C" {

ps_status ps_step_scalars(const ps_hparams* hp, int64_t step, float out[10]) {
  g_err[0] = 0;
  if (ps_status s = check_hparams(hp)) return s;
  if (step < 1) return fail(PS_ERR_INVALID_ARG, "step must be >= 1 (got %lld)", (long long)step);
  if (!out) return fail(PS_ERR_INVALID_ARG, "out is NULL");
  StepScalars c;
  step_scalars(*hp, step, &c);
  const float v[10] = {c.B1, c.C1, c.B2, c.C2, c.EPS, c.A, c.RS2, c.AG, c.AM, c.CWD};
  memcpy(out, v, sizeof(v));
  return PS_OK;
}

ps_status ps_opt_step_multi(const ps_tensor* tensors, int32_t n_tensors, const ps_hparams* hp, int64_t step,
                            ps_stream_t stream) {
  g_err[0] = 0;
  if (ps_status s = check_hparams(hp)) return s;
  if (step < 1) return fail(PS_ERR_INVALID_ARG, "step must be >= 1 (got %lld)", (long long)step);
  // Per-thread buffers and the last step's scalars are kept between calls:
  // a caller that steps tensor by tensor (one call per gradient hook) makes
  // many calls with the same hyperparameters and step.
  thread_local std::vector<DevTensor> recs;
  thread_local std::vector<uint32_t> ends;
  thread_local std::vector<DevTensorEx> xrecs;
  thread_local std::vector<uint32_t> xends;
  recs.clear();
  ends.clear();
  xrecs.clear();
  xends.clear();
  if (ps_status s = build_active(tensors, n_tensors, hp->split_mode != PS_SPLIT_STOCHASTIC, recs, ends, xrecs, xends))
    return s;
  if (recs.empty() && xrecs.empty()) return PS_OK;
  thread_local ps_hparams last_hp;
  thread_local int64_t last_step = 0;
  thread_local StepScalars c;
  if (last_step != step || memcmp(&last_hp, hp, sizeof(ps_hparams)) != 0) {
    step_scalars(*hp, step, &c);
    last_hp = *hp;
    last_step = step;
  }
  hipStream_t s = (hipStream_t)stream;
  if (!xrecs.empty()) {
    TableLease lease(table_cache());   // held until the launch that reads the table is enqueued
    const size_t rb = xrecs.size() * sizeof(DevTensorEx), eb = xends.size() * sizeof(uint32_t);
    std::vector<unsigned char> blob(rb + eb);
    memcpy(blob.data(), xrecs.data(), rb);
    memcpy(blob.data() + rb, xends.data(), eb);
    const void* d = nullptr;
    if (ps_status st = device_blob(blob.data(), blob.size(), s, &d, lease)) return st;
    TableExPtr tx{(const DevTensorEx*)d, (const uint32_t*)((const char*)d + rb), (int32_t)xrecs.size()};
    if (ps_status st = launch_adam_ex(tx, xends.back(), *hp, c, s)) return st;
  }
  if (recs.empty()) return PS_OK;
  const uint32_t total = ends.back();
  if (recs.size() == 1) {   // one call per gradient hook: the smallest argument block
    TableOne t1;
    t1.recs[0] = recs[0];
    t1.item_end[0] = ends[0];
    t1.n = 1;
    return launch_adam_one(t1, total, *hp, c, s);
  }
  if (recs.size() <= (size_t)kInlineMax) {
    TableInline tb;
    memset(&tb, 0, sizeof(tb));
    for (size_t i = 0; i < recs.size(); ++i) {
      tb.recs[i] = recs[i];
      tb.item_end[i] = ends[i];
    }
    tb.n = (int32_t)recs.size();
    return launch_adam_inline(tb, total, *hp, c, s);
  }
  TableLease lease(table_cache());     // held until the launch is enqueued
  TablePtr tp;
  if (ps_status st = get_table(recs, ends, s, &tp, lease)) return st;
  return launch_adam_ptr(tp, total, *hp, c, s);
}

ps_status ps_split(const float* w32, uint16_t* hi, uint16_t* lo, int64_t n, int32_t mode, ps_stream_t stream) {
  g_err[0] = 0;
  if (mode == PS_SPLIT_STOCHASTIC) return fail(PS_ERR_UNSUPPORTED, "ps_split: stochastic rounding needs a step and seed");
  if (mode != PS_SPLIT_TRUNC && mode != PS_SPLIT_NEAREST_AWAY) return fail(PS_ERR_INVALID_ARG, "unknown split mode %d", mode);
  if (ps_status s = check_elementwise(n, {{w32, "w32"}, {hi, "hi"}, {lo, "lo"}}, {})) return s;
  if (n == 0) return PS_OK;
  return launch_split(w32, hi, lo, n, mode, (hipStream_t)stream);
}

ps_status ps_join(const uint16_t* hi, const uint16_t* lo, float* w32, int64_t n, int32_t mode, ps_stream_t stream) {
  g_err[0] = 0;
  if (mode == PS_SPLIT_STOCHASTIC) return fail(PS_ERR_UNSUPPORTED, "ps_join: stochastic rounding keeps no residual");
  if (mode != PS_SPLIT_TRUNC && mode != PS_SPLIT_NEAREST_AWAY) return fail(PS_ERR_INVALID_ARG, "unknown split mode %d", mode);
  if (ps_status s = check_elementwise(n, {{w32, "w32"}, {hi, "hi"}, {lo, "lo"}}, {})) return s;
  if (n == 0) return PS_OK;
  return launch_join(hi, lo, w32, n, mode, (hipStream_t)stream);
}

ps_status ps_encode_moments(const float* x, uint16_t* code, float* scale, int64_t n, int32_t kind,
                            ps_stream_t stream) {
  g_err[0] = 0;
  if (kind != PS_MOMENT_SIGNED && kind != PS_MOMENT_UNSIGNED) return fail(PS_ERR_INVALID_ARG, "unknown moment kind %d", kind);
  if (ps_status s = check_elementwise(n, {{x, "x"}, {code, "code"}}, {{scale, "scale"}})) return s;
  if (n == 0) return PS_OK;
  return launch_encode(x, code, scale, n, kind, (hipStream_t)stream);
}

ps_status ps_decode_moments(const uint16_t* code, const float* scale, float* x, int64_t n, int32_t kind,
                            ps_stream_t stream) {
  g_err[0] = 0;
  if (kind != PS_MOMENT_SIGNED && kind != PS_MOMENT_UNSIGNED) return fail(PS_ERR_INVALID_ARG, "unknown moment kind %d", kind);
  if (ps_status s = check_elementwise(n, {{x, "x"}, {code, "code"}}, {{scale, "scale"}})) return s;
  if (n == 0) return PS_OK;
  return launch_decode(code, scale, x, n, kind, (hipStream_t)stream);
}

const char* ps_status_string(ps_status s) {
  switch (s) {
    case PS_OK: return "ok";
    case PS_ERR_INVALID_ARG: return "invalid argument";
    case PS_ERR_ALIGNMENT: return "misaligned pointer";
    case PS_ERR_SHAPE: return "bad shape";
    case PS_ERR_UNSUPPORTED: return "unsupported";
    case PS_ERR_HIP: return "HIP runtime error";
    case PS_ERR_NO_MEMORY: return "out of memory";
    case PS_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* ps_last_error(void) { return g_err; }

const char* ps_version(void) { return "precision_state_amd 0.1 (gfx950)"; }

}  // extern "C"
