// ps_offload.cpp - host-offload pipeline for the fused (N)AdamW step [NADAM,
// opening post: the moments (and here the Kahan residuals) stay in host memory
// and cross PCIe every step; KAHAN: only the 16 residual bits travel; with
// stochastic rounding, the pages' setting when host memory is short, no
// residual exists and only the moments travel].
//
// Two modes (ps_offload_options.mode):
//
// DIRECT (the default): the resident step kernel reads and writes the
// host-resident residuals, codes and scales in place, over PCIe, through the
// device addresses of the pinned allocations: no staging buffers and no copy
// engines. The kernel is bound by the link (reads from the host and writes to
// it travel in the two directions at once) and needs few waves in flight, so
// it runs on a stream restricted to n_cus compute units (8 by default),
// which leaves the rest of the GPU to other work. Measured over the FLUX
// double block x 57: 45-48 GB/s each way on 8 to 64 CUs, against 48.7 GB/s
// each way for DMA copies in both directions at once.
//
// STAGED: kSlots (2) device staging slots hold one group's residuals, codes and
// scales each. Group k uses slot s = k % 2:
//   upload stream:   wait(download of k-2 done) -> copies host->slot -> event in[s]
//   compute stream:  wait(in[s]) -> fused step of group k -> event done[s]
//   download stream: wait(done[s]) -> copies slot->host -> event out[s]
// so the upload of k+1 and the download of k-1 overlap the step of k, and the
// two copy directions run concurrently on hardware queues of their own (a third slot measured no faster: the
// pipeline already moves data at the link's duplex rate). The step kernel is the resident one,
// reading the slot through a per-(group, slot) device table, so results are
// bit-identical to ps_opt_step_multi on device-resident state.
#include <cstring>
#include <vector>

#include "ps_internal.h"

constexpr int kSlots = 2;   // device staging slots (group k uses slot k % kSlots)

struct ps_offload_plan {
  int device = -1;
  struct Copy {
    void* host;
    size_t dev_off;
    size_t bytes;
  };
  struct Group {
    std::vector<Copy> copies;          // codes and scales, same list for both directions
    std::vector<Copy> lo_copies;       // residuals (skipped under stochastic rounding)
    size_t table_off[kSlots] = {};     // device table of this group for each slot
    int32_t n_active = 0;
    uint32_t total_items = 0;
  };
  std::vector<Group> groups;
  size_t slot_bytes = 0;
  char* slots[kSlots] = {};
  char* tables = nullptr;
  hipStream_t up = nullptr, down = nullptr, comp = nullptr;   // DIRECT: comp only (CU-restricted)
  bool own_queues = false;             // the plan's streams each have a hardware queue of their own
  int32_t mode = PS_OFFLOAD_DIRECT;
  hipEvent_t in_ev[kSlots] = {}, done_ev[kSlots] = {}, out_ev[kSlots] = {};
  hipEvent_t start_ev = nullptr, end_ev = nullptr;
  uint64_t bytes_per_dir = 0;          // residual modes
  uint64_t lo_bytes_per_dir = 0;       // of which residuals
  uint64_t last_bytes_per_dir = 0;     // the most recent run
  bool has_residual = true;            // every active tensor has w_lo
  bool out_recorded[kSlots] = {};     // out_ev[s] has been recorded by some run
};

namespace ps {
namespace {

constexpr size_t kAlignBytes = 256;
size_t up256(size_t x) { return (x + kAlignBytes - 1) / kAlignBytes * kAlignBytes; }

void destroy(ps_offload_plan* p) {
  if (!p) return;
  if (p->device >= 0) (void)hipDeviceSynchronize();
  for (int s = 0; s < kSlots; ++s) {
    if (p->slots[s]) (void)hipFree(p->slots[s]);
    if (p->in_ev[s]) (void)hipEventDestroy(p->in_ev[s]);
    if (p->done_ev[s]) (void)hipEventDestroy(p->done_ev[s]);
    if (p->out_ev[s]) (void)hipEventDestroy(p->out_ev[s]);
  }
  if (p->start_ev) (void)hipEventDestroy(p->start_ev);
  if (p->end_ev) (void)hipEventDestroy(p->end_ev);
  if (p->tables) (void)hipFree(p->tables);
  if (p->up) (void)hipStreamDestroy(p->up);
  if (p->down) (void)hipStreamDestroy(p->down);
  if (p->comp) (void)hipStreamDestroy(p->comp);
  delete p;
}

ps_status check_host(const void* p, const char* what, int g, int i, uintptr_t align) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "group %d tensor %d: %s is NULL", g, i, what);
  if (!is_aligned(p, align)) return fail(PS_ERR_ALIGNMENT, "group %d tensor %d: %s misaligned", g, i, what);
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeHost) {
    (void)hipGetLastError();   // the query's failure must not surface at a later launch check
    return fail(PS_ERR_INVALID_ARG, "group %d tensor %d: %s is not pinned host memory", g, i, what);
  }
  return PS_OK;
}

void add_copy(std::vector<ps_offload_plan::Copy>& cl, void* host, size_t dev_off, size_t bytes, uint64_t& total) {
  if (!cl.empty() && (char*)cl.back().host + cl.back().bytes == (char*)host && cl.back().dev_off + cl.back().bytes == dev_off)
    cl.back().bytes += bytes;
  else
    cl.push_back({host, dev_off, bytes});
  total += bytes;
}

// A copy stream with a hardware queue of its own. HIP maps streams onto a
// small pool of hardware queues (GPU_MAX_HW_QUEUES, 4 by default, shared by
// every stream of the process, torch's stream pool included), and streams
// that share a queue run in one order: the uploads of group k+1 then wait for
// the downloads of group k and the pipeline moves one direction at a time
// (measured on one box: 27.9 GB/s each way, against 47.8 GB/s each way with
// the two directions on queues of their own). A stream created with a CU mask
// always gets a new queue; the mask here enables every CU. Such a stream is
// blocking (it orders itself with the null stream), so the plan launches its
// kernels on a stream of its own, not on the caller's. Falls back to a plain
// non-blocking stream if the CU-mask stream cannot be made.
// n_cus > 0 enables only the first n_cus CUs (the DIRECT mode's kernel stream).
ps_status create_copy_stream(hipStream_t* s, bool* own_queue, int n_cus = 0) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
    const int on = (n_cus > 0 && n_cus < cus) ? n_cus : cus;
    std::vector<uint32_t> mask((size_t)(cus + 31) / 32, 0u);
    for (int c = 0; c < on; ++c) mask[(size_t)c / 32] |= 1u << (c % 32);
    if (hipExtStreamCreateWithCUMask(s, (uint32_t)mask.size(), mask.data()) == hipSuccess) {
      *own_queue = true;
      return PS_OK;
    }
    (void)hipGetLastError();
  }
  *own_queue = false;
  return hip_check(hipStreamCreateWithFlags(s, hipStreamNonBlocking), "hipStreamCreate");
}

// Device address of pinned host memory (DIRECT mode).
ps_status dev_of_host(void* host, const char* what, int g, int i, void** dev) {
  *dev = nullptr;
  if (!host) return PS_OK;
  if (hipHostGetDevicePointer(dev, host, 0) != hipSuccess || !*dev) {
    (void)hipGetLastError();
    return fail(PS_ERR_INVALID_ARG, "group %d tensor %d: %s has no device address", g, i, what);
  }
  return PS_OK;
}

ps_status check_dev(const void* p, const char* what, int g, int i) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "group %d tensor %d: %s is NULL", g, i, what);
  if (!is_aligned(p, 16)) return fail(PS_ERR_ALIGNMENT, "group %d tensor %d: %s is not 16-byte aligned", g, i, what);
  return PS_OK;
}

}  // namespace
}  // namespace ps

using namespace ps;

extern "C" {

ps_status ps_offload_plan_create(const ps_offload_group* groups, int32_t n_groups, ps_offload_plan** plan) {
  return ps_offload_plan_create_ex(groups, n_groups, nullptr, plan);
}

ps_status ps_offload_plan_create_ex(const ps_offload_group* groups, int32_t n_groups, const ps_offload_options* opt,
                                    ps_offload_plan** plan) {
  if (!plan) return fail(PS_ERR_INVALID_ARG, "plan is NULL");
  *plan = nullptr;
  if (n_groups < 0 || (n_groups > 0 && !groups)) return fail(PS_ERR_INVALID_ARG, "bad group list");
  const ps_offload_options o = opt ? *opt : ps_offload_options{PS_OFFLOAD_DIRECT, PS_OFFLOAD_DEFAULT_CUS, 0, 0};
  if (o.mode != PS_OFFLOAD_DIRECT && o.mode != PS_OFFLOAD_STAGED)
    return fail(PS_ERR_INVALID_ARG, "unknown offload mode %d", o.mode);
  if (o.n_cus < 0 || o.reserved0 || o.reserved1) return fail(PS_ERR_INVALID_ARG, "bad offload options");
  const bool direct = o.mode == PS_OFFLOAD_DIRECT;
  ps_offload_plan* p = new ps_offload_plan;
  p->mode = o.mode;
  if (ps_status st = hip_check(hipGetDevice(&p->device), "hipGetDevice")) {
    delete p;
    return st;
  }
  // Lay out each group's staging slot (lo | m codes | v codes | m scales |
  // v scales, tensors in order, 256-byte aligned) and its copy list.
  std::vector<std::vector<DevTensor>> recs(n_groups);
  std::vector<std::vector<uint32_t>> ends(n_groups);
  uint32_t tid_base = 0;   // stochastic-rounding key: position in the concatenated group lists
  p->groups.resize(n_groups);
  for (int32_t g = 0; g < n_groups; ++g) {
    const ps_offload_group& G = groups[g];
    if (G.n_tensors < 0 || (G.n_tensors > 0 && !G.tensors)) {
      destroy(p);
      return fail(PS_ERR_INVALID_ARG, "group %d: bad tensor list", g);
    }
    struct Part { const ps_tensor* t; size_t lo, mc, vc, ms, vs; uint32_t tid; };
    std::vector<Part> parts;
    size_t off_lo = 0, n16 = 0, nsc = 0;
    for (int32_t i = 0; i < G.n_tensors; ++i) {
      const ps_tensor& x = G.tensors[i];
      if (x.numel < 0 || x.numel > (int64_t(1) << 40)) {
        destroy(p);
        return fail(PS_ERR_SHAPE, "group %d tensor %d: numel out of range", g, i);
      }
      if (x.flags || x.reserved) {
        destroy(p);
        return fail(PS_ERR_UNSUPPORTED, "group %d tensor %d: storage flags are not supported here", g, i);
      }
      if (x.numel == 0 || !x.grad) continue;
      ps_status st;
      if (!x.w_lo) p->has_residual = false;   // the plan then runs stochastic rounding only
      if ((st = check_dev(x.w_hi, "w_hi", g, i)) || (st = check_dev(x.grad, "grad", g, i)) ||
          (x.w_lo && (st = check_host(x.w_lo, "w_lo", g, i, 16))) || (st = check_host(x.m_code, "m_code", g, i, 16)) ||
          (st = check_host(x.v_code, "v_code", g, i, 16)) || (st = check_host(x.m_scale, "m_scale", g, i, 4)) ||
          (st = check_host(x.v_scale, "v_scale", g, i, 4))) {
        destroy(p);
        return st;
      }
      parts.push_back(Part{&x, 0, 0, 0, 0, 0, tid_base + (uint32_t)i});
      n16 += up256((size_t)x.numel * 2);
      nsc += up256((size_t)((x.numel + kBlock - 1) / kBlock) * 4);
    }
    // region bases within the slot
    const size_t base_mc = n16, base_vc = 2 * n16, base_ms = 3 * n16, base_vs = 3 * n16 + nsc;
    size_t o16 = 0, osc = 0;
    uint64_t items = 0;
    for (Part& q : parts) {
      const ps_tensor& x = *q.t;
      const size_t b16 = (size_t)x.numel * 2, bsc = (size_t)((x.numel + kBlock - 1) / kBlock) * 4;
      q.lo = off_lo + o16;
      q.mc = base_mc + o16;
      q.vc = base_vc + o16;
      q.ms = base_ms + osc;
      q.vs = base_vs + osc;
      o16 += up256(b16);
      osc += up256(bsc);
      items += (uint64_t)((x.numel + kStepItemElems - 1) / kStepItemElems);
      if (items > 0x7FFFFFFFull) {
        destroy(p);
        return fail(PS_ERR_SHAPE, "group %d too large", g);
      }
      ends[g].push_back((uint32_t)items);
      if (direct) {   // the kernel works on the host arrays in place
        void *lo = nullptr, *mc = nullptr, *vc = nullptr, *ms = nullptr, *vs = nullptr;
        ps_status st;
        if ((st = dev_of_host(x.w_lo, "w_lo", g, (int)(q.tid - tid_base), &lo)) ||
            (st = dev_of_host(x.m_code, "m_code", g, (int)(q.tid - tid_base), &mc)) ||
            (st = dev_of_host(x.v_code, "v_code", g, (int)(q.tid - tid_base), &vc)) ||
            (st = dev_of_host(x.m_scale, "m_scale", g, (int)(q.tid - tid_base), &ms)) ||
            (st = dev_of_host(x.v_scale, "v_scale", g, (int)(q.tid - tid_base), &vs))) {
          destroy(p);
          return st;
        }
        recs[g].push_back(DevTensor{x.w_hi, (uint16_t*)lo, x.grad, (uint16_t*)mc, (float*)ms, (uint16_t*)vc,
                                    (float*)vs, x.numel, q.tid, 0});
      } else {
        // records are completed with the slot base at upload time (below)
        recs[g].push_back(DevTensor{x.w_hi, (uint16_t*)q.lo, x.grad, (uint16_t*)q.mc, (float*)q.ms, (uint16_t*)q.vc,
                                    (float*)q.vs, x.numel, q.tid, 0});
      }
    }
    // copies region by region, tensors in order, so that contiguous host
    // slabs merge into one copy per region
    for (int region = 0; region < 5; ++region)
      for (const Part& q : parts) {
        const ps_tensor& x = *q.t;
        const size_t b16 = (size_t)x.numel * 2, bsc = (size_t)((x.numel + kBlock - 1) / kBlock) * 4;
        void* const host[5] = {x.w_lo, x.m_code, x.v_code, x.m_scale, x.v_scale};
        const size_t off[5] = {q.lo, q.mc, q.vc, q.ms, q.vs};
        if (region == 0) {
          if (x.w_lo) add_copy(p->groups[g].lo_copies, host[0], off[0], b16, p->lo_bytes_per_dir);
        } else {
          add_copy(p->groups[g].copies, host[region], off[region], region <= 2 ? b16 : bsc, p->bytes_per_dir);
        }
      }
    tid_base += (uint32_t)G.n_tensors;
    p->groups[g].n_active = (int32_t)parts.size();
    p->groups[g].total_items = (uint32_t)items;
    const size_t slot = 3 * n16 + 2 * nsc;
    if (slot > p->slot_bytes) p->slot_bytes = slot;
  }
  // device tables: per group and slot (DIRECT: per group), DevTensor[n] then item ends[n]
  const int n_tab = direct ? 1 : kSlots;
  std::vector<unsigned char> tab;
  for (int32_t g = 0; g < n_groups; ++g)
    for (int s = 0; s < n_tab; ++s) {
      p->groups[g].table_off[s] = tab.size();
      const size_t n = recs[g].size();
      tab.resize(tab.size() + up256(n * sizeof(DevTensor)) + up256(n * sizeof(uint32_t)));
    }
  ps_status st = PS_OK;
  for (int s = 0; s < (direct ? 0 : kSlots) && !st; ++s)
    if (hipMalloc((void**)&p->slots[s], p->slot_bytes ? p->slot_bytes : 256) != hipSuccess)
      st = fail(PS_ERR_NO_MEMORY, "offload staging slot allocation failed (%zu bytes)", p->slot_bytes);
  if (!st && hipMalloc((void**)&p->tables, tab.empty() ? 256 : tab.size()) != hipSuccess)
    st = fail(PS_ERR_NO_MEMORY, "offload table allocation failed");
  if (st) {
    destroy(p);
    return st;
  }
  for (int32_t g = 0; g < n_groups; ++g)
    for (int s = 0; s < n_tab; ++s) {
      const size_t n = recs[g].size();
      DevTensor* dst = (DevTensor*)(tab.data() + p->groups[g].table_off[s]);
      for (size_t i = 0; i < n; ++i) {
        DevTensor r = recs[g][i];
        if (!direct) {
          char* base = p->slots[s];
          r.lo = (uint16_t*)(base + (size_t)r.lo);
          r.mc = (uint16_t*)(base + (size_t)r.mc);
          r.vc = (uint16_t*)(base + (size_t)r.vc);
          r.ms = (float*)(base + (size_t)r.ms);
          r.vs = (float*)(base + (size_t)r.vs);
        }
        dst[i] = r;
      }
      if (n) memcpy(tab.data() + p->groups[g].table_off[s] + up256(n * sizeof(DevTensor)), ends[g].data(),
                    n * sizeof(uint32_t));
    }
  p->bytes_per_dir += p->lo_bytes_per_dir;
  p->last_bytes_per_dir = p->bytes_per_dir;
  if (!tab.empty()) st = hip_check(hipMemcpy(p->tables, tab.data(), tab.size(), hipMemcpyHostToDevice), "table upload");
  if (direct) {
    if (!st) st = create_copy_stream(&p->comp, &p->own_queues, o.n_cus);
  } else {
    bool q_up = false, q_down = false;
    if (!st) st = create_copy_stream(&p->up, &q_up);
    if (!st) st = create_copy_stream(&p->down, &q_down);
    if (!st) st = hip_check(hipStreamCreateWithFlags(&p->comp, hipStreamNonBlocking), "hipStreamCreate");
    p->own_queues = q_up && q_down;
  }
  for (int s = 0; s < (direct ? 0 : kSlots) && !st; ++s) {
    st = hip_check(hipEventCreateWithFlags(&p->in_ev[s], hipEventDisableTiming), "hipEventCreate");
    if (!st) st = hip_check(hipEventCreateWithFlags(&p->done_ev[s], hipEventDisableTiming), "hipEventCreate");
    if (!st) st = hip_check(hipEventCreateWithFlags(&p->out_ev[s], hipEventDisableTiming), "hipEventCreate");
  }
  if (!st) st = hip_check(hipEventCreateWithFlags(&p->start_ev, hipEventDisableTiming), "hipEventCreate");
  if (!st) st = hip_check(hipEventCreateWithFlags(&p->end_ev, hipEventDisableTiming), "hipEventCreate");
  if (st) {
    destroy(p);
    return st;
  }
  *plan = p;
  return PS_OK;
}

ps_status ps_offload_run(ps_offload_plan* p, const ps_hparams* hp, int64_t step, ps_stream_t stream) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "plan is NULL");
  if (!hp) return fail(PS_ERR_INVALID_ARG, "hparams is NULL");
  const ps_hparams h = *hp;
  const bool sr = h.split_mode == PS_SPLIT_STOCHASTIC;
  if (!sr && !p->has_residual)
    return fail(PS_ERR_INVALID_ARG, "the plan has tensors without w_lo; only stochastic rounding can run it");
  float scratch_out[10];
  // the resident path's validation of the hyperparameters and the step
  if (ps_status s = ps_step_scalars(&h, step, scratch_out)) return s;
  StepScalars c;
  step_scalars(h, step, &c);
  hipStream_t caller = (hipStream_t)stream, cs = p->comp;
  if (p->mode == PS_OFFLOAD_DIRECT) {
    // one launch per group on the plan's CU-restricted stream, after the
    // caller's work so far; the caller's stream then waits for the last one
    ps_status st = hip_check(hipEventRecord(p->start_ev, caller), "hipEventRecord");
    if (!st) st = hip_check(hipStreamWaitEvent(cs, p->start_ev, 0), "hipStreamWaitEvent");
    for (size_t k = 0; k < p->groups.size() && !st; ++k) {
      const auto& grp = p->groups[k];
      if (grp.n_active == 0) continue;
      const char* t = p->tables + grp.table_off[0];
      TablePtr tp{(const DevTensor*)t, (const uint32_t*)(t + up256(grp.n_active * sizeof(DevTensor))), grp.n_active};
      st = launch_adam_ptr(tp, grp.total_items, h, c, cs);
    }
    if (!st) st = hip_check(hipEventRecord(p->end_ev, cs), "hipEventRecord");
    if (!st) st = hip_check(hipStreamWaitEvent(caller, p->end_ev, 0), "hipStreamWaitEvent");
    if (!st) p->last_bytes_per_dir = sr ? p->bytes_per_dir - p->lo_bytes_per_dir : p->bytes_per_dir;
    return st;
  }
  // STAGED: the plan's streams start after the caller's work so far; the step
  // kernels run on the plan's own compute stream
  ps_status st = hip_check(hipEventRecord(p->start_ev, caller), "hipEventRecord");
  if (!st) st = hip_check(hipStreamWaitEvent(p->up, p->start_ev, 0), "hipStreamWaitEvent");
  if (!st) st = hip_check(hipStreamWaitEvent(p->down, p->start_ev, 0), "hipStreamWaitEvent");
  if (!st) st = hip_check(hipStreamWaitEvent(cs, p->start_ev, 0), "hipStreamWaitEvent");
  const int G = (int)p->groups.size();
  for (int k = 0; k < G && !st; ++k) {
    const auto& grp = p->groups[k];
    const int s = k % kSlots;
    // the slot is free once its previous download (this run's group k-2, or
    // an earlier run's last group on it, whatever stream that run was given)
    // has landed
    if (p->out_recorded[s]) st = hip_check(hipStreamWaitEvent(p->up, p->out_ev[s], 0), "hipStreamWaitEvent");
    for (int list = sr ? 1 : 0; list < 2; ++list)
      for (const auto& cp : list ? grp.copies : grp.lo_copies) {
        if (st) break;
        st = hip_check(hipMemcpyAsync(p->slots[s] + cp.dev_off, cp.host, cp.bytes, hipMemcpyHostToDevice, p->up),
                       "offload upload");
      }
    if (!st) st = hip_check(hipEventRecord(p->in_ev[s], p->up), "hipEventRecord");
    if (!st) st = hip_check(hipStreamWaitEvent(cs, p->in_ev[s], 0), "hipStreamWaitEvent");
    if (!st && grp.n_active > 0) {
      const char* t = p->tables + grp.table_off[s];
      TablePtr tp{(const DevTensor*)t, (const uint32_t*)(t + up256(grp.n_active * sizeof(DevTensor))), grp.n_active};
      st = launch_adam_ptr(tp, grp.total_items, h, c, cs);
    }
    if (!st) st = hip_check(hipEventRecord(p->done_ev[s], cs), "hipEventRecord");
    if (!st) st = hip_check(hipStreamWaitEvent(p->down, p->done_ev[s], 0), "hipStreamWaitEvent");
    for (int list = sr ? 1 : 0; list < 2; ++list)
      for (const auto& cp : list ? grp.copies : grp.lo_copies) {
        if (st) break;
        st = hip_check(hipMemcpyAsync(cp.host, p->slots[s] + cp.dev_off, cp.bytes, hipMemcpyDeviceToHost, p->down),
                       "offload download");
      }
    if (!st) st = hip_check(hipEventRecord(p->out_ev[s], p->down), "hipEventRecord");
    if (!st) p->out_recorded[s] = true;
  }
  // the caller's stream completes only after every download has landed (the
  // last download waits for the last step kernel) and every upload has ended
  if (!st) st = hip_check(hipEventRecord(p->end_ev, p->down), "hipEventRecord");
  if (!st) st = hip_check(hipStreamWaitEvent(caller, p->end_ev, 0), "hipStreamWaitEvent");
  if (!st) st = hip_check(hipEventRecord(p->end_ev, p->up), "hipEventRecord");
  if (!st) st = hip_check(hipStreamWaitEvent(caller, p->end_ev, 0), "hipStreamWaitEvent");
  if (!st) p->last_bytes_per_dir = sr ? p->bytes_per_dir - p->lo_bytes_per_dir : p->bytes_per_dir;
  return st;
}

ps_status ps_offload_bytes(const ps_offload_plan* p, uint64_t* h2d, uint64_t* d2h) {
  if (!p || !h2d || !d2h) return fail(PS_ERR_INVALID_ARG, "NULL argument");
  *h2d = p->last_bytes_per_dir;
  *d2h = p->last_bytes_per_dir;
  return PS_OK;
}

ps_status ps_offload_plan_destroy(ps_offload_plan* p) {
  destroy(p);
  return PS_OK;
}

}  // extern "C"
