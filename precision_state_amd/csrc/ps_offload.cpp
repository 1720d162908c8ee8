// ps_offload.cpp - host-offload pipeline for the fused (N)AdamW step [NADAM,
// opening post: the moments (and here the Kahan residuals) stay in host memory
// and cross PCIe every step; KAHAN: only the 16 residual bits travel; with
// stochastic rounding, the pages' setting when host memory is short, no
// residual exists and only the moments travel].
//
// kSlots (2) device staging slots hold one group's residuals, codes and
// scales each. Group k uses slot s = k % 2:
//   upload stream:   wait(download of k-2 done) -> copies host->slot -> event in[s]
//   compute stream:  wait(in[s]) -> fused step of group k -> event done[s]
//   download stream: wait(done[s]) -> copies slot->host -> event out[s]
// so the upload of k+1 and the download of k-1 overlap the step of k, and the
// two copy directions run concurrently (a third slot measured no faster: the
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
  hipStream_t up = nullptr, down = nullptr;
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
  delete p;
}

ps_status check_host(const void* p, const char* what, int g, int i, uintptr_t align) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "group %d tensor %d: %s is NULL", g, i, what);
  if (!is_aligned(p, align)) return fail(PS_ERR_ALIGNMENT, "group %d tensor %d: %s misaligned", g, i, what);
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeHost)
    return fail(PS_ERR_INVALID_ARG, "group %d tensor %d: %s is not pinned host memory", g, i, what);
  return PS_OK;
}

void add_copy(std::vector<ps_offload_plan::Copy>& cl, void* host, size_t dev_off, size_t bytes, uint64_t& total) {
  if (!cl.empty() && (char*)cl.back().host + cl.back().bytes == (char*)host && cl.back().dev_off + cl.back().bytes == dev_off)
    cl.back().bytes += bytes;
  else
    cl.push_back({host, dev_off, bytes});
  total += bytes;
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
  if (!plan) return fail(PS_ERR_INVALID_ARG, "plan is NULL");
  *plan = nullptr;
  if (n_groups < 0 || (n_groups > 0 && !groups)) return fail(PS_ERR_INVALID_ARG, "bad group list");
  ps_offload_plan* p = new ps_offload_plan;
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
      // records are completed with the slot base at upload time (below)
      recs[g].push_back(DevTensor{x.w_hi, (uint16_t*)q.lo, x.grad, (uint16_t*)q.mc, (float*)q.ms, (uint16_t*)q.vc,
                                  (float*)q.vs, x.numel, q.tid, 0});
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
  // device tables: per group and slot, DevTensor[n] then item ends[n]
  std::vector<unsigned char> tab;
  for (int32_t g = 0; g < n_groups; ++g)
    for (int s = 0; s < kSlots; ++s) {
      p->groups[g].table_off[s] = tab.size();
      const size_t n = recs[g].size();
      tab.resize(tab.size() + up256(n * sizeof(DevTensor)) + up256(n * sizeof(uint32_t)));
    }
  ps_status st = PS_OK;
  for (int s = 0; s < kSlots && !st; ++s)
    if (hipMalloc((void**)&p->slots[s], p->slot_bytes ? p->slot_bytes : 256) != hipSuccess)
      st = fail(PS_ERR_NO_MEMORY, "offload staging slot allocation failed (%zu bytes)", p->slot_bytes);
  if (!st && hipMalloc((void**)&p->tables, tab.empty() ? 256 : tab.size()) != hipSuccess)
    st = fail(PS_ERR_NO_MEMORY, "offload table allocation failed");
  if (st) {
    destroy(p);
    return st;
  }
  for (int32_t g = 0; g < n_groups; ++g)
    for (int s = 0; s < kSlots; ++s) {
      const size_t n = recs[g].size();
      DevTensor* dst = (DevTensor*)(tab.data() + p->groups[g].table_off[s]);
      for (size_t i = 0; i < n; ++i) {
        DevTensor r = recs[g][i];
        char* base = p->slots[s];
        r.lo = (uint16_t*)(base + (size_t)r.lo);
        r.mc = (uint16_t*)(base + (size_t)r.mc);
        r.vc = (uint16_t*)(base + (size_t)r.vc);
        r.ms = (float*)(base + (size_t)r.ms);
        r.vs = (float*)(base + (size_t)r.vs);
        dst[i] = r;
      }
      if (n) memcpy(tab.data() + p->groups[g].table_off[s] + up256(n * sizeof(DevTensor)), ends[g].data(),
                    n * sizeof(uint32_t));
    }
  p->bytes_per_dir += p->lo_bytes_per_dir;
  p->last_bytes_per_dir = p->bytes_per_dir;
  if (!tab.empty()) st = hip_check(hipMemcpy(p->tables, tab.data(), tab.size(), hipMemcpyHostToDevice), "table upload");
  if (!st) st = hip_check(hipStreamCreateWithFlags(&p->up, hipStreamNonBlocking), "hipStreamCreate");
  if (!st) st = hip_check(hipStreamCreateWithFlags(&p->down, hipStreamNonBlocking), "hipStreamCreate");
  for (int s = 0; s < kSlots && !st; ++s) {
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
  hipStream_t cs = (hipStream_t)stream;
  ps_status st = hip_check(hipEventRecord(p->start_ev, cs), "hipEventRecord");
  if (!st) st = hip_check(hipStreamWaitEvent(p->up, p->start_ev, 0), "hipStreamWaitEvent");
  if (!st) st = hip_check(hipStreamWaitEvent(p->down, p->start_ev, 0), "hipStreamWaitEvent");
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
  // the caller's stream completes only after every download has landed
  if (!st) st = hip_check(hipEventRecord(p->end_ev, p->down), "hipEventRecord");
  if (!st) st = hip_check(hipStreamWaitEvent(cs, p->end_ev, 0), "hipStreamWaitEvent");
  if (!st) st = hip_check(hipEventRecord(p->end_ev, p->up), "hipEventRecord");
  if (!st) st = hip_check(hipStreamWaitEvent(cs, p->end_ev, 0), "hipStreamWaitEvent");
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
