// ps_internal.h - declarations shared by the host layer and the kernels of
// libps.so. Not part of the public ABI (include/ps.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ps.h"

namespace ps {

constexpr int kBlock = PS_BLOCK;   // elements per moment-scale block
constexpr int kItemBlocks = 4;     // blocks per wave work item (16 lanes per block)
constexpr int kItemElems = kBlock * kItemBlocks;
constexpr int kInlineMax = 16;     // tensor lists up to this size travel in kernel arguments

// Device record of one tensor in a multi-tensor launch (64 bytes).
struct DevTensor {
  uint16_t* hi;
  uint16_t* lo;
  const uint16_t* g;
  uint16_t* mc;
  float* ms;
  uint16_t* vc;
  float* vs;
  int64_t numel;
};

// fp32 scalars of one update (see ps_step_scalars).
struct StepScalars {
  float B1, C1, B2, C2, EPS, A, RS2, AG, AM, CWD;
};

// Work decomposition of a tensor list: tensor t owns the work items
// [item_end[t-1], item_end[t]); one work item is kItemElems elements.
struct TablePtr {
  const DevTensor* recs;
  const uint32_t* item_end;
  int32_t n;
};

struct TableInline {
  DevTensor recs[kInlineMax];
  uint32_t item_end[kInlineMax];
  int32_t n;
};

// ---- errors (ps_abi.cpp) ----
ps_status fail(ps_status s, const char* fmt, ...);
ps_status hip_check(hipError_t e, const char* what);

// ---- host scalars (ps_scalars.cpp) ----
void step_scalars(const ps_hparams& hp, int64_t step, StepScalars* out);

// ---- device properties (ps_abi.cpp) ----
int device_cu_count();

// ---- launchers (k_adam.hip, k_elementwise.hip) ----
ps_status launch_adam_ptr(const TablePtr& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                          hipStream_t s);
ps_status launch_adam_inline(const TableInline& tbl, uint32_t total_items, const ps_hparams& hp,
                             const StepScalars& c, hipStream_t s);
ps_status launch_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, int mode, hipStream_t s);
ps_status launch_join(const uint16_t* hi, const uint16_t* lo, float* w, int64_t n, int mode, hipStream_t s);
ps_status launch_encode(const float* x, uint16_t* code, float* scale, int64_t n, int kind, hipStream_t s);
ps_status launch_decode(const uint16_t* code, const float* scale, float* x, int64_t n, int kind, hipStream_t s);

}  // namespace ps
