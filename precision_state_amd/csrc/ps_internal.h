// ps_internal.h - declarations shared by the host layer and the kernels of
// libps.so. Not part of the public ABI (include/ps.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/ps.h"
#include "blob_cache.h"

namespace ps {

constexpr int kBlock = PS_BLOCK;   // elements per moment-scale block
constexpr int kItemBlocks = 4;     // blocks per 1024-element work item (elementwise and factored kernels)
constexpr int kItemElems = kBlock * kItemBlocks;
constexpr int kStepItemBlocks = 2; // blocks per (N)AdamW step work item: one wave, 32 lanes per block
constexpr int kStepItemElems = kBlock * kStepItemBlocks;
constexpr int kInlineMax = 16;     // tensor lists up to this size travel in kernel arguments
constexpr int kApplyItemElems = 512; // factored apply pass: elements per 64-lane work item (the step's layout)

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
  uint32_t tid;      // index in the caller's list (stochastic rounding stream key)
  uint32_t pad;
};

// Device record of a tensor with storage flags (generic-format kernel).
struct DevTensorEx {
  void* w;          // bf16 bits, or float when PS_TENSOR_FP32_PARAM
  uint16_t* lo;
  const void* g;    // bf16 bits, or float when PS_TENSOR_FP32_PARAM
  void* m;          // codes, or float when PS_TENSOR_FP32_MOMENTS
  float* ms;
  void* v;
  float* vs;
  int64_t numel;
  uint32_t flags;
  uint32_t tid;     // index in the caller's list (stochastic rounding stream key)
};

struct TableExPtr {
  const DevTensorEx* recs;
  const uint32_t* item_end;
  int32_t n;
};

// fp32 scalars of one update (see ps_step_scalars).
struct StepScalars {
  float B1, C1, B2, C2, EPS, A, RS2, AG, AM, CWD;
  uint32_t sr_step;   // stochastic rounding: the update number mod 2^32
  uint32_t pad;
  uint64_t sr_seed;   // stochastic rounding: the run's seed
};

// Work decomposition of a tensor list: tensor t owns the work items
// [item_end[t-1], item_end[t]); one work item is kStepItemElems elements.
struct TablePtr {
  const DevTensor* recs;
  const uint32_t* item_end;
  int32_t n;
};

// Tables that travel in the kernel arguments: up to kInlineMax tensors, and a
// one-tensor form for per-hook calls (about 72 bytes of arguments instead of
// about 1.1 KiB).
template <int N>
struct TableInlineN {
  DevTensor recs[N];
  uint32_t item_end[N];
  int32_t n;
};
using TableInline = TableInlineN<kInlineMax>;
using TableOne = TableInlineN<1>;

// ---- factored step (ps_factored.cpp, k_factored.hip) ----
constexpr int kFTileRows = 64;     // 2-D tile: 64 rows x 256 columns, one 256-thread workgroup
constexpr int kFTileCols = 256;
constexpr int kSTileRows = 256;    // stats tile: 256 rows x 256 columns, 4 chunks of kFTileRows rows
constexpr int kFRowColChunk = 256; // rows or columns per finalize workgroup
constexpr int kURows = 8;          // U^2 row tile (C % 8 == 0): 8 rows x 512 columns, one 64-lane wave
constexpr int kUCols = 512;
// Row-strip stats pass (tensors with C % 512 == 0 and C <= kStripMaxC): one
// kSNT-thread workgroup per group of whole rows, kStripGroups groups, taken
// when the list's eligible tensors have at least kStripMinGroupRows rows per
// group (each group writes and the finalize reads 16 bytes per column, which
// fewer rows per group would not amortise; smaller lists take the tiles).
constexpr int kSNT = 768;
constexpr int kStripGroups = 256;
constexpr int kStripMinGroupRows = 64;
constexpr int kStripMaxC = 2 * kSNT * 8;

// 2-D tensor [R, C] of a factored step; workspace pointers are per tensor.
struct F2D {
  uint16_t* hi;
  uint16_t* lo;
  const uint16_t* g;
  float* row;        // [R] EMA of row means (caller state)
  float* col;        // [C] EMA of column means (caller state)
  double* rowpart;   // [nrp][R] row sums per tile column (strip: [1][R], whole rows)
  double* colpart;   // [sntr][C] column sums per 256-row stats band (strip: per row segment)
  double* qpart;     // strip: [sntr][C] column sums of g^2 / r_i per row segment; else NULL
  double* rpart;     // [nrw] sums of the new row EMAs per 256-row chunk
  float* rho;        // [R] 1/sqrt(r_i / mean r)
  float* kap;        // [C] 1/sqrt(c_j)
  double* rinv;      // [R] 1/r_i in double, for the U^2 pass (NULL if strip)
  double* cinv;      // [C] 1/c_j in double, for the U^2 pass (NULL if strip)
  double* upart;     // sums of g^2 / (r_i c_j) per column chunk, row tile, item or tile (times mean r: sum of U^2)
  float* f;          // clip factor lr / max(1, RMS(U)/d)
  uint16_t* mc;      // first moment codes (signed kind) or NULL
  float* ms;         // first moment block scales or NULL
  int32_t R, C, ntr, ntc, nrw, ncw;
  int32_t nuc;       // vec: column bands of the U^2 row tiles (kUCols wide)
  int32_t sntr;      // stats tiles along the rows (kSTileRows tall); colpart has sntr rows
  int32_t vec;       // C % 8 == 0: 16-byte row segments
  int32_t flat;      // R*C < 2^31 and (vec or a first moment): U^2 and apply passes run over 1024-element items
  int32_t nitems;    // flat: items of 1024 elements
  int32_t npart;     // entries of upart: column chunks if strip, U^2 row tiles if vec, else nitems if flat, else ntr * ntc
  uint32_t tid;      // index in the caller's list (stochastic rounding stream key)
  int32_t strip;     // stats in the row-strip pass; sum of U^2 = rbar * sum_j Q_j / c_j (upart: per column chunk)
  int32_t nrp;       // row partials per row in rowpart (ntc, or 1 for strip)
  int32_t pad;
};

// Rows [row0, row1) of 2-D tensor t2[t], one segment of a strip-pass group;
// its column partials go to row `slot` of the tensor's colpart and qpart.
struct FSeg {
  uint32_t t;
  int32_t row0, row1, slot;
};

// 1-D tensor of a factored step (second moment kept in the uint16 codec).
struct F1D {
  uint16_t* hi;
  uint16_t* lo;
  const uint16_t* g;
  uint16_t* vc;
  float* vs;
  float* v;          // [n] this step's v (workspace)
  double* upart;     // [nitems] sums of U^2 per 1024-element item
  float* f;
  uint16_t* mc;      // first moment codes (signed kind) or NULL
  float* ms;         // first moment block scales or NULL
  int64_t n;
  int32_t nitems;
  uint32_t tid;      // index in the caller's list (stochastic rounding stream key)
};

struct FScalars {
  float B2, C2, EPS1, CWD;
  float B1, C1;      // first moment EMA (fm != 0)
  double lr, clip;
  int32_t wd;
  int32_t fm;        // first moment kept in mc / ms
  uint64_t sr_seed;  // stochastic rounding: the run's seed
  uint32_t sr_step;  // stochastic rounding: the update number mod 2^32
  uint32_t pad;
};

struct FPlan {      // device tables of one factored call
  const F2D* t2;
  const uint32_t* tile_end;    // [n2] prefix ends over 2-D tiles
  const uint32_t* rc_end;      // [n2] prefix ends over row/column finalize workgroups
  const uint32_t* tile_nf_end; // [n2] prefix ends over tiles of tensors that are not flat
  const uint32_t* item2_end;   // [n2] prefix ends over 1024-element items of flat tensors
  const uint32_t* rt_end;      // [n2] prefix ends over U^2 row tiles of vec tensors
  const uint32_t* tile_u_end;  // [n2] prefix ends over U^2 tiles of tensors neither vec nor flat
  const uint32_t* item2u_end;  // [n2] prefix ends over U^2 items of flat tensors that are not vec
  const F1D* t1;
  const uint32_t* item_end;    // [n1] prefix ends over 1-D items
  const uint32_t* seg_end;     // [n_groups] prefix ends over strip segments
  const FSeg* segs;            // strip segments, group by group
  int32_t n2, n1;
  uint32_t n_tiles, n_rc, n_items, n_tiles_nf, n_items2;
  uint32_t n_rt, n_tiles_u, n_items2u;
  uint32_t n_groups;           // workgroups of the strip pass
};

ps_status launch_factored(const FPlan& plan, const FScalars& sc, int split_mode, hipStream_t s);

// One factored call prepared on the host (ps_factored.cpp): the device plan's
// image (F2D[n2] | F1D[n1] | seven [n2] prefix-end lists | item_end[n1] |
// seg_end[n_groups] | FSeg[]) with
// its workspace pointers final, the workspace size and the scalars. The
// plan's table pointers are offsets into the image until factored_bind.
struct FactoredCall {
  std::vector<unsigned char> image;
  size_t ws_bytes = 0;
  FPlan plan{};
  FScalars sc{};
  bool empty = true;   // no tensor to step
};
// Validates the call and lays out the workspace at `ws` (NULL: sizes only).
ps_status factored_prepare(const ps_tensor* t, int32_t n, const ps_factored_hparams* hp, int64_t step, char* ws,
                           FactoredCall& c);
// Points the plan's tables into a device copy of the image.
void factored_bind(FactoredCall& c, const void* dev_image);

// ---- errors (ps_abi.cpp) ----
ps_status fail(ps_status s, const char* fmt, ...);
ps_status hip_check(hipError_t e, const char* what);

// Device copies of host blobs, cached by content (blob_cache.h; the HIP
// backend is in ps_abi.cpp). A caller holds a TableLease from before
// device_blob until the launches that read the blob are enqueued.
struct HipBlobBackend {
  using Stream = hipStream_t;
  using Event = hipEvent_t;
  int alloc_chunk(size_t bytes, char** d, char** h);
  void free_chunk(char* d, char* h);
  int create_event(hipEvent_t* e);
  void destroy_event(hipEvent_t e);
  int upload(char* d, const char* h, size_t bytes, hipStream_t s, hipEvent_t e);
  bool event_done(hipEvent_t e);
  int stream_wait(hipStream_t s, hipEvent_t e);
  int device_sync();
  void sync_stream(hipStream_t s);
};
using TableCache = BlobCache<HipBlobBackend>;
using TableLease = TableCache::Lease;
TableCache& table_cache();
ps_status device_blob(const void* data, size_t bytes, hipStream_t s, const void** dptr, TableLease& lease);
bool is_finite(double x);
bool is_aligned(const void* p, uintptr_t a);

// ---- host scalars (ps_scalars.cpp) ----
void step_scalars(const ps_hparams& hp, int64_t step, StepScalars* out);

// ---- device properties (ps_abi.cpp) ----

// ---- launchers (k_adam.hip, k_elementwise.hip) ----
ps_status launch_adam_ptr(const TablePtr& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                          hipStream_t s);
ps_status launch_adam_one(const TableOne& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                          hipStream_t s);
ps_status launch_adam_inline(const TableInline& tbl, uint32_t total_items, const ps_hparams& hp,
                             const StepScalars& c, hipStream_t s);
ps_status launch_adam_ex(const TableExPtr& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                         hipStream_t s);
ps_status launch_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, int mode, hipStream_t s);
ps_status launch_join(const uint16_t* hi, const uint16_t* lo, float* w, int64_t n, int mode, hipStream_t s);
ps_status launch_encode(const float* x, uint16_t* code, float* scale, int64_t n, int kind, hipStream_t s);
ps_status launch_decode(const uint16_t* code, const float* scale, float* x, int64_t n, int kind, hipStream_t s);

}  // namespace ps
