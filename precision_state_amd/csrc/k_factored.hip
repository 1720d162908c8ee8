// k_factored.hip - Adafactor-style step: factored second moment (row/column
// EMAs of mean g^2 + eps1, constant beta2 or the 1 - t^decay_rate schedule),
// update clipping by the tensor's RMS, optional first moment (EMA of the
// clipped update in the signed codec), decoupled weight decay, residual split
// [ADAF, adafactor_step_param; PRODIGY, beta1 = 0 / factored / update
// clipping].
//
// 2-D tensors [R, C] are cut into 64 x 256 tiles, one 256-thread workgroup
// each; thread t handles columns (t % 32) * 8 .. + 8 of rows t / 32 + 8k,
// k = 0..7, so each half-wave reads one 512-byte row segment per load.
// Passes over the gradient: tile row/column sums of q = g^2 + eps1 (double);
// row/column finalize (EMAs, chunk sums of the new row EMA); factors
// rho_i = 1/sqrt(r_i / rbar), kap_j = 1/sqrt(c_j); tile sums of U^2 (double);
// clip factor per tensor; apply. 1-D tensors keep v in the uint16 codec and
// use 1024-element items like the fused (N)AdamW step.
//
// All reductions use fixed trees (no atomics), so results are deterministic.
#include "dev_common.h"
#include "ps_internal.h"

namespace ps {
namespace {

constexpr int kT = 256;
// The U^2 launch and the flat apply pass give each XCD runs of 256
// consecutive workgroups: about 2% less time per step than plain index order
// on the double-block shapes when both ran over 1024-element items (runs of
// 128 to 1024 items measured alike).
constexpr uint32_t kFlatXcdChunk = 256;
// The flat apply pass takes the fused step's lane layout and work order: one
// 512-element item per 64-lane workgroup, lane t owning elements 8t .. 8t+7
// (a 256-element block per 32 lanes, so each load or store instruction of a
// wave covers 1 KiB of one stream), each XCD taking runs of 2048 items. A
// streaming kernel with this pass's 3-read/2-write mix and no arithmetic ran
// 6% faster in this layout than with two 8-element runs per lane at offsets
// la and la + 128 over 1024-element items.
constexpr uint32_t kApplyXcdChunk = 2048;

// The apply pass touches the weights, residuals and first-moment codes once
// per step: those accesses carry the non-temporal hint (measured ~9% faster
// per step), and so do the stats pass's interior-tile gradient loads (~1%).
// The U^2 pass keeps plain loads (the hint there changed nothing).
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const u32x4 t = __builtin_nontemporal_load((const GLOBAL u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_stream(uint16_t* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (GLOBAL u32x4*)p);
}

// First entry of the wave-uniform prefix-end array greater than x.
__device__ __forceinline__ int find_end(const uint32_t* __restrict__ end, int n, uint32_t x, uint32_t& begin) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (end[mid] > x)
      hi = mid;
    else
      lo = mid + 1;
  }
  begin = lo ? end[lo - 1] : 0u;
  return lo;
}

// 8 consecutive 16-bit values of row r starting at column c (bits of missing
// elements are 0, valid bit j set when column c + j exists).
__device__ __forceinline__ uint32_t load_row8(const uint16_t* __restrict__ base, const F2D& X, int r, int c,
                                              uint32_t* w) {
  w[0] = w[1] = w[2] = w[3] = 0u;
  if (r >= X.R || c >= X.C) return 0u;
  const uint16_t* p = base + (size_t)r * (size_t)X.C + (size_t)c;
  if (X.vec && c + 8 <= X.C) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    return 0xFFu;
  }
  uint32_t valid = 0;
  for (int j = 0; j < 8; ++j)
    if (c + j < X.C) {
      w[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
      valid |= 1u << j;
    }
  return valid;
}

__device__ __forceinline__ void store_row8(uint16_t* __restrict__ base, const F2D& X, int r, int c, uint32_t valid,
                                           const uint32_t* w) {
  if (r >= X.R || c >= X.C) return;
  uint16_t* p = base + (size_t)r * (size_t)X.C + (size_t)c;
  if (valid == 0xFFu && X.vec) {
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  for (int j = 0; j < 8; ++j)
    if (valid & (1u << j)) p[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
}

__device__ __forceinline__ float bf16_at(const uint32_t* w, int j) {
  return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
}

// Stochastic rounding: the random 16 bits of element e of the stream s
// (output e/4, bits 16*(e % 4)), for element runs that do not start on a
// multiple of 4.
__device__ __forceinline__ uint32_t sr_bits1(uint64_t s, int64_t e) {
  const uint64_t w = splitmix64_mix(s + ((uint64_t)(e >> 2) + 1) * kGolden);
  return (uint32_t)(w >> (16 * (e & 3))) & 0xFFFFu;
}

// Sum of a double over the 256 threads of the workgroup, fixed tree.
__device__ __forceinline__ double block_sum(double x, double* red) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int o = kT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  double r = red[0];
  __syncthreads();
  return r;
}

// ---- pass 1: tile row and column sums of q = g^2 + eps1 ---------------------
// One 256 x 256 stats tile per 256-thread workgroup, walked in 4 chunks of 64
// rows: thread (rg, cg) takes columns c .. c+7 (c = 8 cg) of chunk rows
// rg + 8 k. Row sums are finished per chunk (a 256-column partial per row);
// column sums run on across the chunks, so the LDS reduction, its barrier and
// the column-partial stores come once per 128 KiB of gradient: with one per
// 64-row tile they took a fifth of the pass.
__global__ __launch_bounds__(kT) void k_f_stats(FPlan P, FScalars S) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.tile_end, P.n2, blockIdx.x, begin)];
  const uint32_t tile = blockIdx.x - begin;
  const int ts = (int)(tile / (uint32_t)X.ntc), tc = (int)(tile - (uint32_t)ts * X.ntc);
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c = tc * kFTileCols + cg * 8;
  double cacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cacc[j] = 0.0;
  for (int ch = 0; ch < kSTileRows / kFTileRows; ++ch) {
    const int row0 = ts * kSTileRows + ch * kFTileRows;   // first row of the chunk
    if (row0 >= X.R) break;   // uniform
    double rs[8];
    if (X.vec && row0 + kFTileRows <= X.R && (tc + 1) * kFTileCols <= X.C) {
      // Interior chunk: all eight row segments are requested at once, then
      // summed in the same order as below.
      uint32_t w[8][4];
      const uint16_t* p = X.g + (size_t)(row0 + rg) * (size_t)X.C + (size_t)c;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x4 v = __builtin_nontemporal_load((const GLOBAL u32x4*)(p + (size_t)(8 * k) * (size_t)X.C));
        w[k][0] = v.x; w[k][1] = v.y; w[k][2] = v.z; w[k][3] = v.w;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        rs[k] = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float g = bf16_at(w[k], j);
          const float q = g * g + S.EPS1;
          rs[k] += (double)q;
          cacc[j] += (double)q;
        }
      }
    } else {
      for (int k = 0; k < 8; ++k) {
        const int r = row0 + rg + 8 * k;
        uint32_t w[4];
        const uint32_t valid = load_row8(X.g, X, r, c, w);
        rs[k] = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float g = bf16_at(w, j);
          const float q = (valid >> j & 1u) ? g * g + S.EPS1 : 0.0f;
          rs[k] += (double)q;
          cacc[j] += (double)q;
        }
      }
    }
    // Row sums over the 32 column groups of a half-wave by transpose-reduce:
    // at each exchange a lane keeps half of its rows and receives its
    // partner's partial of those rows (9 shuffles instead of 8 x 5). Lane bits
    // 4, 3, 2 of cg select the row k = 4*b4 + 2*b3 + b2 the lane ends with.
    const int b4 = (cg >> 4) & 1, b3 = (cg >> 3) & 1, b2 = (cg >> 2) & 1;
    double a[4], bb[2], x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double keep = b4 ? rs[4 + q] : rs[q], send = b4 ? rs[q] : rs[4 + q];
      a[q] = keep + __shfl_xor(send, 16, 32);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const double keep = b3 ? a[2 + q] : a[q], send = b3 ? a[q] : a[2 + q];
      bb[q] = keep + __shfl_xor(send, 8, 32);
    }
    {
      const double keep = b2 ? bb[1] : bb[0], send = b2 ? bb[0] : bb[1];
      x = keep + __shfl_xor(send, 4, 32);
    }
    x += __shfl_xor(x, 2, 32);
    x += __shfl_xor(x, 1, 32);
    const int r = row0 + rg + 8 * (4 * b4 + 2 * b3 + b2);
    if ((cg & 3) == 0 && r < X.R) X.rowpart[(size_t)tc * X.R + r] = x;
  }
  __shared__ double lds[8][kFTileCols];
#pragma unroll
  for (int j = 0; j < 8; ++j) lds[rg][cg * 8 + j] = cacc[j];
  __syncthreads();
  const int cc = tc * kFTileCols + (int)threadIdx.x;
  if (cc < X.C) {
    double s = 0.0;
    for (int q = 0; q < 8; ++q) s += lds[q][threadIdx.x];
    X.colpart[(size_t)ts * X.C + cc] = s;
  }
}

// ---- pass 2: row/column EMAs and chunk sums of the new row EMA -------------
__global__ __launch_bounds__(kT) void k_f_rowcol(FPlan P, FScalars S) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.rc_end, P.n2, blockIdx.x, begin)];
  const int w = (int)(blockIdx.x - begin);
  __shared__ double red[kT];
  if (w < X.nrw) {
    const int i = w * kFRowColChunk + (int)threadIdx.x;
    double rv = 0.0;
    if (i < X.R) {
      double s = 0.0;
#pragma unroll 8
      for (int tc = 0; tc < X.ntc; ++tc) s += X.rowpart[(size_t)tc * X.R + i];
      const float mean = (float)(s / (double)X.C);
      const float r = __builtin_fmaf(S.B2, X.row[i], S.C2 * mean);
      X.row[i] = r;
      rv = (double)r;
    }
    const double t = block_sum(rv, red);
    if (threadIdx.x == 0) X.rpart[w] = t;
  } else {
    const int j = (w - X.nrw) * kFRowColChunk + (int)threadIdx.x;
    if (j < X.C) {
      double s = 0.0;
#pragma unroll 16
      for (int tr = 0; tr < X.sntr; ++tr) s += X.colpart[(size_t)tr * X.C + j];
      const float mean = (float)(s / (double)X.R);
      X.col[j] = __builtin_fmaf(S.B2, X.col[j], S.C2 * mean);
    }
  }
}

// ---- pass 3: factors of V^-1/2 ----------------------------------------------
__global__ __launch_bounds__(kT) void k_f_factors(FPlan P) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.rc_end, P.n2, blockIdx.x, begin)];
  const int w = (int)(blockIdx.x - begin);
  if (w < X.nrw) {
    double s = 0.0;
    for (int q = 0; q < X.nrw; ++q) s += X.rpart[q];
    const float rbar = (float)(s / (double)X.R);
    const int i = w * kFRowColChunk + (int)threadIdx.x;
    if (i < X.R) X.rho[i] = 1.0f / __builtin_sqrtf(X.row[i] / rbar);
  } else {
    const int j = (w - X.nrw) * kFRowColChunk + (int)threadIdx.x;
    if (j < X.C) X.kap[j] = 1.0f / __builtin_sqrtf(X.col[j]);
  }
}

// ---- pass 4: tile sums of U^2, U = (g * rho_i) * kap_j (tensors whose rows
// are not 16-byte runs and that keep no first moment) ---------------------------
__global__ __launch_bounds__(kT) void k_f_usq(FPlan P) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.tile_u_end, P.n2, blockIdx.x, begin)];
  const uint32_t tile = blockIdx.x - begin;
  const int tr = (int)(tile / (uint32_t)X.ntc), tc = (int)(tile - (uint32_t)tr * X.ntc);
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c = tc * kFTileCols + cg * 8;
  float kap[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kap[j] = (c + j < X.C) ? X.kap[c + j] : 0.0f;
  double acc = 0.0;
  for (int k = 0; k < 8; ++k) {
    const int r = tr * kFTileRows + rg + 8 * k;
    uint32_t w[4];
    const uint32_t valid = load_row8(X.g, X, r, c, w);
    if (!valid) continue;
    const float rho = X.rho[r];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float U = (bf16_at(w, j) * rho) * kap[j];
      acc += (valid >> j & 1u) ? (double)U * (double)U : 0.0;
    }
  }
  __shared__ double red[kT];
  const double t = block_sum(acc, red);
  if (threadIdx.x == 0) X.upart[tile] = t;
}

// ---- flat items of 2-D tensors --------------------------------------------------
// The U^2 pass of tensors whose rows are not 16-byte runs takes 1024-element
// items (each lane two runs of 8); the apply pass takes the fused step's
// 512-element items (k_f_apply_flat). Column counts that are not a multiple
// of 8 (only with a first moment) take per-element factors.

__device__ __forceinline__ void load_kap8(const float* __restrict__ kap, uint32_t j, float* k) {
  const float4 a = *reinterpret_cast<const float4*>(kap + j);
  const float4 b = *reinterpret_cast<const float4*>(kap + j + 4);
  k[0] = a.x; k[1] = a.y; k[2] = a.z; k[3] = a.w; k[4] = b.x; k[5] = b.y; k[6] = b.z; k[7] = b.w;
}

// Flat items of a tensor whose column count is not a multiple of 8 (taken
// only with a first moment, whose per-256 blocks follow the flattened index):
// a run of 8 may cross rows and the tensor's last run may be partial, so the
// row and column of each element are found one by one and the loads and
// stores of a partial run go element by element. Missing elements read as
// `fill` and are not written.
template <class I>
__device__ __forceinline__ uint4 ld_run(const uint16_t* p, I e, I n, uint32_t fill, bool nt) {
  if (e + 8 <= n) return nt ? ld_stream(p + e) : *reinterpret_cast<const uint4*>(p + e);
  const GLOBAL uint16_t* q = (const GLOBAL uint16_t*)p;
  uint32_t w[4];
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = (e + 2 * j < n) ? q[e + 2 * j] : (fill & 0xFFFFu);
    const uint32_t b = (e + 2 * j + 1 < n) ? q[e + 2 * j + 1] : (fill >> 16);
    w[j] = a | (b << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <class I>
__device__ __forceinline__ void st_run(uint16_t* p, I e, I n, const uint32_t* w) {
  if (e + 8 <= n) {
    st_stream(p + e, make_uint4(w[0], w[1], w[2], w[3]));
    return;
  }
  GLOBAL uint16_t* q = (GLOBAL uint16_t*)p;
  for (int j = 0; j < 8; ++j)
    if (e + j < n) q[e + j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
}

// Factor rho_i * kap_j of flattened element e (e < R*C).
__device__ __forceinline__ void elem_factors(const F2D& X, uint32_t e, float& rho, float& kap) {
  const uint32_t i = e / (uint32_t)X.C;
  rho = X.rho[i];
  kap = X.kap[e - i * (uint32_t)X.C];
}

// U^2 sum of one item, any column count (same per-lane order as the run path).
__device__ __forceinline__ void usq_item_any(const F2D& X, uint32_t item) {
  const uint32_t n = (uint32_t)X.R * (uint32_t)X.C;
  const uint32_t la = (threadIdx.x >> 4) * (uint32_t)kBlock + (threadIdx.x & 15) * 8u;
  double acc = 0.0;
  for (int h = 0; h < 2; ++h) {
    const uint32_t e = item * (uint32_t)kItemElems + la + 128u * h;
    if (e >= n) continue;
    const uint4 gv = ld_run(X.g, e, n, 0u, false);
    const uint32_t w[4] = {gv.x, gv.y, gv.z, gv.w};
    for (int jj = 0; jj < 8; ++jj) {
      if (e + jj >= n) break;
      float rho, kap;
      elem_factors(X, e + jj, rho, kap);
      const float U = (bf16_at(w, jj) * rho) * kap;
      acc += (double)U * (double)U;
    }
  }
  for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (threadIdx.x == 0) X.upart[item] = acc;
}

__device__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w);

// U^2 sum of one row tile of a tensor whose rows are 16-byte runs: kURows
// rows x kUCols columns, lane l taking columns c .. c+7 (c = band start +
// 8 l) of every row of the tile. The lane loads its 8 column factors once and
// all its rows' gradient runs at once (8 KiB per wave in flight), and each
// row's factor is one scalar load; per element the flat items instead load a
// column factor (4 bytes) for every 2-byte gradient. Lane order: row by row,
// columns in order; then the wave's xor tree. Lanes past the last column and
// rows past the last row hold g = 0 and add exact zeros.
__device__ __forceinline__ void usq_row_tile(const FPlan& P, uint32_t w) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.rt_end, P.n2, w, begin)];
  const uint32_t t = w - begin;
  const int tr = (int)(t / (uint32_t)X.nuc), tc = (int)(t - (uint32_t)tr * X.nuc);
  const int c = tc * kUCols + (int)threadIdx.x * 8;
  const int r0 = tr * kURows;
  const bool col_ok = c < X.C;
  float kap[8];
  if (col_ok) {
    load_kap8(X.kap, (uint32_t)c, kap);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) kap[j] = 0.0f;
  }
  uint4 gv[kURows];
#pragma unroll
  for (int k = 0; k < kURows; ++k) {
    const int r = r0 + k;
    gv[k] = (col_ok && r < X.R) ? ld_stream(X.g + (size_t)r * (size_t)X.C + (size_t)c) : make_uint4(0u, 0u, 0u, 0u);
  }
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < kURows; ++k) {
    const int r = r0 + k;
    const float rho = r < X.R ? X.rho[r] : 0.0f;
    const uint32_t g[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float U = (bf16_at(g, j) * rho) * kap[j];
      acc += (double)U * (double)U;
    }
  }
  for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (threadIdx.x == 0) X.upart[t] = acc;
}

__device__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w);

// The U^2 pass in one launch of 64-lane workgroups: the row tiles of tensors
// whose rows are 16-byte runs, then the flat items of the other tensors that
// keep a first moment, then the 1-D tensors' stats items (decode v, EMA,
// U^2), which thus do not wait on a launch of their own.
__global__ __launch_bounds__(64) void k_f_usq_flat(FPlan P, FScalars S) {
  const uint32_t wg = xcd_item<kFlatXcdChunk>(blockIdx.x, gridDim.x);
  if (wg < P.n_rt) {   // uniform
    usq_row_tile(P, wg);
    return;
  }
  const uint32_t w2 = wg - P.n_rt;
  if (w2 >= P.n_items2u) {   // uniform: an item of a 1-D tensor
    f1_stats_item(P, S, w2 - P.n_items2u);
    return;
  }
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.item2u_end, P.n2, w2, begin)];
  usq_item_any(X, w2 - begin);
}

// Apply of one 512-element item, any column count: the arithmetic of the run
// path below, with each element's own row and column factors.
template <int SPLIT>
__device__ __forceinline__ void apply_item_any(const F2D& X, uint32_t item, const FScalars& S, float f) {
  constexpr bool SR = SPLIT == PS_SPLIT_STOCHASTIC;
  const uint32_t n = (uint32_t)X.R * (uint32_t)X.C;
  const uint32_t e = item * (uint32_t)kApplyItemElems + threadIdx.x * 8u;
  const uint32_t blk = item * 2u + (threadIdx.x >> 5);
  const bool blk_ok = blk * (uint32_t)kBlock < n;
  const float ms_old = (S.fm && blk_ok) ? X.ms[blk] : 0.0f;
  float m[8];
  float mx = 0.0f;
  for (int j = 0; j < 8; ++j) m[j] = 0.0f;
  if (e < n) {
    const uint4 gv = ld_run(X.g, e, n, 0u, true), hv = ld_run(X.hi, e, n, 0u, true);
    const uint4 lv = SR ? make_uint4(0u, 0u, 0u, 0u) : ld_run(X.lo, e, n, 0u, true);
    const uint4 mv = S.fm ? ld_run(X.mc, e, n, 0x80008000u, true) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
    const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
    const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
    uint32_t oh[4], ol[4];
    uint64_t rnd[2] = {0u, 0u};
    if (SR) sr_bits8(sr_stream(S.sr_seed, S.sr_step, X.tid), e, rnd);
    for (int p = 0; p < 4; ++p) {
      uint32_t wb[2];
      for (int o = 0; o < 2; ++o) {
        const int jj = 2 * p + o;
        const float w = SR ? bf16_at(hw, jj) : __uint_as_float(join_pair_elem<SPLIT>(hw[p], lw[p], o));
        float x = 0.0f;
        if (e + jj < n) {
          float rho, kap;
          elem_factors(X, e + jj, rho, kap);
          x = ((bf16_at(gw, jj) * rho) * kap) * f;
          if (S.fm) {
            const float m0 = dec_signed(o ? code_hi_f(mw[p]) : code_lo_f(mw[p]), ms_old);
            x = __builtin_fmaf(S.B1, m0, S.C1 * x);
            m[jj] = x;
            mx = __builtin_fmaxf(mx, __builtin_fabsf(x));
          }
          if (S.wd) x = __builtin_fmaf(S.CWD, w, x);
        }
        wb[o] = __float_as_uint(w - x);
      }
      if (SR) {
        const uint64_t q = rnd[p >> 1] >> (32 * (p & 1));
        oh[p] = sr_pair(wb[0], wb[1], (uint32_t)q & 0xFFFFu, (uint32_t)(q >> 16) & 0xFFFFu);
      } else {
        split_pair<SPLIT>(wb[0], wb[1], oh[p], ol[p]);
      }
    }
    st_run(X.hi, e, n, oh);
    if (!SR) st_run(X.lo, e, n, ol);
  }
  if (!S.fm) return;   // uniform
  float sm, inv;
  block_scale(row32_max(mx), sm, inv);
  if (e < n) {
    uint32_t om[4];
    for (int p = 0; p < 4; ++p) om[p] = enc_signed(m[2 * p], inv) | (enc_signed(m[2 * p + 1], inv) << 16);
    st_run(X.mc, e, n, om);
  }
  if ((threadIdx.x & 31) == 0 && blk_ok) X.ms[blk] = sm;
}

// Flat apply over the 2-D items. (The 1-D apply items stay in a launch of
// their own: riding at the end of this one, they made this kernel's code
// 25% slower.) Lane t's run is elements 8t .. 8t+7 of the item; with
// C % 8 == 0 it never crosses a row, and with C >= 512 the item spans at most
// two rows, so the run's row and column come from one division per workgroup
// and a wrap test.
template <int SPLIT>
__global__ __launch_bounds__(64) void k_f_apply_flat(FPlan P, FScalars S) {
  constexpr bool SR = SPLIT == PS_SPLIT_STOCHASTIC;
  uint32_t begin;
  const uint32_t wg = xcd_item<kApplyXcdChunk>(blockIdx.x, gridDim.x);
  const F2D& X = P.t2[find_end(P.item2_end, P.n2, wg, begin)];
  const uint32_t item = wg - begin;
  const float f = *X.f;
  if (!X.vec) {   // uniform per tensor
    apply_item_any<SPLIT>(X, item, S, f);
    return;
  }
  const uint32_t n = (uint32_t)X.R * (uint32_t)X.C;
  const uint32_t C = (uint32_t)X.C;
  const uint32_t elem0 = item * (uint32_t)kApplyItemElems, off = threadIdx.x * 8u;
  const uint32_t e = elem0 + off;
  const bool ok = e < n;
  uint32_t i, j;
  if (C >= (uint32_t)kApplyItemElems) {
    i = elem0 / C;
    j = elem0 - i * C + off;
    if (j >= C) {
      j -= C;
      ++i;
    }
  } else {
    i = e / C;
    j = e - i * C;
  }
  // first moment: the item's 2 blocks are the 2 DPP row pairs (32 lanes each)
  const uint32_t blk = item * 2u + (threadIdx.x >> 5);
  const bool blk_ok = blk * (uint32_t)kBlock < n;
  const float ms_old = (S.fm && blk_ok) ? X.ms[blk] : 0.0f;
  float m[8];
  float mx = 0.0f;
  for (int jj = 0; jj < 8; ++jj) m[jj] = 0.0f;
  if (ok) {
    const uint4 gv = ld_stream(X.g + e), hv = ld_stream(X.hi + e);
    const uint4 lv = SR ? make_uint4(0u, 0u, 0u, 0u) : ld_stream(X.lo + e);
    const uint4 mv = S.fm ? ld_stream(X.mc + e) : make_uint4(0u, 0u, 0u, 0u);
    float kap[8];
    load_kap8(X.kap, j, kap);
    const float rho = X.rho[i];
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
    const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
    const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
    uint32_t oh[4], ol[4];
    uint64_t rnd[2] = {0u, 0u};
    if (SR) sr_bits8(sr_stream(S.sr_seed, S.sr_step, X.tid), e, rnd);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t wb[2];
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int jj = 2 * p + o;
        const float U = (bf16_at(gw, jj) * rho) * kap[jj];
        const float w = SR ? bf16_at(hw, jj) : __uint_as_float(join_pair_elem<SPLIT>(hw[p], lw[p], o));
        float x = U * f;
        if (S.fm) {
          const float m0 = dec_signed(o ? code_hi_f(mw[p]) : code_lo_f(mw[p]), ms_old);
          x = __builtin_fmaf(S.B1, m0, S.C1 * x);
          m[jj] = x;
          mx = __builtin_fmaxf(mx, __builtin_fabsf(x));
        }
        if (S.wd) x = __builtin_fmaf(S.CWD, w, x);
        wb[o] = __float_as_uint(w - x);
      }
      if (SR) {
        const uint64_t q = rnd[p >> 1] >> (32 * (p & 1));
        oh[p] = sr_pair(wb[0], wb[1], (uint32_t)q & 0xFFFFu, (uint32_t)(q >> 16) & 0xFFFFu);
      } else {
        split_pair<SPLIT>(wb[0], wb[1], oh[p], ol[p]);
      }
    }
    st_stream(X.hi + e, make_uint4(oh[0], oh[1], oh[2], oh[3]));
    if (!SR) st_stream(X.lo + e, make_uint4(ol[0], ol[1], ol[2], ol[3]));
  }
  if (!S.fm) return;   // uniform
  float sm, inv;
  block_scale(row32_max(mx), sm, inv);
  if (ok) {
    uint32_t om[4];
    for (int p = 0; p < 4; ++p) om[p] = enc_signed(m[2 * p], inv) | (enc_signed(m[2 * p + 1], inv) << 16);
    st_stream(X.mc + e, make_uint4(om[0], om[1], om[2], om[3]));
  }
  if ((threadIdx.x & 31) == 0 && blk_ok) X.ms[blk] = sm;
}

// 1-D tensors, one 1024-element item per 64-lane workgroup (item w of the
// 1-D list): decode v, its EMA, sum of U^2. These items ride at the end of the
// U^2 launch.
__device__ __forceinline__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w) {
  uint32_t begin;
  const F1D& X = P.t1[find_end(P.item_end, P.n1, w, begin)];
  const int64_t elem0 = (int64_t)(w - begin) * kItemElems;
  const int lane = threadIdx.x, b = lane >> 4, r = lane & 15;
  const int64_t blk = (elem0 >> 8) + b;
  const float vs_old = (blk * kBlock < X.n) ? X.vs[blk] : 0.0f;
  double acc = 0.0;
  for (int half = 0; half < 2; ++half) {
    const int64_t e = elem0 + b * kBlock + half * 128 + r * 8;
    for (int j = 0; j < 8; ++j) {
      if (e + j >= X.n) break;
      const float g = __uint_as_float((uint32_t)X.g[e + j] << 16);
      const float v0 = dec_unsigned(__uint_as_float(0x4B000000u | X.vc[e + j]), vs_old);
      const float q = g * g + S.EPS1;
      const float v = __builtin_fmaf(S.B2, v0, S.C2 * q);
      X.v[e + j] = v;
      const float U = g * (1.0f / __builtin_sqrtf(v));
      acc += (double)U * (double)U;
    }
  }
  for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) X.upart[w - begin] = acc;
}

// ---- clip factor per tensor: lr / max(1, RMS(U) / clip) ---------------------
constexpr int kClipT = 1024;

__global__ __launch_bounds__(kClipT) void k_f_clip(FPlan P, FScalars S) {
  const double* parts;
  int np;
  double n;
  float* f;
  if ((int)blockIdx.x < P.n2) {
    const F2D& X = P.t2[blockIdx.x];
    parts = X.upart; np = X.npart; n = (double)X.R * (double)X.C; f = X.f;
  } else {
    const F1D& X = P.t1[blockIdx.x - P.n2];
    parts = X.upart; np = X.nitems; n = (double)X.n; f = X.f;
  }
  double s = 0.0;
#pragma unroll 8
  for (int q = threadIdx.x; q < np; q += kClipT) s += parts[q];
  __shared__ double red[kClipT];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = kClipT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double rms = sqrt(red[0] / n);
    const double r = rms / S.clip;
    *f = (float)(S.lr / (r > 1.0 ? r : 1.0));
  }
}

// ---- apply to 2-D tensors ----------------------------------------------------
template <int SPLIT>
__global__ __launch_bounds__(kT) void k_f_apply(FPlan P, FScalars S) {
  constexpr bool SR = SPLIT == PS_SPLIT_STOCHASTIC;
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.tile_nf_end, P.n2, blockIdx.x, begin)];
  const uint32_t tile = blockIdx.x - begin;
  const int tr = (int)(tile / (uint32_t)X.ntc), tc = (int)(tile - (uint32_t)tr * X.ntc);
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c = tc * kFTileCols + cg * 8;
  const float f = *X.f;
  float kap[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kap[j] = (c + j < X.C) ? X.kap[c + j] : 0.0f;
  for (int k = 0; k < 8; ++k) {
    const int r = tr * kFTileRows + rg + 8 * k;
    uint32_t gw[4], hw[4], lw[4] = {0u, 0u, 0u, 0u};
    const uint32_t valid = load_row8(X.g, X, r, c, gw);
    if (!valid) continue;
    load_row8(X.hi, X, r, c, hw);
    if (!SR) load_row8(X.lo, X, r, c, lw);
    const float rho = X.rho[r];
    const int64_t e0 = (int64_t)r * X.C + c;   // flattened index of column c
    const uint64_t srs = SR ? sr_stream(S.sr_seed, S.sr_step, X.tid) : 0u;
    uint32_t oh[4], ol[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t wb[2];
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int j = 2 * p + o;
        const float U = (bf16_at(gw, j) * rho) * kap[j];
        const float w = SR ? bf16_at(hw, j) : __uint_as_float(join_pair_elem<SPLIT>(hw[p], lw[p], o));
        float x = U * f;
        if (S.wd) x = __builtin_fmaf(S.CWD, w, x);
        wb[o] = __float_as_uint(w - x);
      }
      if (SR)
        oh[p] = sr_pair(wb[0], wb[1], sr_bits1(srs, e0 + 2 * p), sr_bits1(srs, e0 + 2 * p + 1));
      else
        split_pair<SPLIT>(wb[0], wb[1], oh[p], ol[p]);
    }
    store_row8(X.hi, X, r, c, valid, oh);
    if (!SR) store_row8(X.lo, X, r, c, valid, ol);
  }
}

// ---- apply to 1-D tensors and re-encode v --------------------------------------
// Item w of the 1-D list.
template <int SPLIT>
__device__ __forceinline__ void f1_apply_item(const FPlan& P, const FScalars& S, uint32_t w) {
  constexpr bool SR = SPLIT == PS_SPLIT_STOCHASTIC;
  uint32_t begin;
  const F1D& X = P.t1[find_end(P.item_end, P.n1, w, begin)];
  const int64_t n = X.n;
  const int64_t elem0 = (int64_t)(w - begin) * kItemElems;
  const int lane = threadIdx.x, b = lane >> 4, r = lane & 15;
  const int64_t blk = (elem0 >> 8) + b;
  const bool blk_ok = blk * kBlock < n;
  const float f = *X.f;
  const float ms_old = (S.fm && blk_ok) ? X.ms[blk] : 0.0f;
  // Runs of 8 as in the flat 2-D items (16-byte loads and stores, element by
  // element only in the tensor's last run); this step's v comes from the
  // stats item through the workspace.
  float v[16], m[16];
  float mx = 0.0f, mxm = 0.0f;
  for (int h = 0; h < 2; ++h) {
    const int64_t e = elem0 + b * kBlock + h * 128 + r * 8;
    for (int j = 0; j < 8; ++j) {
      v[8 * h + j] = 0.0f;
      m[8 * h + j] = 0.0f;
    }
    if (e >= n) continue;
    const uint4 gv = ld_run(X.g, e, n, 0u, true), hv = ld_run(X.hi, e, n, 0u, true);
    const uint4 lv = SR ? make_uint4(0u, 0u, 0u, 0u) : ld_run(X.lo, e, n, 0u, true);
    const uint4 mv = S.fm ? ld_run(X.mc, e, n, 0x80008000u, true) : make_uint4(0u, 0u, 0u, 0u);
    float vv[8];
    if (e + 8 <= n) {
      const float4 a = *reinterpret_cast<const float4*>(X.v + e), c = *reinterpret_cast<const float4*>(X.v + e + 4);
      vv[0] = a.x; vv[1] = a.y; vv[2] = a.z; vv[3] = a.w; vv[4] = c.x; vv[5] = c.y; vv[6] = c.z; vv[7] = c.w;
    } else {
      for (int j = 0; j < 8; ++j) vv[j] = (e + j < n) ? X.v[e + j] : 0.0f;
    }
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
    const uint32_t lw[4] = {lv.x, lv.y, lv.z, lv.w};
    const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
    uint64_t rnd[2] = {0u, 0u};
    if (SR) sr_bits8(sr_stream(S.sr_seed, S.sr_step, X.tid), e, rnd);
    uint32_t oh[4], ol[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t wb[2];
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int jj = 2 * p + o;
        const float wv = SR ? bf16_at(hw, jj) : __uint_as_float(join_pair_elem<SPLIT>(hw[p], lw[p], o));
        float x = 0.0f;
        if (e + jj < n) {
          const float vj = vv[jj];
          v[8 * h + jj] = vj;
          mx = __builtin_fmaxf(mx, vj);
          const float U = bf16_at(gw, jj) * (1.0f / __builtin_sqrtf(vj));
          x = U * f;
          if (S.fm) {
            const float m0 = dec_signed(o ? code_hi_f(mw[p]) : code_lo_f(mw[p]), ms_old);
            x = __builtin_fmaf(S.B1, m0, S.C1 * x);
            m[8 * h + jj] = x;
            mxm = __builtin_fmaxf(mxm, __builtin_fabsf(x));
          }
          if (S.wd) x = __builtin_fmaf(S.CWD, wv, x);
        }
        wb[o] = __float_as_uint(wv - x);
      }
      if (SR) {
        const uint64_t q = rnd[p >> 1] >> (32 * (p & 1));
        oh[p] = sr_pair(wb[0], wb[1], (uint32_t)q & 0xFFFFu, (uint32_t)(q >> 16) & 0xFFFFu);
      } else {
        split_pair<SPLIT>(wb[0], wb[1], oh[p], ol[p]);
      }
    }
    st_run(X.hi, e, n, oh);
    if (!SR) st_run(X.lo, e, n, ol);
  }
  float s, inv, sm = 0.0f, invm = 0.0f;
  block_scale(row16_max(mx), s, inv);
  if (S.fm) block_scale(row16_max(mxm), sm, invm);   // uniform
  for (int h = 0; h < 2; ++h) {
    const int64_t e = elem0 + b * kBlock + h * 128 + r * 8;
    if (e >= n) continue;
    uint32_t cv[4], cm[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      cv[p] = enc_unsigned(v[8 * h + 2 * p], inv) | (enc_unsigned(v[8 * h + 2 * p + 1], inv) << 16);
      cm[p] = S.fm ? enc_signed(m[8 * h + 2 * p], invm) | (enc_signed(m[8 * h + 2 * p + 1], invm) << 16) : 0u;
    }
    st_run(X.vc, e, n, cv);
    if (S.fm) st_run(X.mc, e, n, cm);
  }
  if (r == 0 && blk_ok) {
    X.vs[blk] = s;
    if (S.fm) X.ms[blk] = sm;
  }
}

template <int SPLIT>
__global__ __launch_bounds__(64) void k_f1_apply(FPlan P, FScalars S) {
  f1_apply_item<SPLIT>(P, S, blockIdx.x);
}

template <int SPLIT>
ps_status launch_all(const FPlan& P, const FScalars& S, hipStream_t s) {
  // U^2 row tiles, flat items without 16-byte rows and the 1-D stats items
  // share a launch (their sum is checked on the host to fit 32 bits)
  const uint32_t n_usq = P.n_rt + P.n_items2u + P.n_items;
  if (P.n_tiles) hipLaunchKernelGGL(k_f_stats, dim3(P.n_tiles), dim3(kT), 0, s, P, S);
  if (P.n_rc) hipLaunchKernelGGL(k_f_rowcol, dim3(P.n_rc), dim3(kT), 0, s, P, S);
  if (P.n_rc) hipLaunchKernelGGL(k_f_factors, dim3(P.n_rc), dim3(kT), 0, s, P);
  if (P.n_tiles_u) hipLaunchKernelGGL(k_f_usq, dim3(P.n_tiles_u), dim3(kT), 0, s, P);
  if (n_usq) hipLaunchKernelGGL(k_f_usq_flat, dim3(n_usq), dim3(64), 0, s, P, S);
  hipLaunchKernelGGL(k_f_clip, dim3(P.n2 + P.n1), dim3(kClipT), 0, s, P, S);
  if (P.n_tiles_nf) hipLaunchKernelGGL((k_f_apply<SPLIT>), dim3(P.n_tiles_nf), dim3(kT), 0, s, P, S);
  if (P.n_items2) hipLaunchKernelGGL((k_f_apply_flat<SPLIT>), dim3(P.n_items2), dim3(64), 0, s, P, S);
  if (P.n_items) hipLaunchKernelGGL((k_f1_apply<SPLIT>), dim3(P.n_items), dim3(64), 0, s, P, S);
  return hip_check(hipGetLastError(), "factored step launch");
}

}  // namespace

ps_status launch_factored(const FPlan& plan, const FScalars& sc, int split_mode, hipStream_t s) {
  if (split_mode == PS_SPLIT_NEAREST_AWAY) return launch_all<PS_SPLIT_NEAREST_AWAY>(plan, sc, s);
  if (split_mode == PS_SPLIT_STOCHASTIC) return launch_all<PS_SPLIT_STOCHASTIC>(plan, sc, s);
  return launch_all<PS_SPLIT_TRUNC>(plan, sc, s);
}

}  // namespace ps
