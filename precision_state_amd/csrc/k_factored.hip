// k_factored.hip - Adafactor-style step: factored second moment (row/column
// EMAs of mean g^2 + eps1, constant beta2 or the 1 - t^decay_rate schedule),
// update clipping by the tensor's RMS, optional first moment (EMA of the
// clipped update in the signed codec), decoupled weight decay, residual split
// [ADAF, adafactor_step_param; PRODIGY, beta1 = 0 / factored / update
// clipping].
//
// Passes: statistics (row and column sums of q = g^2 + eps1, in double);
// row/column finalize (EMAs, chunk sums of the new row EMA); factors
// rho_i = 1/sqrt(r_i / rbar), kap_j = 1/sqrt(c_j); the sum of U^2 over each
// tensor; clip factor per tensor; apply, with the fp32 U = (g * rho_i) * kap_j.
// The RMS behind the clip is evaluated in double from the factored estimate,
// U_ij^2 = g_ij^2 * rbar / (r_i c_j) (1-D: g^2 / v).
//  - Tensors whose rows are whole multiples of 512 columns (up to 12288) take
//    the row-strip statistics pass, which also sums g^2 / r_i per column, so
//    the gradient is read twice per step (statistics, apply).
//  - Others take 64 x 256 statistics tiles (thread t: columns (t % 32) * 8 ..
//    + 8 of rows t / 32 + 8k, so each half-wave reads one 512-byte row segment
//    per load) and a pass of their own for the sum of U^2: three reads.
// 1-D tensors keep v in the uint16 codec and use 1024-element items.
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

// Direct-to-LDS gradient copies of the row-strip pass: lane i's 16 bytes land
// at dst + 16 i (dst wave-uniform); cache-policy bit 1 marks them non-temporal.
constexpr int kLdsDmaNt = 2;
typedef __attribute__((address_space(3))) void lds_void;

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

// ---- pass 1, row strips: row sums, row EMA, column sums of q and of g^2 / r_i
// Tensors with C % 512 == 0 and C <= kStripMaxC. The sum of U^2 needs no
// pass of its own: U_ij^2 = g_ij^2 * rbar / (r_i c_j), so
//   sum_ij U_ij^2 = rbar * sum_j Q_j / c_j,   Q_j = sum_i g_ij^2 / r_i,
// and r_i, the new row EMA, is known as soon as row i has been read. So a
// workgroup takes whole rows: a group of rows (the host cuts the strip
// tensors' rows into groups of equal element counts, one per workgroup),
// walked in steps of `grows` rows (one row when a row has more 16-byte runs
// than the workgroup has threads). Thread t owns the runs u0 = t mod Ur (and,
// for rows of more than kSNT runs, u0 + kSNT) of row t / Ur of a step, so its
// 8 (or 16) column sums stay in registers for the whole group.
// The gradient goes straight to LDS (global_load_lds, 16 bytes per lane, each
// thread later reading back only its own entries) in batches of 48 KiB, three
// buffers deep: two batches stay in flight while one is summed, and the
// prefetch costs no registers. One barrier per batch publishes each wave's row
// partials (a wave lies within one row because Ur % 64 == 0); lane d of every
// wave then adds the partials of step d's row in a fixed pairwise order and
// forms that row's EMA from the same double sum the finalize kernel uses (the
// sum it stores), with the same correctly rounded mean. Column sums of
// q and of g^2 / r_i are in double; the threads of a step that share columns
// add theirs in row order through LDS at the end of the group.

// Barrier for LDS data only: this wave's LDS accesses complete, gradient
// loads stay in flight. The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave sums of D doubles by transpose-reduce, lane exchanges only (no LDS):
// lane l ends with the sum over the 64 lanes of v[k], k = l >> (6 - log2 D),
// in a fixed order. v_permlane32_swap / v_permlane16_swap hand each half (row
// pair) the other's values, and an exchange of two different values leaves
// each half the sum of one of them; the last four lane bits are folded by DPP
// within each row of 16 (every lane of the row ends with the row's sum).
__device__ __forceinline__ uint32_t lo32(double x) { return (uint32_t)__double_as_longlong(x); }
__device__ __forceinline__ uint32_t hi32(double x) { return (uint32_t)((uint64_t)__double_as_longlong(x) >> 32); }
__device__ __forceinline__ double mk64(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// lanes 0..31: a + a of lane + 32; lanes 32..63: b of lane - 32 + b
__device__ __forceinline__ double swap32_sum(double a, double b) {
  const auto l = __builtin_amdgcn_permlane32_swap(lo32(a), lo32(b), false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi32(a), hi32(b), false, false);
  return mk64(l[0], h[0]) + mk64(l[1], h[1]);
}
// even rows of 16: a + a of the next row; odd rows: b of the previous row + b
__device__ __forceinline__ double swap16_sum(double a, double b) {
  const auto l = __builtin_amdgcn_permlane16_swap(lo32(a), lo32(b), false, false);
  const auto h = __builtin_amdgcn_permlane16_swap(hi32(a), hi32(b), false, false);
  return mk64(l[0], h[0]) + mk64(l[1], h[1]);
}
// A plain DPP move (no old value: every source lane of these row-local
// patterns exists, so nothing needs initialising before the move).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  return mk64((uint32_t)__builtin_amdgcn_mov_dpp((int)lo32(x), CTRL, 0xF, 0xF, true),
              (uint32_t)__builtin_amdgcn_mov_dpp((int)hi32(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ double row16_sum(double x) {
  x += dpp_f64<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_f64<0x141>(x);   // row_half_mirror
  x += dpp_f64<0x140>(x);   // row_mirror
  return x;
}
template <int D>
__device__ __forceinline__ double wave_sums(const double* v) {
  if constexpr (D == 4) {
    const double a0 = swap32_sum(v[0], v[2]), a1 = swap32_sum(v[1], v[3]);   // index 2 b5 + {0, 1}
    return row16_sum(swap16_sum(a0, a1));                                     // index 2 b5 + b4
  } else {
    static_assert(D == 2, "D is 2 or 4");
    const double a = swap32_sum(v[0], v[1]);   // index b5
    return row16_sum(swap16_sum(a, a));
  }
}

// Register pinning: an empty asm statement that reads and rewrites x. Placed
// after each 16-byte run, it keeps the compiler from interleaving the
// double-precision work of many runs (which needed more registers than three
// waves per SIMD leave, and the spill reloads then waited on the gradient
// loads in flight).
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

constexpr int kSWaves = kSNT / 64;
constexpr int kSBufRuns = 4 * kSNT;    // 16-byte runs per LDS batch buffer (48 KiB)
constexpr int kSBufBytes = kSBufRuns * 16;

// LDS reads of the batch buffers, in asm: the compiler cannot tell the
// batch being summed from those still being filled and would wait for every
// copy in flight before any LDS read of them; after the explicit wait for the
// batch at hand, the newer ones stay in flight. Each asm statement waits for
// its own results.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// The four runs (D * K) of this thread in a batch buffer, entry (d * K + k)
// at byte offset (d * K + k) * kSNT * 16 from the thread's first at a, and
// the 4-byte word at b (a row EMA copied in with them).
__device__ __forceinline__ void lds_read_runs(uint32_t a, uint32_t b, u32x4 (&x)[4], float& w) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:12288\n\t"
      "ds_read_b128 %2, %5 offset:24576\n\t"
      "ds_read_b128 %3, %5 offset:36864\n\t"
      "ds_read_b32 %4, %6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(w)   // early clobber: the addresses
      : "v"(a), "v"(b)                                                  // outlive the first result
      : "memory");
}
static_assert(kSNT * 16 == 12288, "the offsets in lds_read_runs");

// Three batch buffers; a segment's column sums of the rows after the first of
// a step pass through the first two at the end (at most kSNT - 64 threads x
// 16 doubles = 90112 bytes). s_ro holds the old row EMA of each wave's row of
// each step of a batch, s_wsum the wave row partials by batch parity.
__shared__ u32x4 s_buf[3 * kSBufRuns];   // buffer h at s_buf + h * kSBufRuns
__shared__ float s_ro[3][4][kSWaves];
__shared__ double s_wsum[2][4][kSWaves];

__device__ __forceinline__ double* comb_entry(int e) {   // 16 doubles (8 runs) per entry
  return (double*)&s_buf[8 * e];
}
static_assert((kSNT - 64) * 8 <= 2 * kSBufRuns, "the column sums fit two buffers");

// What a segment needs of its tensor and the scalars, held in registers: the
// asm statements' memory clobbers would otherwise make the compiler reload
// the tensor record (and wait for every load in flight) inside the loop.
struct StripArgs {
  const GLOBAL uint16_t* g;
  const GLOBAL float* row;
  GLOBAL double* rowpart;
  GLOBAL double* colpart;
  GLOBAL double* qpart;
  int C, row0, row1, slot;
  float EPS1, B2, C2;
};

template <int K, int D>
__device__ __forceinline__ void strip_segment(const StripArgs& A, int& par) {
  static_assert(D * K * kSNT == kSBufRuns && D * K == 4, "a batch fills one LDS buffer");
  constexpr int OPS = D * K + D;   // vector memory operations per batch and wave
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int C = A.C, Ur = C >> 3;
  int grows, rr, u0, nwr, w0;
  if (K == 1) {
    grows = kSNT / Ur;
    rr = __builtin_amdgcn_readfirstlane(t / Ur);   // wave-uniform (Ur % 64 == 0)
    u0 = t - rr * Ur;
    nwr = Ur >> 6;
    w0 = rr * nwr;
  } else {
    grows = 1;
    rr = 0;
    u0 = t;
    nwr = kSWaves;
    w0 = 0;
  }
  const bool act = rr < grows;                       // wave-uniform
  const bool run1 = K == 2 && u0 + kSNT < Ur;        // the second run exists
  const int row0 = A.row0, row1 = A.row1;
  const double Cd = (double)C, rC = 1.0 / Cd;
  const int nsteps = (row1 - row0 + grows - 1) / grows;
  const int nb = (nsteps + D - 1) / D;
  double P[K][8], Q[K][8];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) P[k][j] = Q[k][j] = 0.0;

  auto row_of = [&](int b, int d) { return row0 + (b * D + d) * grows + rr; };
  // Every wave issues exactly D * K gradient copies and D row-EMA copies per
  // batch, with addresses clamped into the segment (data of rows past the
  // segment, of idle threads and of missing second runs are loaded and not
  // used), so that vmcnt(n * OPS) waits for all but the n newest batches.
  auto issue = [&](int b) {
    const int h = b % 3;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = min(row_of(b, d), row1 - 1);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int u = (k == 1 && run1) ? u0 + kSNT : u0;
        __builtin_amdgcn_global_load_lds((const GLOBAL void*)(A.g + (size_t)i * (size_t)C + (size_t)(8 * u)),
                                         (lds_void*)&s_buf[h * kSBufRuns + (d * K + k) * kSNT + wave * 64], 16, 0, kLdsDmaNt);
      }
      if (lane == 0)
        __builtin_amdgcn_global_load_lds((const GLOBAL void*)(A.row + i), (lds_void*)&s_ro[h][d][wave], 4, 0, 0);
    }
    asm volatile("" ::: "memory");
  };

  if (nb > 0) issue(0);
  if (nb > 1) issue(1);
  for (int b = 0; b < nb; ++b) {
    if (b + 2 < nb) issue(b + 2);
    const int newer = min(nb - 1 - b, 2);   // batches issued after this one
    if (newer == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * OPS) : "memory");
    else if (newer == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int h = b % 3;
    const uint32_t abuf = lds_addr(&s_buf[h * kSBufRuns + t]);

    // g^2 (exact in fp32 for a bf16 g) and q = g^2 + eps1 into the column
    // sums and this lane's row partials; g^2 stays in registers for the
    // second half. Lane d < D also takes step d's old row EMA (this wave's
    // own copy, so it is read here, ahead of the barrier).
    u32x4 x[4];
    float ro;
    lds_read_runs(abuf, lds_addr(&s_ro[h][min(lane, D - 1)][wave]), x, ro);
    float g2[D][K][8];
    double rp[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      rp[d] = 0.0;
      const bool ok = act && row_of(b, d) < row1;   // wave-uniform
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t w[4] = {x[d * K + k].x, x[d * K + k].y, x[d * K + k].z, x[d * K + k].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float g = bf16_at(w, j);
          g2[d][k][j] = g * g;
        }
        if (!ok) continue;
        double sq;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double q = (double)(g2[d][k][j] + A.EPS1);
          P[k][j] += q;
          sq = j ? sq + q : q;
        }
        if (k == 0)
          rp[d] = sq;
        else
          rp[d] += run1 ? sq : 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) pin(P[k][j]);
        pin(rp[d]);
      }
    }
    const double ws = wave_sums<D>(rp);
    if ((lane & (64 / D - 1)) == 0) s_wsum[par][lane / (64 / D)][wave] = ws;
    lds_barrier();

    // lane d: step d's row sum (the nwr <= 12 wave partials added pairwise
    // in a fixed order, missing ones as 0), the new row EMA (as the finalize
    // kernel forms it) and 1 / r_i. Every wave runs this chain right after
    // the barrier with nothing to overlap it, so it is kept short:
    //  - sum / C as Markstein's corrected product: with y = RN(1/C), for
    //    every C = m * 512, m <= 24, y is within 2^-54 of 1/C relatively,
    //    so q0 = RN(sum * y) is within one ulp of sum / C and
    //    RN(q0 + (sum - C q0) y) is the correctly rounded quotient, the
    //    value of an IEEE division; an infinite sum leaves a NaN residual
    //    and keeps q0 (infinity);
    //  - 1 / r_i: the reciprocal estimate and one third-order Newton step,
    //    y (1 + e + e^2) with e = 1 - r y.
    double inv_l = 0.0;
    if (lane < D) {
      const int i = row_of(b, lane);
      double a[kSWaves];
#pragma unroll
      for (int q = 0; q < kSWaves; ++q) a[q] = q < nwr ? s_wsum[par][lane][min(w0 + q, kSWaves - 1)] : 0.0;
      static_assert(kSWaves == 12, "the pairwise order below");
      const double sum = (((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]))) +
                         ((a[8] + a[9]) + (a[10] + a[11]));
      const double q0 = sum * rC;
      const double res = __builtin_fma(-Cd, q0, sum);
      const double qc = __builtin_fma(res, rC, q0);
      const float mean = (float)(res == res ? qc : q0);
      const double r = (double)__builtin_fmaf(A.B2, ro, A.C2 * mean);
      const double y = __builtin_amdgcn_rcp(r);
      const double e = __builtin_fma(-r, y, 1.0);
      inv_l = __builtin_fma(y, __builtin_fma(e, e, e), y);
      if (act && i < row1 && wave == w0) A.rowpart[i] = sum;
    }
    // then g^2 / r_i into the column sums
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (!(act && row_of(b, d) < row1)) continue;   // wave-uniform
      const double inv = mk64(__builtin_amdgcn_readlane(lo32(inv_l), d), __builtin_amdgcn_readlane(hi32(inv_l), d));
#pragma unroll
      for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int j = 0; j < 8; ++j) Q[k][j] = __builtin_fma((double)g2[d][k][j], inv, Q[k][j]);
#pragma unroll
        for (int j = 0; j < 8; ++j) pin(Q[k][j]);
      }
    }
    par ^= 1;
  }

  // Threads of a step that share columns (K == 1, grows > 1): rows after the
  // first deposit their sums, the first row's threads add them in row order.
  // The first barrier also ends every wave's reads of the batch buffers.
  if (K == 1 && grows > 1) {   // uniform
    lds_barrier();
    if (act && rr > 0) {
      double* c = comb_entry((rr - 1) * Ur + u0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        c[j] = P[0][j];
        c[8 + j] = Q[0][j];
      }
    }
    lds_barrier();
    if (rr == 0) {
      for (int q = 1; q < grows; ++q) {
        const double* c = comb_entry((q - 1) * Ur + u0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          P[0][j] += c[j];
          Q[0][j] += c[8 + j];
        }
      }
    }
  }
  // the buffers are free again for the next segment's first batches
  lds_barrier();
  if (rr == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k == 1 && !run1) continue;
      const size_t o = (size_t)A.slot * (size_t)C + (size_t)(8 * (u0 + k * kSNT));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        A.colpart[o + j] = P[k][j];
        A.qpart[o + j] = Q[k][j];
      }
    }
  }
}

// Wave-uniform copies in scalar registers: read once, before the first
// gradient copies are issued, so no later use waits on the copies in flight.
template <class T>
__device__ __forceinline__ GLOBAL T* uni(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (GLOBAL T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__global__ __launch_bounds__(kSNT) void k_f_strip(FPlan P, FScalars S) {
  const uint32_t g = blockIdx.x;
  const uint32_t s0 = g ? P.seg_end[g - 1] : 0u, s1 = P.seg_end[g];
  int par = 0;
  for (uint32_t s = s0; s < s1; ++s) {
    const FSeg sg = P.segs[s];
    const F2D& X = P.t2[sg.t];
    const StripArgs A{uni(X.g), uni(X.row), uni(X.rowpart), uni(X.colpart), uni(X.qpart), uni(X.C),
                      uni(sg.row0), uni(sg.row1), uni(sg.slot), S.EPS1, S.B2, S.C2};
    if ((A.C >> 3) <= kSNT)   // uniform
      strip_segment<1, 4>(A, par);
    else
      strip_segment<2, 2>(A, par);
  }
}

// ---- pass 2: row/column EMAs and chunk sums of the new row EMA -------------
__device__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w, int lane);

// Workgroups past the finalize ones (launched only when no U^2 pass runs)
// take the 1-D tensors' stats items, one per wave.
__global__ __launch_bounds__(kT) void k_f_rowcol(FPlan P, FScalars S) {
  if (blockIdx.x >= P.n_rc) {   // uniform
    const uint32_t w = (blockIdx.x - P.n_rc) * (uint32_t)(kT / 64) + (threadIdx.x >> 6);
    if (w < P.n_items) f1_stats_item(P, S, w, (int)(threadIdx.x & 63));
    return;
  }
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
      for (int tc = 0; tc < X.nrp; ++tc) s += X.rowpart[(size_t)tc * X.R + i];
      const float mean = (float)(s / (double)X.C);
      const float r = __builtin_fmaf(S.B2, X.row[i], S.C2 * mean);
      X.row[i] = r;
      rv = (double)r;
    }
    const double t = block_sum(rv, red);
    if (threadIdx.x == 0) X.rpart[w] = t;
  } else {
    const int j = (w - X.nrw) * kFRowColChunk + (int)threadIdx.x;
    double qc = 0.0;
    if (j < X.C) {
      double s = 0.0;
#pragma unroll 16
      for (int tr = 0; tr < X.sntr; ++tr) s += X.colpart[(size_t)tr * X.C + j];
      const float mean = (float)(s / (double)X.R);
      const float c = __builtin_fmaf(S.B2, X.col[j], S.C2 * mean);
      X.col[j] = c;
      if (X.strip) {   // uniform
        double qs = 0.0;
#pragma unroll 16
        for (int tr = 0; tr < X.sntr; ++tr) qs += X.qpart[(size_t)tr * X.C + j];
        qc = qs / (double)c;
      }
    }
    if (X.strip) {   // uniform: this chunk's sum_j Q_j / c_j
      const double t = block_sum(qc, red);
      if (threadIdx.x == 0) X.upart[w - X.nrw] = t;
    }
  }
}

// ---- pass 3: factors of V^-1/2 ----------------------------------------------
template <int NT>
__device__ void clip_one(const FPlan& P, const FScalars& S, int idx, double* red);

// Sum of a 2-D tensor's row-chunk sums rpart[0 .. nrw) (mean(r)'s numerator)
// in an order that does not depend on the block size NT >= kT: thread t < kT
// adds chunks t, t + kT, ... in turn, then a tree over the kT partials. The
// factors and the clip factor both take mean(r) from it, so they agree bit
// for bit, and a tall tensor costs each block nrw / kT loads, not nrw. Every
// thread of the block must call it; all get the sum.
template <int NT>
__device__ __forceinline__ double rpart_sum(const F2D& X, double* red) {
  static_assert(NT >= kT, "one partial per thread of the first kT");
  if ((int)threadIdx.x < kT) {
    double s = 0.0;
    for (int q = (int)threadIdx.x; q < X.nrw; q += kT) s += X.rpart[q];
    red[threadIdx.x] = s;
  }
  __syncthreads();
  for (int o = kT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Workgroups past the factor ones (launched only when no U^2 pass runs, so
// every sum of U^2 is complete after the finalize launch) take the clip
// factors, one tensor each.
__global__ __launch_bounds__(kT) void k_f_factors(FPlan P, FScalars S) {
  __shared__ double red[kT];
  if (blockIdx.x >= P.n_rc) {   // uniform
    clip_one<kT>(P, S, (int)(blockIdx.x - P.n_rc), red);
    return;
  }
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.rc_end, P.n2, blockIdx.x, begin)];
  const int w = (int)(blockIdx.x - begin);
  if (w < X.nrw) {   // uniform
    const float rbar = (float)(rpart_sum<kT>(X, red) / (double)X.R);
    const int i = w * kFRowColChunk + (int)threadIdx.x;
    if (i < X.R) {
      X.rho[i] = 1.0f / __builtin_sqrtf(X.row[i] / rbar);
      if (X.rinv) X.rinv[i] = 1.0 / (double)X.row[i];
    }
  } else {
    const int j = (w - X.nrw) * kFRowColChunk + (int)threadIdx.x;
    if (j < X.C) {
      X.kap[j] = 1.0f / __builtin_sqrtf(X.col[j]);
      if (X.cinv) X.cinv[j] = 1.0 / (double)X.col[j];
    }
  }
}

// ---- pass 4: sums of U^2 / mean(r) = g^2 / (r_i c_j), in double, for the
// tensors that do not take the row-strip pass; this per tile (rows that are
// not 16-byte runs, no first moment) -----------------------------------------
__global__ __launch_bounds__(kT) void k_f_usq(FPlan P) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.tile_u_end, P.n2, blockIdx.x, begin)];
  const uint32_t tile = blockIdx.x - begin;
  const int tr = (int)(tile / (uint32_t)X.ntc), tc = (int)(tile - (uint32_t)tr * X.ntc);
  const int cg = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c = tc * kFTileCols + cg * 8;
  double ci[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ci[j] = (c + j < X.C) ? X.cinv[c + j] : 0.0;
  double acc = 0.0;
  for (int k = 0; k < 8; ++k) {
    const int r = tr * kFTileRows + rg + 8 * k;
    uint32_t w[4];
    const uint32_t valid = load_row8(X.g, X, r, c, w);
    if (!valid) continue;
    double sr = 0.0;   // sum_j g^2 / c_j over the row segment (g^2 exact in fp32), then times 1 / r_i
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float g = bf16_at(w, j);
      sr = (valid >> j & 1u) ? __builtin_fma((double)(g * g), ci[j], sr) : sr;
    }
    acc = __builtin_fma(sr, X.rinv[r], acc);
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

// Sum of g^2 / (r_i c_j) over one item, any column count (same per-lane order
// as the run path).
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
      const uint32_t i = (e + jj) / (uint32_t)X.C;
      const double g = (double)bf16_at(w, jj);
      acc += g * g * X.rinv[i] * X.cinv[e + jj - i * (uint32_t)X.C];
    }
  }
  for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (threadIdx.x == 0) X.upart[item] = acc;
}

__device__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w, int lane);

// Sum of g^2 / (r_i c_j) over one row tile of a tensor whose rows are 16-byte
// runs (and that does not take the row-strip pass): kURows rows x kUCols
// columns, lane l taking columns c .. c+7 (c = band start + 8 l) of every row
// of the tile. The lane loads its 8 column factors once and all its rows'
// gradient runs at once (8 KiB per wave in flight), and each row's factor is
// one scalar load. Lane order: row by row, columns in order; then the wave's
// xor tree. Lanes past the last column and rows past the last row hold g = 0
// and add exact zeros.
__device__ __forceinline__ void usq_row_tile(const FPlan& P, uint32_t w) {
  uint32_t begin;
  const F2D& X = P.t2[find_end(P.rt_end, P.n2, w, begin)];
  const uint32_t t = w - begin;
  const int tr = (int)(t / (uint32_t)X.nuc), tc = (int)(t - (uint32_t)tr * X.nuc);
  const int c = tc * kUCols + (int)threadIdx.x * 8;
  const int r0 = tr * kURows;
  const bool col_ok = c < X.C;
  double ci[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ci[j] = col_ok ? X.cinv[c + j] : 0.0;
  uint4 gv[kURows];
#pragma unroll
  for (int k = 0; k < kURows; ++k) {
    const int r = r0 + k;
    gv[k] = (col_ok && r < X.R) ? ld_stream(X.g + (size_t)r * (size_t)X.C + (size_t)c) : make_uint4(0u, 0u, 0u, 0u);
  }
  // per row: sum_j g^2 / c_j (g^2 exact in fp32), then times 1 / r_i
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < kURows; ++k) {
    const int r = r0 + k;
    const double ri = r < X.R ? X.rinv[r] : 0.0;
    const uint32_t g[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
    double sr = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gj = bf16_at(g, j);
      sr = __builtin_fma((double)(gj * gj), ci[j], sr);
    }
    acc = __builtin_fma(sr, ri, acc);
  }
  for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (threadIdx.x == 0) X.upart[t] = acc;
}

__device__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w, int lane);

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
    f1_stats_item(P, S, w2 - P.n_items2u, (int)threadIdx.x);
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

// 1-D tensors, one 1024-element item per 64-lane wave (item w of the 1-D
// list): decode v, its EMA, sum of U^2. These items ride at the end of the
// finalize launch, or of the U^2 launch when one runs.
__device__ __forceinline__ void f1_stats_item(const FPlan& P, const FScalars& S, uint32_t w, int lane) {
  uint32_t begin;
  const F1D& X = P.t1[find_end(P.item_end, P.n1, w, begin)];
  const int64_t elem0 = (int64_t)(w - begin) * kItemElems;
  const int b = lane >> 4, r = lane & 15;
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
      acc += (double)g * (double)g / (double)v;   // U^2 = g^2 / v in double
    }
  }
  for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) X.upart[w - begin] = acc;
}

// ---- clip factor per tensor: lr / max(1, RMS(U) / clip) ---------------------
// Tensor `idx` of the 2-D list followed by the 1-D list, NT threads.
template <int NT>
__device__ __forceinline__ void clip_one(const FPlan& P, const FScalars& S, int idx, double* red) {
  const double* parts;
  int np;
  double n;
  float* f;
  double scale = 1.0;   // 2-D: parts are sums of g^2 / (r_i c_j); times mean(r)
  if (idx < P.n2) {
    const F2D& X = P.t2[idx];
    parts = X.upart; np = X.npart; n = (double)X.R * (double)X.C; f = X.f;
    scale = rpart_sum<NT>(X, red) / (double)X.R;
  } else {
    const F1D& X = P.t1[idx - P.n2];
    parts = X.upart; np = X.nitems; n = (double)X.n; f = X.f;
  }
  double s = 0.0;
#pragma unroll 8
  for (int q = threadIdx.x; q < np; q += NT) s += parts[q];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double rms = sqrt(red[0] * scale / n);
    const double r = rms / S.clip;
    *f = (float)(S.lr / (r > 1.0 ? r : 1.0));
  }
}

constexpr int kClipT = 1024;

__global__ __launch_bounds__(kClipT) void k_f_clip(FPlan P, FScalars S) {
  __shared__ double red[kClipT];
  clip_one<kClipT>(P, S, (int)blockIdx.x, red);
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
  if (P.n_groups) hipLaunchKernelGGL(k_f_strip, dim3(P.n_groups), dim3(kSNT), 0, s, P, S);
  if (P.n_tiles) hipLaunchKernelGGL(k_f_stats, dim3(P.n_tiles), dim3(kT), 0, s, P, S);
  if (P.n_tiles == 0 && P.n_rt == 0 && P.n_items2u == 0 && P.n_tiles_u == 0) {
    // No U^2 pass (every 2-D tensor took the row-strip pass): the 1-D stats
    // items ride with the finalize launch and the clip factors with the
    // factor launch.
    const uint32_t n1wg = (P.n_items + kT / 64 - 1) / (kT / 64);
    if (P.n_rc + n1wg) hipLaunchKernelGGL(k_f_rowcol, dim3(P.n_rc + n1wg), dim3(kT), 0, s, P, S);
    hipLaunchKernelGGL(k_f_factors, dim3(P.n_rc + P.n2 + P.n1), dim3(kT), 0, s, P, S);
  } else {
    const uint32_t n_usq = P.n_rt + P.n_items2u + P.n_items;
    if (P.n_rc) hipLaunchKernelGGL(k_f_rowcol, dim3(P.n_rc), dim3(kT), 0, s, P, S);
    if (P.n_rc) hipLaunchKernelGGL(k_f_factors, dim3(P.n_rc), dim3(kT), 0, s, P, S);
    if (P.n_tiles_u) hipLaunchKernelGGL(k_f_usq, dim3(P.n_tiles_u), dim3(kT), 0, s, P);
    if (n_usq) hipLaunchKernelGGL(k_f_usq_flat, dim3(n_usq), dim3(64), 0, s, P, S);
    hipLaunchKernelGGL(k_f_clip, dim3(P.n2 + P.n1), dim3(kClipT), 0, s, P, S);
  }
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
