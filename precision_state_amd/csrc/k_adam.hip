// k_adam.hip - fused multi-tensor (N)AdamW step on residual-split bf16
// weights with uint16-coded moments [NADAM; KAHAN].
//
// Mapping (gfx950, wave64): the tensor list is cut into work items of 1024
// elements (4 moment blocks) that never cross a tensor boundary. A work item
// belongs to one wave; a 256-element block belongs to 16 lanes (one DPP row),
// and each lane holds 16 elements: two runs of 8 at offsets r*8 and 128 + r*8
// of its block, so each of the wave's 16-byte loads covers whole 128-byte
// lines. Each work item is one 64-lane workgroup.
//
// Per element the kernel reads hi, lo, grad, m_code, v_code (10 bytes) and
// writes hi, lo, m_code, v_code (8 bytes); per block it reads and writes the
// two scales (16 bytes).
#include "dev_common.h"
#include "ps_internal.h"

namespace ps {
namespace {

struct Regs {       // one lane's 16 elements, 16-bit streams as packed pairs
  uint32_t h[8], l[8], g[8], mc[8], vc[8];
};

__device__ __forceinline__ void load8(const uint16_t* p, uint32_t* dst) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const uint32_t* src) {
  *reinterpret_cast<uint4*>(p) = make_uint4(src[0], src[1], src[2], src[3]);
}

// Guarded variants for the last work item of a tensor: element e + j exists
// when e + j < n; missing elements read as `fill` and are not written.
__device__ __forceinline__ void load8_guard(const uint16_t* p, int64_t e, int64_t n, uint32_t fill, uint32_t* dst) {
  if (e + 8 <= n) {
    load8(p + e, dst);
    return;
  }
  for (int j = 0; j < 4; ++j) {
    uint32_t lo = (e + 2 * j < n) ? p[e + 2 * j] : (fill & 0xFFFFu);
    uint32_t hi = (e + 2 * j + 1 < n) ? p[e + 2 * j + 1] : (fill >> 16);
    dst[j] = lo | (hi << 16);
  }
}

__device__ __forceinline__ void store8_guard(uint16_t* p, int64_t e, int64_t n, const uint32_t* src) {
  if (e + 8 <= n) {
    store8(p + e, src);
    return;
  }
  for (int j = 0; j < 8; ++j)
    if (e + j < n) p[e + j] = (uint16_t)(src[j >> 1] >> (16 * (j & 1)));
}

template <int ALGO, bool WD, int SPLIT>
__device__ __forceinline__ void process_item(const DevTensor& T, int64_t elem0, int lane, const StepScalars& c) {
  const int b = lane >> 4;                 // block of the item, 0..3
  const int r = lane & 15;                 // lane within the block's DPP row
  const int64_t n = T.numel;
  const int64_t blk = (elem0 >> 8) + b;    // block index within the tensor
  const int64_t ea = elem0 + b * kBlock + r * 8;
  const int64_t eb = ea + 128;
  const bool full = elem0 + kItemElems <= n;  // uniform per wave

  Regs R;
  float ms_old = 0.0f, vs_old = 0.0f;
  // Full items: uniform base pointers plus 32-bit lane offsets.
  const uint32_t la = (uint32_t)(b * kBlock + r * 8), lb = la + 128;
  if (full) {
    const uint16_t* ph = T.hi + elem0;
    const uint16_t* pl = T.lo + elem0;
    const uint16_t* pg = T.g + elem0;
    const uint16_t* pm = T.mc + elem0;
    const uint16_t* pv = T.vc + elem0;
    load8(ph + la, R.h); load8(ph + lb, R.h + 4);
    load8(pl + la, R.l); load8(pl + lb, R.l + 4);
    load8(pg + la, R.g); load8(pg + lb, R.g + 4);
    load8(pm + la, R.mc); load8(pm + lb, R.mc + 4);
    load8(pv + la, R.vc); load8(pv + lb, R.vc + 4);
    ms_old = T.ms[blk];
    vs_old = T.vs[blk];
  } else {
    load8_guard(T.hi, ea, n, 0u, R.h); load8_guard(T.hi, eb, n, 0u, R.h + 4);
    load8_guard(T.lo, ea, n, 0u, R.l); load8_guard(T.lo, eb, n, 0u, R.l + 4);
    load8_guard(T.g, ea, n, 0u, R.g); load8_guard(T.g, eb, n, 0u, R.g + 4);
    load8_guard(T.mc, ea, n, 0x80008000u, R.mc); load8_guard(T.mc, eb, n, 0x80008000u, R.mc + 4);
    load8_guard(T.vc, ea, n, 0u, R.vc); load8_guard(T.vc, eb, n, 0u, R.vc + 4);
    if (blk * kBlock < n) {
      ms_old = T.ms[blk];
      vs_old = T.vs[blk];
    }
  }

  // Phase 1: decode, EMA, block maxima. Missing tail elements have g = 0 and
  // zero-coded moments, so m = v = 0 and they never raise a maximum.
  float m[16], v[16];
  float mx_m = 0.0f, mx_v = 0.0f;
  uint32_t tiny = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int w = j >> 1;
    const bool odd = j & 1;
    float g = odd ? bf16_hi(R.g[w]) : bf16_lo(R.g[w]);
    float m0 = dec_signed(odd ? code_hi_f(R.mc[w]) : code_lo_f(R.mc[w]), ms_old);
    float v0 = dec_unsigned(odd ? code_hi_f(R.vc[w]) : code_lo_f(R.vc[w]), vs_old);
    m[j] = __builtin_fmaf(c.B1, m0, c.C1 * g);
    v[j] = __builtin_fmaf(c.B2, v0, c.C2 * (g * g));
    mx_m = __builtin_fmaxf(mx_m, __builtin_fabsf(m[j]));
    mx_v = __builtin_fmaxf(mx_v, v[j]);
    tiny = __builtin_elementwise_min(tiny, __float_as_uint(v[j]) - 1u);
  }
  // 0 < v < 2^-96 anywhere in the wave: the fast square root's residual test
  // could underflow there, so the whole wave takes the library sequence.
  const bool slow_sqrt = __builtin_amdgcn_ballot_w64(tiny < 0x0F7FFFFFu) != 0;

  // Phase 2: block scales (row-wide max over the 16 lanes).
  float sm, inv_m, sv, inv_v;
  block_scale(row16_max(mx_m), sm, inv_m);
  block_scale(row16_max(mx_v), sv, inv_v);
  const float sq_inv_v = fast_sqrt(inv_v);

  // Phase 3: update, split, encode.
  uint32_t oh[8], ol[8], omc[8], ovc[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t wb[2], cm[2], cv[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int j = 2 * w + o;
      float g = o ? bf16_hi(R.g[w]) : bf16_lo(R.g[w]);
      float wf = __uint_as_float(join_pair_elem<SPLIT>(R.h[w], R.l[w], o));
      float rv = slow_sqrt ? __builtin_sqrtf(v[j]) : sqrt_rn_fast(v[j]);
      float d = __builtin_fmaf(rv, c.RS2, c.EPS);
      float u;
      if (ALGO == PS_ALGO_ADAM)
        u = c.A * (m[j] / d);
      else
        u = __builtin_fmaf(c.AG, g, c.AM * m[j]) / d;
      if (WD) u = __builtin_fmaf(c.CWD, wf, u);
      wb[o] = __float_as_uint(wf - u);
      cm[o] = enc_signed(m[j], inv_m);
      cv[o] = enc_unsigned_y(v[j], inv_v, fast_sqrt(rv * sq_inv_v));
    }
    split_pair<SPLIT>(wb[0], wb[1], oh[w], ol[w]);
    omc[w] = cm[0] | (cm[1] << 16);
    ovc[w] = cv[0] | (cv[1] << 16);
  }

  if (full) {
    uint16_t* ph = T.hi + elem0;
    uint16_t* pl = T.lo + elem0;
    uint16_t* pm = T.mc + elem0;
    uint16_t* pv = T.vc + elem0;
    store8(ph + la, oh); store8(ph + lb, oh + 4);
    store8(pl + la, ol); store8(pl + lb, ol + 4);
    store8(pm + la, omc); store8(pm + lb, omc + 4);
    store8(pv + la, ovc); store8(pv + lb, ovc + 4);
  } else {
    store8_guard(T.hi, ea, n, oh); store8_guard(T.hi, eb, n, oh + 4);
    store8_guard(T.lo, ea, n, ol); store8_guard(T.lo, eb, n, ol + 4);
    store8_guard(T.mc, ea, n, omc); store8_guard(T.mc, eb, n, omc + 4);
    store8_guard(T.vc, ea, n, ovc); store8_guard(T.vc, eb, n, ovc + 4);
  }
  if (r == 0 && blk * kBlock < n) {
    T.ms[blk] = sm;
    T.vs[blk] = sv;
  }
}

template <class TBL>
__device__ __forceinline__ const DevTensor& rec(const TBL& t, int i) { return t.recs[i]; }
template <class TBL>
__device__ __forceinline__ uint32_t item_end(const TBL& t, int i) { return t.item_end[i]; }

// One work item per 64-lane workgroup. Workgroups are dispatched in index
// order, so the waves in flight at any moment cover a compact address range;
// this keeps HBM pages open and measured faster than persistent waves that
// stride over the items. The tensor of the item is found by a wave-uniform
// binary search over the prefix ends (scalar loads).
template <class TBL, int ALGO, bool WD, int SPLIT>
__global__ __launch_bounds__(64) void k_adam_step(TBL tbl, StepScalars c) {
  const uint32_t item = blockIdx.x;
  int lo = 0, hi = tbl.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (item_end(tbl, mid) > item)
      hi = mid;
    else
      lo = mid + 1;
  }
  const uint32_t begin = lo ? item_end(tbl, lo - 1) : 0u;
  process_item<ALGO, WD, SPLIT>(rec(tbl, lo), (int64_t)(item - begin) * kItemElems, (int)threadIdx.x, c);
}

template <class TBL, int ALGO, bool WD, int SPLIT>
ps_status launch_t(const TBL& tbl, uint32_t total_items, const StepScalars& c, hipStream_t s) {
  hipLaunchKernelGGL((k_adam_step<TBL, ALGO, WD, SPLIT>), dim3(total_items), dim3(64), 0, s, tbl, c);
  return hip_check(hipGetLastError(), "k_adam_step launch");
}

template <class TBL>
ps_status dispatch(const TBL& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                   hipStream_t s) {
  const bool wd = hp.weight_decay != 0.0;
  const bool na = hp.split_mode == PS_SPLIT_NEAREST_AWAY;
#define PS_CASE(A, W, S) \
  if (hp.algo == A && wd == W && na == (S == PS_SPLIT_NEAREST_AWAY)) return launch_t<TBL, A, W, S>(tbl, total_items, c, s);
  PS_CASE(PS_ALGO_NADAM, false, PS_SPLIT_TRUNC)
  PS_CASE(PS_ALGO_NADAM, true, PS_SPLIT_TRUNC)
  PS_CASE(PS_ALGO_ADAM, false, PS_SPLIT_TRUNC)
  PS_CASE(PS_ALGO_ADAM, true, PS_SPLIT_TRUNC)
  PS_CASE(PS_ALGO_NADAM, false, PS_SPLIT_NEAREST_AWAY)
  PS_CASE(PS_ALGO_NADAM, true, PS_SPLIT_NEAREST_AWAY)
  PS_CASE(PS_ALGO_ADAM, false, PS_SPLIT_NEAREST_AWAY)
  PS_CASE(PS_ALGO_ADAM, true, PS_SPLIT_NEAREST_AWAY)
#undef PS_CASE
  return fail(PS_ERR_UNSUPPORTED, "no kernel for algo %d split_mode %d", hp.algo, hp.split_mode);
}

}  // namespace

ps_status launch_adam_ptr(const TablePtr& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                          hipStream_t s) {
  return dispatch(tbl, total_items, hp, c, s);
}

ps_status launch_adam_inline(const TableInline& tbl, uint32_t total_items, const ps_hparams& hp,
                             const StepScalars& c, hipStream_t s) {
  return dispatch(tbl, total_items, hp, c, s);
}

}  // namespace ps
