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
  const u32x4 v = *(const GLOBAL u32x4*)p;
  dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const uint32_t* src) {
  *(GLOBAL u32x4*)p = u32x4{src[0], src[1], src[2], src[3]};
}

// Guarded variants for the last work item of a tensor: element e + j exists
// when e + j < n; missing elements read as `fill` and are not written.
__device__ __forceinline__ void load8_guard(const uint16_t* p, int64_t e, int64_t n, uint32_t fill, uint32_t* dst) {
  if (e + 8 <= n) {
    load8(p + e, dst);
    return;
  }
  const GLOBAL uint16_t* q = (const GLOBAL uint16_t*)p;
  for (int j = 0; j < 4; ++j) {
    uint32_t lo = (e + 2 * j < n) ? q[e + 2 * j] : (fill & 0xFFFFu);
    uint32_t hi = (e + 2 * j + 1 < n) ? q[e + 2 * j + 1] : (fill >> 16);
    dst[j] = lo | (hi << 16);
  }
}

__device__ __forceinline__ void store8_guard(uint16_t* p, int64_t e, int64_t n, const uint32_t* src) {
  if (e + 8 <= n) {
    store8(p + e, src);
    return;
  }
  GLOBAL uint16_t* q = (GLOBAL uint16_t*)p;
  for (int j = 0; j < 8; ++j)
    if (e + j < n) q[e + j] = (uint16_t)(src[j >> 1] >> (16 * (j & 1)));
}

// Phase 3 of a work item: update, residual split and moment encode of one
// lane's 16 elements. SLOW selects the library square root for the whole wave.
template <int ALGO, bool WD, int SPLIT, bool SLOW>
__device__ __forceinline__ void update_encode(const Regs& R, const float* m, const float* v, const StepScalars& c,
                                              float inv_m, float inv_v, float sq_inv_v, uint32_t* oh, uint32_t* ol,
                                              uint32_t* omc, uint32_t* ovc) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t wb[2], cm[2], cv[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int j = 2 * w + o;
      float g = o ? bf16_hi(R.g[w]) : bf16_lo(R.g[w]);
      float wf = __uint_as_float(join_pair_elem<SPLIT>(R.h[w], R.l[w], o));
      float rv = SLOW ? __builtin_sqrtf(v[j]) : sqrt_rn_fast(v[j]);
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
    ms_old = ((const GLOBAL float*)T.ms)[blk];
    vs_old = ((const GLOBAL float*)T.vs)[blk];
  } else {
    load8_guard(T.hi, ea, n, 0u, R.h); load8_guard(T.hi, eb, n, 0u, R.h + 4);
    load8_guard(T.lo, ea, n, 0u, R.l); load8_guard(T.lo, eb, n, 0u, R.l + 4);
    load8_guard(T.g, ea, n, 0u, R.g); load8_guard(T.g, eb, n, 0u, R.g + 4);
    load8_guard(T.mc, ea, n, 0x80008000u, R.mc); load8_guard(T.mc, eb, n, 0x80008000u, R.mc + 4);
    load8_guard(T.vc, ea, n, 0u, R.vc); load8_guard(T.vc, eb, n, 0u, R.vc + 4);
    if (blk * kBlock < n) {
      ms_old = ((const GLOBAL float*)T.ms)[blk];
      vs_old = ((const GLOBAL float*)T.vs)[blk];
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

  // Phase 3: update, split, encode. The wave-uniform choice of square root
  // is taken once so the common path carries no per-element branch.
  uint32_t oh[8], ol[8], omc[8], ovc[8];
  if (slow_sqrt)
    update_encode<ALGO, WD, SPLIT, true>(R, m, v, c, inv_m, inv_v, sq_inv_v, oh, ol, omc, ovc);
  else
    update_encode<ALGO, WD, SPLIT, false>(R, m, v, c, inv_m, inv_v, sq_inv_v, oh, ol, omc, ovc);

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
    ((GLOBAL float*)T.ms)[blk] = sm;
    ((GLOBAL float*)T.vs)[blk] = sv;
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

// ---------------------------------------------------------------------------
// Tensors with storage flags: fp32 or f24 moments instead of codes and/or an fp32
// parameter and gradient instead of bf16 + residual. Same lane layout and
// element arithmetic; the flags are uniform per work item.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load_f8(const float* p, int64_t e, int64_t n, float* d) {
  const GLOBAL float* q = (const GLOBAL float*)p;
  if (e + 8 <= n) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 a = *(const GLOBAL f32x4*)(q + e), b = *(const GLOBAL f32x4*)(q + e + 4);
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w; d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    return;
  }
  for (int j = 0; j < 8; ++j) d[j] = (e + j < n) ? q[e + j] : 0.0f;
}

__device__ __forceinline__ void store_f8(float* p, int64_t e, int64_t n, const float* s) {
  GLOBAL float* q = (GLOBAL float*)p;
  if (e + 8 <= n) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    *(GLOBAL f32x4*)(q + e) = f32x4{s[0], s[1], s[2], s[3]};
    *(GLOBAL f32x4*)(q + e + 4) = f32x4{s[4], s[5], s[6], s[7]};
    return;
  }
  for (int j = 0; j < 8; ++j)
    if (e + j < n) q[e + j] = s[j];
}

// Eight f24 values of elements e..e+7 (24 bytes at byte offset 3e, which is
// 8-byte aligned since e is a multiple of 8).
__device__ __forceinline__ void load_f24x8(const uint8_t* p, int64_t e, int64_t n, float* d) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const GLOBAL uint8_t* b8 = (const GLOBAL uint8_t*)p;
  if (e + 8 <= n) {
    const GLOBAL u32x2* q = (const GLOBAL u32x2*)(b8 + 3 * e);
    const u32x2 a = q[0], b = q[1], c = q[2];
    f24_unpack4(a.x, a.y, b.x, d);
    f24_unpack4(b.y, c.x, c.y, d + 4);
    return;
  }
  for (int j = 0; j < 8; ++j) {
    const int64_t o = 3 * (e + j);
    d[j] = (e + j < n) ? __uint_as_float(((uint32_t)b8[o] << 8) | ((uint32_t)b8[o + 1] << 16) | ((uint32_t)b8[o + 2] << 24))
                       : 0.0f;
  }
}

__device__ __forceinline__ void store_f24x8(uint8_t* p, int64_t e, int64_t n, const float* s) {
  uint32_t t[8];
  for (int j = 0; j < 8; ++j) t[j] = f24_round(s[j]);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  GLOBAL uint8_t* b8 = (GLOBAL uint8_t*)p;
  if (e + 8 <= n) {
    uint32_t w[6];
    f24_pack4(t, w[0], w[1], w[2]);
    f24_pack4(t + 4, w[3], w[4], w[5]);
    GLOBAL u32x2* q = (GLOBAL u32x2*)(b8 + 3 * e);
    q[0] = u32x2{w[0], w[1]};
    q[1] = u32x2{w[2], w[3]};
    q[2] = u32x2{w[4], w[5]};
    return;
  }
  for (int j = 0; j < 8; ++j)
    if (e + j < n) {
      const int64_t o = 3 * (e + j);
      b8[o] = (uint8_t)(t[j] >> 8);
      b8[o + 1] = (uint8_t)(t[j] >> 16);
      b8[o + 2] = (uint8_t)(t[j] >> 24);
    }
}

template <int ALGO, bool WD, int SPLIT>
__device__ __forceinline__ void process_item_ex(const DevTensorEx& T, int64_t elem0, int lane, const StepScalars& c) {
  const int b = lane >> 4, r = lane & 15;
  const int64_t n = T.numel;
  const int64_t blk = (elem0 >> 8) + b;
  const bool fpm = (T.flags & PS_TENSOR_FP32_MOMENTS) != 0;   // uniform per item
  const bool fpp = (T.flags & PS_TENSOR_FP32_PARAM) != 0;
  const bool f24 = (T.flags & PS_TENSOR_F24_MOMENTS) != 0;
  const bool codec = !fpm && !f24;
  const int64_t run[2] = {elem0 + b * kBlock + r * 8, elem0 + b * kBlock + 128 + r * 8};
  float w[16], g[16], m[16], v[16];
  uint32_t hw[8], lw[8];
  float ms_old = 0.0f, vs_old = 0.0f;
  if (codec && blk * kBlock < n) {
    ms_old = ((const GLOBAL float*)T.ms)[blk];
    vs_old = ((const GLOBAL float*)T.vs)[blk];
  }
  for (int h = 0; h < 2; ++h) {
    if (fpp) {
      load_f8((const float*)T.w, run[h], n, w + 8 * h);
      load_f8((const float*)T.g, run[h], n, g + 8 * h);
    } else {
      uint32_t gw[4];
      load8_guard((const uint16_t*)T.w, run[h], n, 0u, hw + 4 * h);
      load8_guard(T.lo, run[h], n, 0u, lw + 4 * h);
      load8_guard((const uint16_t*)T.g, run[h], n, 0u, gw);
      for (int j = 0; j < 8; ++j) {
        w[8 * h + j] = __uint_as_float(join_pair_elem<SPLIT>(hw[4 * h + (j >> 1)], lw[4 * h + (j >> 1)], j & 1));
        g[8 * h + j] = (j & 1) ? bf16_hi(gw[j >> 1]) : bf16_lo(gw[j >> 1]);
      }
    }
    if (fpm) {
      load_f8((const float*)T.m, run[h], n, m + 8 * h);
      load_f8((const float*)T.v, run[h], n, v + 8 * h);
    } else if (f24) {
      load_f24x8((const uint8_t*)T.m, run[h], n, m + 8 * h);
      load_f24x8((const uint8_t*)T.v, run[h], n, v + 8 * h);
    } else {
      uint32_t mw[4], vw[4];
      load8_guard((const uint16_t*)T.m, run[h], n, 0x80008000u, mw);
      load8_guard((const uint16_t*)T.v, run[h], n, 0u, vw);
      for (int j = 0; j < 8; ++j) {
        m[8 * h + j] = dec_signed((j & 1) ? code_hi_f(mw[j >> 1]) : code_lo_f(mw[j >> 1]), ms_old);
        v[8 * h + j] = dec_unsigned((j & 1) ? code_hi_f(vw[j >> 1]) : code_lo_f(vw[j >> 1]), vs_old);
      }
    }
  }
  float mx_m = 0.0f, mx_v = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float m1 = __builtin_fmaf(c.B1, m[k], c.C1 * g[k]);
    const float v1 = __builtin_fmaf(c.B2, v[k], c.C2 * (g[k] * g[k]));
    m[k] = m1;
    v[k] = v1;
    mx_m = __builtin_fmaxf(mx_m, __builtin_fabsf(m1));
    mx_v = __builtin_fmaxf(mx_v, v1);
  }
  float sm = 0.0f, inv_m = 0.0f, sv = 0.0f, inv_v = 0.0f;
  if (codec) {
    block_scale(row16_max(mx_m), sm, inv_m);
    block_scale(row16_max(mx_v), sv, inv_v);
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float d = __builtin_fmaf(__builtin_sqrtf(v[k]), c.RS2, c.EPS);
    float u;
    if (ALGO == PS_ALGO_ADAM)
      u = c.A * (m[k] / d);
    else
      u = __builtin_fmaf(c.AG, g[k], c.AM * m[k]) / d;
    if (WD) u = __builtin_fmaf(c.CWD, w[k], u);
    w[k] = w[k] - u;
  }
  for (int h = 0; h < 2; ++h) {
    if (fpp) {
      store_f8((float*)T.w, run[h], n, w + 8 * h);
    } else {
      uint32_t oh[4], ol[4];
      for (int q = 0; q < 4; ++q)
        split_pair<SPLIT>(__float_as_uint(w[8 * h + 2 * q]), __float_as_uint(w[8 * h + 2 * q + 1]), oh[q], ol[q]);
      store8_guard((uint16_t*)T.w, run[h], n, oh);
      store8_guard(T.lo, run[h], n, ol);
    }
    if (fpm) {
      store_f8((float*)T.m, run[h], n, m + 8 * h);
      store_f8((float*)T.v, run[h], n, v + 8 * h);
    } else if (f24) {
      store_f24x8((uint8_t*)T.m, run[h], n, m + 8 * h);
      store_f24x8((uint8_t*)T.v, run[h], n, v + 8 * h);
    } else {
      uint32_t om[4], ov[4];
      for (int q = 0; q < 4; ++q) {
        const int k = 8 * h + 2 * q;
        om[q] = enc_signed(m[k], inv_m) | (enc_signed(m[k + 1], inv_m) << 16);
        ov[q] = enc_unsigned(v[k], inv_v) | (enc_unsigned(v[k + 1], inv_v) << 16);
      }
      store8_guard((uint16_t*)T.m, run[h], n, om);
      store8_guard((uint16_t*)T.v, run[h], n, ov);
    }
  }
  if (codec && r == 0 && blk * kBlock < n) {
    ((GLOBAL float*)T.ms)[blk] = sm;
    ((GLOBAL float*)T.vs)[blk] = sv;
  }
}

template <int ALGO, bool WD, int SPLIT>
__global__ __launch_bounds__(64) void k_adam_step_ex(TableExPtr tbl, StepScalars c) {
  const uint32_t item = blockIdx.x;
  int lo = 0, hi = tbl.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tbl.item_end[mid] > item)
      hi = mid;
    else
      lo = mid + 1;
  }
  const uint32_t begin = lo ? tbl.item_end[lo - 1] : 0u;
  process_item_ex<ALGO, WD, SPLIT>(tbl.recs[lo], (int64_t)(item - begin) * kItemElems, (int)threadIdx.x, c);
}

template <int ALGO, bool WD, int SPLIT>
ps_status launch_ex_t(const TableExPtr& tbl, uint32_t total_items, const StepScalars& c, hipStream_t s) {
  hipLaunchKernelGGL((k_adam_step_ex<ALGO, WD, SPLIT>), dim3(total_items), dim3(64), 0, s, tbl, c);
  return hip_check(hipGetLastError(), "k_adam_step_ex launch");
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

ps_status launch_adam_ex(const TableExPtr& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                         hipStream_t s) {
  const bool wd = hp.weight_decay != 0.0;
  const bool na = hp.split_mode == PS_SPLIT_NEAREST_AWAY;
#define PS_CASE(A, W, S) \
  if (hp.algo == A && wd == W && na == (S == PS_SPLIT_NEAREST_AWAY)) return launch_ex_t<A, W, S>(tbl, total_items, c, s);
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

}  // namespace ps
