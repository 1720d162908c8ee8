// k_adam.hip - fused multi-tensor (N)AdamW step on residual-split bf16
// weights with uint16-coded moments [NADAM; KAHAN].
//
// Mapping (gfx950, wave64): the tensor list is cut into work items of 512
// elements (2 moment blocks) that never cross a tensor boundary; one work
// item is one 64-lane workgroup. A 256-element block belongs to 32 lanes (a
// pair of DPP rows) and each lane holds one run of 8 consecutive elements at
// offset r*8 of its block, so the block's 32 lanes read and write 512
// contiguous bytes of every 16-bit stream with 16-byte accesses. The block
// maximum is a butterfly within each row plus one row-pair exchange.
//
// Order of memory traffic within a wave: gradient and moment codes into
// registers (they decide the block scales), and in the same breath the weight
// words of a full item straight into LDS (global_load_lds_dwordx4, 2 KiB per
// wave), so all five streams are in flight at once without holding the weight
// words in VGPRs through the decode, EMA and block-maximum phase; the update
// reads them from LDS. This measured 1.5% faster per step than loading the
// weight words into registers after the block scales (which in turn was
// 3-12% faster than every stream loaded into registers up front with 16
// elements per lane). The block maxima are taken on float bit patterns (one
// fused DPP max per step); the occupancy hint keeps the NAdam kernels at 7
// waves per SIMD without spills.
//
// Per element the kernel reads hi, lo, grad, m_code, v_code (10 bytes) and
// writes hi, lo, m_code, v_code (8 bytes); per block it reads and writes the
// two scales (16 bytes).
#include "dev_common.h"
#include "ps_internal.h"

namespace ps {
namespace {

// Every byte of the state streams through once per step: the 16-byte loads
// and stores carry the non-temporal hint (3-4% faster per step, but only when
// both directions use it; loads alone were slower). The f24 arrays' 8-byte
// accesses stay plain: with the hint they were slower.
template <class V>
__device__ __forceinline__ V ld_nt(const V* p) {
  return __builtin_nontemporal_load((const GLOBAL V*)p);
}
template <class V>
__device__ __forceinline__ void st_nt(V* p, V v) {
  __builtin_nontemporal_store(v, (GLOBAL V*)p);
}

__device__ __forceinline__ void load8(const uint16_t* p, uint32_t* dst) {
  const u32x4 v = ld_nt((const u32x4*)p);
  dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const uint32_t* src) {
  st_nt((u32x4*)p, u32x4{src[0], src[1], src[2], src[3]});
}

// 16 bytes per lane from p straight into LDS: lane i's bytes land at
// dst + 16 i (dst is wave-uniform). Cache-policy bit 1 (nt) marks the load
// non-temporal like the register loads; without it the step was 1.5% slower
// than the register path instead of 1.5% faster.
constexpr int kLdsDmaNt = 2;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void load8_to_lds(const uint16_t* p, u32x4* dst) {
  __builtin_amdgcn_global_load_lds((const GLOBAL void*)p, (lds_void*)dst, 16, 0, kLdsDmaNt);
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

// Update, residual split and moment encode of one lane's 8 elements, then the
// stores. A full item's weight words are waiting in LDS (wl[0]: hi, wl[1]:
// lo, one 16-byte entry per lane); a partial item loads them here with
// per-element guards. SLOW selects the library square root for the wave.
template <int ALGO, bool WD, int SPLIT, bool SLOW>
__device__ __forceinline__ void update_store(const DevTensor& T, int64_t e, int64_t n, bool full, const uint32_t* gw,
                                             const float* m, const float* v, const StepScalars& c, float inv_m,
                                             float inv_v, float sq_inv_v, const u32x4 (*wl)[64]) {
  constexpr bool SR = SPLIT == PS_SPLIT_STOCHASTIC;
  uint32_t hw[4], lw[4] = {0u, 0u, 0u, 0u};
  if (full) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the LDS copies have landed
    const u32x4 a = wl[0][threadIdx.x];
    hw[0] = a.x; hw[1] = a.y; hw[2] = a.z; hw[3] = a.w;
    if (!SR) {
      const u32x4 b = wl[1][threadIdx.x];
      lw[0] = b.x; lw[1] = b.y; lw[2] = b.z; lw[3] = b.w;
    }
  } else {
    load8_guard(T.hi, e, n, 0u, hw);
    if (!SR) load8_guard(T.lo, e, n, 0u, lw);
  }
  uint64_t rnd[2] = {0u, 0u};
  if (SR) sr_bits8(sr_stream(c.sr_seed, c.sr_step, T.tid), e, rnd);
  uint32_t oh[4], ol[4], omc[4], ovc[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t wb[2], cm[2], cv[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int j = 2 * w + o;
      const float g = o ? bf16_hi(gw[w]) : bf16_lo(gw[w]);
      const float wf = SR ? (o ? bf16_hi(hw[w]) : bf16_lo(hw[w]))
                          : __uint_as_float(join_pair_elem<SPLIT>(hw[w], lw[w], o));
      const float rv = SLOW ? __builtin_sqrtf(v[j]) : sqrt_rn_fast(v[j]);
      const float d = __builtin_fmaf(rv, c.RS2, c.EPS);
      float u;
      if (ALGO == PS_ALGO_ADAM)
        u = c.A * (m[j] / d);
      else
        u = __builtin_fmaf(c.AG, g, c.AM * m[j]) / d;
      if (WD) u = __builtin_fmaf(c.CWD, wf, u);
      wb[o] = __float_as_uint(wf - u);
      cm[o] = enc_signed_lo16(m[j], inv_m);
      cv[o] = enc_unsigned_y_lo16(v[j], inv_v, fast_sqrt(rv * sq_inv_v));
    }
    if (SR) {
      const uint64_t q = rnd[w >> 1] >> (32 * (w & 1));
      oh[w] = sr_pair(wb[0], wb[1], (uint32_t)q & 0xFFFFu, (uint32_t)(q >> 16) & 0xFFFFu);
    } else {
      split_pair<SPLIT>(wb[0], wb[1], oh[w], ol[w]);
    }
    omc[w] = pack_lo16(cm[0], cm[1]);
    ovc[w] = pack_lo16(cv[0], cv[1]);
  }
  if (full) {
    store8(T.hi + e, oh);
    if (!SR) store8(T.lo + e, ol);
    store8(T.mc + e, omc);
    store8(T.vc + e, ovc);
  } else {
    store8_guard(T.hi, e, n, oh);
    if (!SR) store8_guard(T.lo, e, n, ol);
    store8_guard(T.mc, e, n, omc);
    store8_guard(T.vc, e, n, ovc);
  }
}

template <int ALGO, bool WD, int SPLIT>
__device__ __forceinline__ void process_item(const DevTensor& T, int64_t elem0, int lane, const StepScalars& c) {
  const int b = lane >> 5;                 // block of the item, 0..1
  const int r = lane & 31;                 // lane within the block's row pair
  const int64_t n = T.numel;
  const int64_t blk = (elem0 >> 8) + b;    // block index within the tensor
  const int64_t e = elem0 + b * kBlock + r * 8;
  const bool full = elem0 + kStepItemElems <= n;  // uniform per wave

  uint32_t gw[4], mw[4], vw[4];
  float ms_old = 0.0f, vs_old = 0.0f;
  __shared__ u32x4 wl[2][64];
  // Both weight pointers are read from the record before the first LDS copy
  // is issued: read after it, they were fetched with a vector load that
  // waited for the copy.
  const uint16_t* const hi_p = T.hi;
  const uint16_t* const lo_p = T.lo;
  if (full) {
    load8(T.g + e, gw);
    load8(T.mc + e, mw);
    load8(T.vc + e, vw);
    ms_old = ((const GLOBAL float*)T.ms)[blk];
    vs_old = ((const GLOBAL float*)T.vs)[blk];
    load8_to_lds(hi_p + e, &wl[0][0]);
    if (SPLIT != PS_SPLIT_STOCHASTIC) load8_to_lds(lo_p + e, &wl[1][0]);
  } else {
    load8_guard(T.g, e, n, 0u, gw);
    load8_guard(T.mc, e, n, 0x80008000u, mw);
    load8_guard(T.vc, e, n, 0u, vw);
    if (blk * kBlock < n) {
      ms_old = ((const GLOBAL float*)T.ms)[blk];
      vs_old = ((const GLOBAL float*)T.vs)[blk];
    }
  }

  // Decode, EMA, block maxima. Missing tail elements have g = 0 and
  // zero-coded moments, so m = v = 0 and they never raise a maximum.
  float m[8], v[8];
  float mx_m = 0.0f, mn_m = 0.0f;  // max and min of m: max |m| = max(mx_m, -mn_m)
  uint32_t mx_v = 0u;              // max of v as a bit pattern (v >= 0, never -0)
  uint32_t tiny = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    const bool odd = j & 1;
    const float g = odd ? bf16_hi(gw[w]) : bf16_lo(gw[w]);
    const float m0 = dec_signed(odd ? code_hi_f(mw[w]) : code_lo_f(mw[w]), ms_old);
    const float v0 = dec_unsigned(odd ? code_hi_f(vw[w]) : code_lo_f(vw[w]), vs_old);
    m[j] = __builtin_fmaf(c.B1, m0, c.C1 * g);
    v[j] = __builtin_fmaf(c.B2, v0, c.C2 * (g * g));
    mx_m = __builtin_fmaxf(mx_m, m[j]);
    mn_m = __builtin_fminf(mn_m, m[j]);
    mx_v = __builtin_elementwise_max(mx_v, __float_as_uint(v[j]));
    tiny = __builtin_elementwise_min(tiny, __float_as_uint(v[j]) - 1u);
  }
  // 0 < v < 2^-96 anywhere in the wave: the fast square root's residual test
  // could underflow there, so the whole wave takes the library sequence.
  const bool slow_sqrt = __builtin_amdgcn_ballot_w64(tiny < 0x0F7FFFFFu) != 0;

  // Block scales (32-lane maximum).
  float sm, inv_m, sv, inv_v;
  const float am = __builtin_fmaxf(mx_m, -mn_m);   // +0 or positive
  block_scale(__uint_as_float(row32_max_u32(__float_as_uint(am))), sm, inv_m);
  block_scale(__uint_as_float(row32_max_u32(mx_v)), sv, inv_v);
  const float sq_inv_v = fast_sqrt(inv_v);

  if (slow_sqrt)
    update_store<ALGO, WD, SPLIT, true>(T, e, n, full, gw, m, v, c, inv_m, inv_v, sq_inv_v, wl);
  else
    update_store<ALGO, WD, SPLIT, false>(T, e, n, full, gw, m, v, c, inv_m, inv_v, sq_inv_v, wl);
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
// stride over the items. Within that range each XCD takes runs of
// kXcdChunk consecutive items (xcd_item): 1.7% faster per step than plain
// index order on the 11.9B set, while runs of 64 items or one contiguous
// eighth of the list per XCD were 3-5% slower. The tensor of the item is found by a wave-uniform
// binary search over the prefix ends (scalar loads).
template <class TBL, int ALGO, bool WD, int SPLIT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(7))) void k_adam_step(TBL tbl, StepScalars c) {
  const uint32_t item = xcd_item<>(blockIdx.x, gridDim.x);
  int lo = 0, hi = tbl.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (item_end(tbl, mid) > item)
      hi = mid;
    else
      lo = mid + 1;
  }
  const uint32_t begin = lo ? item_end(tbl, lo - 1) : 0u;
  process_item<ALGO, WD, SPLIT>(rec(tbl, lo), (int64_t)(item - begin) * kStepItemElems, (int)threadIdx.x, c);
}

template <class TBL, int ALGO, bool WD, int SPLIT>
ps_status launch_t(const TBL& tbl, uint32_t total_items, const StepScalars& c, hipStream_t s) {
  hipLaunchKernelGGL((k_adam_step<TBL, ALGO, WD, SPLIT>), dim3(total_items), dim3(64), 0, s, tbl, c);
  return hip_check(hipGetLastError(), "k_adam_step launch");
}

// ---------------------------------------------------------------------------
// Tensors with storage flags: fp32 or f24 moments instead of codes and/or an
// fp32 parameter and gradient instead of bf16 + residual. Same lane layout and
// element arithmetic; the flags are uniform per work item.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load_f8(const float* p, int64_t e, int64_t n, float* d) {
  const GLOBAL float* q = (const GLOBAL float*)p;
  if (e + 8 <= n) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 a = ld_nt((const f32x4*)(p + e)), b = ld_nt((const f32x4*)(p + e + 4));
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w; d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
    return;
  }
  for (int j = 0; j < 8; ++j) d[j] = (e + j < n) ? q[e + j] : 0.0f;
}

__device__ __forceinline__ void store_f8(float* p, int64_t e, int64_t n, const float* s) {
  GLOBAL float* q = (GLOBAL float*)p;
  if (e + 8 <= n) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    st_nt((f32x4*)(p + e), f32x4{s[0], s[1], s[2], s[3]});
    st_nt((f32x4*)(p + e + 4), f32x4{s[4], s[5], s[6], s[7]});
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
  const int b = lane >> 5, r = lane & 31;
  const int64_t n = T.numel;
  const int64_t blk = (elem0 >> 8) + b;
  const int64_t e = elem0 + b * kBlock + r * 8;
  const bool fpm = (T.flags & PS_TENSOR_FP32_MOMENTS) != 0;   // uniform per item
  const bool fpp = (T.flags & PS_TENSOR_FP32_PARAM) != 0;
  const bool f24 = (T.flags & PS_TENSOR_F24_MOMENTS) != 0;
  const bool codec = !fpm && !f24;
  float w[8], g[8], m[8], v[8];
  float ms_old = 0.0f, vs_old = 0.0f;
  if (codec && blk * kBlock < n) {
    ms_old = ((const GLOBAL float*)T.ms)[blk];
    vs_old = ((const GLOBAL float*)T.vs)[blk];
  }
  if (fpp) {
    load_f8((const float*)T.w, e, n, w);
    load_f8((const float*)T.g, e, n, g);
  } else {
    uint32_t hw[4], lw[4] = {0u, 0u, 0u, 0u}, gw[4];
    load8_guard((const uint16_t*)T.w, e, n, 0u, hw);
    if (SPLIT != PS_SPLIT_STOCHASTIC) load8_guard(T.lo, e, n, 0u, lw);
    load8_guard((const uint16_t*)T.g, e, n, 0u, gw);
    for (int j = 0; j < 8; ++j) {
      w[j] = SPLIT == PS_SPLIT_STOCHASTIC ? ((j & 1) ? bf16_hi(hw[j >> 1]) : bf16_lo(hw[j >> 1]))
                                         : __uint_as_float(join_pair_elem<SPLIT>(hw[j >> 1], lw[j >> 1], j & 1));
      g[j] = (j & 1) ? bf16_hi(gw[j >> 1]) : bf16_lo(gw[j >> 1]);
    }
  }
  if (fpm) {
    load_f8((const float*)T.m, e, n, m);
    load_f8((const float*)T.v, e, n, v);
  } else if (f24) {
    load_f24x8((const uint8_t*)T.m, e, n, m);
    load_f24x8((const uint8_t*)T.v, e, n, v);
  } else {
    uint32_t mw[4], vw[4];
    load8_guard((const uint16_t*)T.m, e, n, 0x80008000u, mw);
    load8_guard((const uint16_t*)T.v, e, n, 0u, vw);
    for (int j = 0; j < 8; ++j) {
      m[j] = dec_signed((j & 1) ? code_hi_f(mw[j >> 1]) : code_lo_f(mw[j >> 1]), ms_old);
      v[j] = dec_unsigned((j & 1) ? code_hi_f(vw[j >> 1]) : code_lo_f(vw[j >> 1]), vs_old);
    }
  }
  float mx_m = 0.0f, mx_v = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float m1 = __builtin_fmaf(c.B1, m[k], c.C1 * g[k]);
    const float v1 = __builtin_fmaf(c.B2, v[k], c.C2 * (g[k] * g[k]));
    m[k] = m1;
    v[k] = v1;
    mx_m = __builtin_fmaxf(mx_m, __builtin_fabsf(m1));
    mx_v = __builtin_fmaxf(mx_v, v1);
  }
  float sm = 0.0f, inv_m = 0.0f, sv = 0.0f, inv_v = 0.0f;
  if (codec) {
    block_scale(row32_max(mx_m), sm, inv_m);
    block_scale(row32_max(mx_v), sv, inv_v);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float d = __builtin_fmaf(__builtin_sqrtf(v[k]), c.RS2, c.EPS);
    float u;
    if (ALGO == PS_ALGO_ADAM)
      u = c.A * (m[k] / d);
    else
      u = __builtin_fmaf(c.AG, g[k], c.AM * m[k]) / d;
    if (WD) u = __builtin_fmaf(c.CWD, w[k], u);
    w[k] = w[k] - u;
  }
  if (fpp) {
    store_f8((float*)T.w, e, n, w);
  } else if (SPLIT == PS_SPLIT_STOCHASTIC) {
    uint64_t rnd[2];
    sr_bits8(sr_stream(c.sr_seed, c.sr_step, T.tid), e, rnd);
    uint32_t oh[4];
    for (int q = 0; q < 4; ++q) {
      const uint64_t b = rnd[q >> 1] >> (32 * (q & 1));
      oh[q] = sr_pair(__float_as_uint(w[2 * q]), __float_as_uint(w[2 * q + 1]), (uint32_t)b & 0xFFFFu,
                      (uint32_t)(b >> 16) & 0xFFFFu);
    }
    store8_guard((uint16_t*)T.w, e, n, oh);
  } else {
    uint32_t oh[4], ol[4];
    for (int q = 0; q < 4; ++q)
      split_pair<SPLIT>(__float_as_uint(w[2 * q]), __float_as_uint(w[2 * q + 1]), oh[q], ol[q]);
    store8_guard((uint16_t*)T.w, e, n, oh);
    store8_guard(T.lo, e, n, ol);
  }
  if (fpm) {
    store_f8((float*)T.m, e, n, m);
    store_f8((float*)T.v, e, n, v);
  } else if (f24) {
    store_f24x8((uint8_t*)T.m, e, n, m);
    store_f24x8((uint8_t*)T.v, e, n, v);
  } else {
    uint32_t om[4], ov[4];
    for (int q = 0; q < 4; ++q) {
      om[q] = enc_signed(m[2 * q], inv_m) | (enc_signed(m[2 * q + 1], inv_m) << 16);
      ov[q] = enc_unsigned(v[2 * q], inv_v) | (enc_unsigned(v[2 * q + 1], inv_v) << 16);
    }
    store8_guard((uint16_t*)T.m, e, n, om);
    store8_guard((uint16_t*)T.v, e, n, ov);
  }
  if (codec && r == 0 && blk * kBlock < n) {
    ((GLOBAL float*)T.ms)[blk] = sm;
    ((GLOBAL float*)T.vs)[blk] = sv;
  }
}

template <int ALGO, bool WD, int SPLIT>
__global__ __launch_bounds__(64) void k_adam_step_ex(TableExPtr tbl, StepScalars c) {
  const uint32_t item = xcd_item<>(blockIdx.x, gridDim.x);
  int lo = 0, hi = tbl.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tbl.item_end[mid] > item)
      hi = mid;
    else
      lo = mid + 1;
  }
  const uint32_t begin = lo ? tbl.item_end[lo - 1] : 0u;
  process_item_ex<ALGO, WD, SPLIT>(tbl.recs[lo], (int64_t)(item - begin) * kStepItemElems, (int)threadIdx.x, c);
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
#define PS_CASE(A, W, S) \
  if (hp.algo == A && wd == W && hp.split_mode == S) return launch_t<TBL, A, W, S>(tbl, total_items, c, s);
#define PS_CASES(S) \
  PS_CASE(PS_ALGO_NADAM, false, S) PS_CASE(PS_ALGO_NADAM, true, S) PS_CASE(PS_ALGO_ADAM, false, S) \
  PS_CASE(PS_ALGO_ADAM, true, S)
  PS_CASES(PS_SPLIT_TRUNC)
  PS_CASES(PS_SPLIT_NEAREST_AWAY)
  PS_CASES(PS_SPLIT_STOCHASTIC)
#undef PS_CASES
#undef PS_CASE
  return fail(PS_ERR_UNSUPPORTED, "no kernel for algo %d split_mode %d", hp.algo, hp.split_mode);
}

}  // namespace

ps_status launch_adam_ptr(const TablePtr& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
                          hipStream_t s) {
  return dispatch(tbl, total_items, hp, c, s);
}

ps_status launch_adam_one(const TableOne& tbl, uint32_t total_items, const ps_hparams& hp, const StepScalars& c,
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
#define PS_CASE(A, W, S) \
  if (hp.algo == A && wd == W && hp.split_mode == S) return launch_ex_t<A, W, S>(tbl, total_items, c, s);
#define PS_CASES(S) \
  PS_CASE(PS_ALGO_NADAM, false, S) PS_CASE(PS_ALGO_NADAM, true, S) PS_CASE(PS_ALGO_ADAM, false, S) \
  PS_CASE(PS_ALGO_ADAM, true, S)
  PS_CASES(PS_SPLIT_TRUNC)
  PS_CASES(PS_SPLIT_NEAREST_AWAY)
  PS_CASES(PS_SPLIT_STOCHASTIC)
#undef PS_CASES
#undef PS_CASE
  return fail(PS_ERR_UNSUPPORTED, "no kernel for algo %d split_mode %d", hp.algo, hp.split_mode);
}

}  // namespace ps
