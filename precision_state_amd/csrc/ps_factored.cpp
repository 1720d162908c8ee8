// ps_factored.cpp - host side of ps_factored_step: validation, workspace
// layout and the device plan [ADAF, adafactor_step_param; PRODIGY].
//
// Workspace (caller-owned device memory), per 2-D tensor [R, C]:
//  - row-strip tensors: row sums [R] and, per row segment of the strip pass,
//    column sums of q and of g^2 / r_i [nseg][C] (double); sums of the new row
//    EMAs per 256-row chunk; rho[R], kap[C]; sums of Q_j / c_j per 256-column
//    chunk; the clip factor;
//  - other tensors: row sums per 256-column band [ntc][R] and column sums per
//    256-row band [sntr][C] (double); sums of the new row EMAs per 256-row
//    chunk; rho[R], kap[C], 1/r_i [R] and 1/c_j [C] (double); sums of
//    g^2 / (r_i c_j) (per row tile, flat item or stats tile, whichever form the
//    U^2 pass takes); the clip factor.
// Per 1-D tensor: this step's v[n], sums of g^2 / v per 1024-element item, the
// clip factor. Every region starts on 256 bytes. The plan image also carries
// the strip pass's groups and segments (strip_partition).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "ps_internal.h"

namespace ps {
namespace {

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

ps_status check_fhparams(const ps_factored_hparams* hp) {
  if (!hp) return fail(PS_ERR_INVALID_ARG, "factored hparams is NULL");
  if (hp->split_mode != PS_SPLIT_TRUNC && hp->split_mode != PS_SPLIT_NEAREST_AWAY &&
      hp->split_mode != PS_SPLIT_STOCHASTIC)
    return fail(PS_ERR_INVALID_ARG, "unknown split_mode %d", hp->split_mode);
  if (hp->reserved != 0) return fail(PS_ERR_INVALID_ARG, "reserved must be 0");
  if (!is_finite(hp->lr) || hp->lr < 0) return fail(PS_ERR_INVALID_ARG, "lr must be finite and >= 0");
  if (!is_finite(hp->beta2) || hp->beta2 < 0 || hp->beta2 >= 1) return fail(PS_ERR_INVALID_ARG, "beta2 must be in [0, 1)");
  if (!is_finite(hp->eps1) || !(hp->eps1 > 0) || !((float)hp->eps1 > 0.0f))
    return fail(PS_ERR_INVALID_ARG, "eps1 must be finite and > 0 once rounded to fp32");
  if (!is_finite(hp->clip_threshold) || !(hp->clip_threshold > 0))
    return fail(PS_ERR_INVALID_ARG, "clip_threshold must be finite and > 0");
  if (!is_finite(hp->weight_decay) || hp->weight_decay < 0)
    return fail(PS_ERR_INVALID_ARG, "weight_decay must be finite and >= 0");
  if (!is_finite(hp->decay_rate) || hp->decay_rate > 0)
    return fail(PS_ERR_INVALID_ARG, "decay_rate must be finite and <= 0");
  if (!is_finite(hp->beta1) || hp->beta1 < 0 || hp->beta1 >= 1) return fail(PS_ERR_INVALID_ARG, "beta1 must be in [0, 1)");
  return PS_OK;
}

ps_status check_ptr(const void* p, const char* what, int i, uintptr_t align) {
  if (!p) return fail(PS_ERR_INVALID_ARG, "tensor %d: %s is NULL", i, what);
  if (!is_aligned(p, align)) return fail(PS_ERR_ALIGNMENT, "tensor %d: %s is not %d-byte aligned", i, what, (int)align);
  return PS_OK;
}

struct Layout {
  std::vector<F2D> t2;
  std::vector<F1D> t1;
  std::vector<uint32_t> tile_end, rc_end, tile_nf_end, item2_end, item_end, rt_end, tile_u_end, item2u_end;
  std::vector<uint32_t> seg_end;   // [groups] prefix ends over segs
  std::vector<FSeg> segs;
  std::vector<int32_t> nseg;       // per caller tensor: strip segments (0 if not in the strip pass)
  std::vector<std::vector<FSeg>> by_group;
  size_t bytes = 0;
  void clear() {
    t2.clear(); t1.clear(); tile_end.clear(); rc_end.clear(); tile_nf_end.clear(); item2_end.clear();
    item_end.clear(); rt_end.clear(); tile_u_end.clear(); item2u_end.clear(); seg_end.clear(); segs.clear();
    nseg.clear(); bytes = 0;
  }
};

// 2-D tensors whose statistics take the row-strip pass: rows of 16-byte runs
// that a wave's 64 lanes cover in whole multiples (C % 512 == 0), at most two
// runs per thread of the workgroup, and flat (fewer than 2^31 elements).
bool strip_ok(const ps_tensor& x) {
  return x.grad != nullptr && x.numel > 0 && x.numel < (int64_t(1) << 31) && x.rows >= 1 && x.cols >= 1 &&
         x.rows <= 0x7FFFFFFF && x.cols <= 0x7FFFFFFF && x.rows * x.cols == x.numel && x.cols % 512 == 0 &&
         x.cols <= kStripMaxC;
}

// Splits the rows of the strip tensors, taken in list order as one sequence,
// into kStripGroups groups of nearly equal element counts (a row goes to the
// group its first element falls in), and each group into segments of one
// tensor's consecutive rows; lists with fewer than kStripGroups *
// kStripMinGroupRows such rows take the statistics tiles instead. Depends on
// the shapes only.
void strip_partition(const ps_tensor* t, int32_t n, Layout& L) {
  L.nseg.assign((size_t)std::max(n, 0), 0);
  std::vector<int32_t> t2idx((size_t)std::max(n, 0), -1);
  int32_t k2 = 0;
  uint64_t total = 0, rows = 0;
  for (int32_t i = 0; i < n; ++i) {
    const ps_tensor& x = t[i];
    if (x.numel <= 0 || x.grad == nullptr || (x.rows == 0 && x.cols == 0)) continue;
    t2idx[i] = k2++;
    if (strip_ok(x)) {
      total += (uint64_t)x.numel;
      rows += (uint64_t)x.rows;
    }
  }
  if (rows < (uint64_t)kStripGroups * kStripMinGroupRows) return;
  const uint64_t G = kStripGroups;
  // group g takes the rows whose first element lies in [B(g), B(g + 1))
  auto B = [&](uint64_t g) { return (uint64_t)(((unsigned __int128)total * g) / G); };
  auto cdiv = [](uint64_t a, uint64_t b) { return (a + b - 1) / b; };
  L.by_group.resize(G);
  for (auto& v : L.by_group) v.clear();
  uint64_t cum = 0, g = 0;
  for (int32_t i = 0; i < n; ++i) {
    const ps_tensor& x = t[i];
    if (t2idx[i] < 0 || !strip_ok(x)) continue;
    const uint64_t C = (uint64_t)x.cols, R = (uint64_t)x.rows, end = cum + R * C;
    while (g + 1 < G && B(g + 1) <= cum) ++g;
    for (uint64_t h = g; h < G && B(h) < end; ++h) {
      const uint64_t r0 = B(h) > cum ? std::min(R, cdiv(B(h) - cum, C)) : 0;
      const uint64_t r1 = h + 1 == G ? R : (B(h + 1) > cum ? std::min(R, cdiv(B(h + 1) - cum, C)) : 0);
      if (r1 > r0) L.by_group[h].push_back(FSeg{(uint32_t)t2idx[i], (int32_t)r0, (int32_t)r1, L.nseg[i]++});
    }
    cum = end;
  }
  for (uint64_t h = 0; h < G; ++h) {
    L.segs.insert(L.segs.end(), L.by_group[h].begin(), L.by_group[h].end());
    L.seg_end.push_back((uint32_t)L.segs.size());
  }
}

// Validates the list and lays out the workspace starting at `ws` (which may be
// NULL when only the size is wanted). fm: a first moment is kept in m_code /
// m_scale.
ps_status plan(const ps_tensor* t, int32_t n, char* ws, bool fm, bool residual, Layout& L) {
  if (n < 0) return fail(PS_ERR_INVALID_ARG, "n_tensors < 0");
  if (n > 0 && !t) return fail(PS_ERR_INVALID_ARG, "tensors is NULL");
  uint64_t tiles = 0, rc = 0, items = 0, tiles_nf = 0, items2 = 0, rt = 0, tiles_u = 0, items2u = 0;
  size_t off = 0;
  strip_partition(t, n, L);
  auto take = [&](size_t bytes) { char* p = ws ? ws + off : nullptr; off += up(bytes); return p; };
  for (int32_t i = 0; i < n; ++i) {
    const ps_tensor& x = t[i];
    if (x.numel < 0 || x.numel > (int64_t(1) << 40)) return fail(PS_ERR_SHAPE, "tensor %d: numel out of range", i);
    if (x.flags || x.reserved) return fail(PS_ERR_UNSUPPORTED, "tensor %d: storage flags are not supported here", i);
    if (x.numel == 0 || x.grad == nullptr) continue;
    ps_status s;
    if ((s = check_ptr(x.w_hi, "w_hi", i, 16)) || (residual && (s = check_ptr(x.w_lo, "w_lo", i, 16))) ||
        (s = check_ptr(x.grad, "grad", i, 16)))
      return s;
    if (fm && ((s = check_ptr(x.m_code, "m_code", i, 16)) || (s = check_ptr(x.m_scale, "m_scale", i, 4)))) return s;
    if (x.rows != 0 || x.cols != 0) {
      if (x.rows < 1 || x.cols < 1 || x.rows > 0x7FFFFFFF || x.cols > 0x7FFFFFFF || x.rows * x.cols != x.numel)
        return fail(PS_ERR_SHAPE, "tensor %d: rows * cols != numel", i);
      if ((s = check_ptr(x.row_ema, "row_ema", i, 4)) || (s = check_ptr(x.col_ema, "col_ema", i, 4))) return s;
      F2D d{};
      d.hi = x.w_hi; d.lo = x.w_lo; d.g = x.grad; d.row = x.row_ema; d.col = x.col_ema;
      d.R = (int32_t)x.rows; d.C = (int32_t)x.cols;
      d.ntr = (d.R + kFTileRows - 1) / kFTileRows;
      d.sntr = (d.R + kSTileRows - 1) / kSTileRows;
      d.ntc = (d.C + kFTileCols - 1) / kFTileCols;
      d.nrw = (d.R + kFRowColChunk - 1) / kFRowColChunk;
      d.ncw = (d.C + kFRowColChunk - 1) / kFRowColChunk;
      d.vec = (d.C % 8) == 0;
      d.strip = L.nseg[i] > 0;
      d.nrp = d.strip ? 1 : d.ntc;
      if (d.strip) d.sntr = L.nseg[i];
      // Flat items: every tensor below 2^31 elements whose rows are 16-byte
      // runs, and with a first moment (per-256 blocks of the flattened index)
      // also the others, whose items then take per-element row/column factors.
      d.flat = (d.vec || fm) && x.numel < (int64_t(1) << 31);
      if (fm && !d.flat)
        return fail(PS_ERR_UNSUPPORTED, "tensor %d: a first moment needs numel < 2^31", i);
      d.mc = fm ? x.m_code : nullptr;
      d.ms = fm ? x.m_scale : nullptr;
      d.tid = (uint32_t)i;
      d.nitems = d.flat ? (int32_t)((x.numel + kItemElems - 1) / kItemElems) : 0;
      // U^2 pass: row tiles when rows are 16-byte runs, else the flat items
      // (first moment) or the stats tiles.
      d.nuc = d.vec ? (d.C + kUCols - 1) / kUCols : 0;
      const int32_t nrt = d.vec ? ((d.R + kURows - 1) / kURows) * d.nuc : 0;
      d.npart = d.strip ? d.ncw : d.vec ? nrt : d.flat ? d.nitems : d.ntr * d.ntc;
      // The U^2 partials get room for every form a tensor of this shape can
      // take, so the workspace layout, and ps_factored_workspace_size, do not
      // depend on whether a first moment is kept.
      const int64_t items_any = x.numel < (int64_t(1) << 31) ? (x.numel + kItemElems - 1) / kItemElems : 0;
      const int64_t upart_n = d.strip ? (int64_t)d.ncw
                              : d.vec ? (int64_t)nrt : std::max<int64_t>(items_any, (int64_t)d.ntr * d.ntc);
      d.rowpart = (double*)take(sizeof(double) * (size_t)d.nrp * d.R);
      d.colpart = (double*)take(sizeof(double) * (size_t)d.sntr * d.C);
      d.qpart = d.strip ? (double*)take(sizeof(double) * (size_t)d.sntr * d.C) : nullptr;
      d.rpart = (double*)take(sizeof(double) * (size_t)d.nrw);
      d.rho = (float*)take(sizeof(float) * (size_t)d.R);
      d.kap = (float*)take(sizeof(float) * (size_t)d.C);
      d.rinv = d.strip ? nullptr : (double*)take(sizeof(double) * (size_t)d.R);
      d.cinv = d.strip ? nullptr : (double*)take(sizeof(double) * (size_t)d.C);
      d.upart = (double*)take(sizeof(double) * (size_t)upart_n);
      d.f = (float*)take(sizeof(float));
      if (!d.strip) tiles += (uint64_t)d.sntr * d.ntc;
      rc += (uint64_t)d.nrw + d.ncw;
      if (d.flat)
        items2 += (uint64_t)((x.numel + kApplyItemElems - 1) / kApplyItemElems);
      else
        tiles_nf += (uint64_t)d.ntr * d.ntc;
      if (d.strip)
        ;   // sum of U^2 from the strip pass's column partials
      else if (d.vec)
        rt += (uint64_t)nrt;
      else if (d.flat)
        items2u += (uint64_t)d.nitems;
      else
        tiles_u += (uint64_t)d.ntr * d.ntc;
      if (tiles > 0x7FFFFFFFull || rc > 0x7FFFFFFFull || items2 > 0x7FFFFFFFull || rt > 0x7FFFFFFFull ||
          items2u > 0x7FFFFFFFull)
        return fail(PS_ERR_SHAPE, "tensor list too large");
      L.t2.push_back(d);
      L.tile_end.push_back((uint32_t)tiles);
      L.rc_end.push_back((uint32_t)rc);
      L.tile_nf_end.push_back((uint32_t)tiles_nf);
      L.item2_end.push_back((uint32_t)items2);
      L.rt_end.push_back((uint32_t)rt);
      L.tile_u_end.push_back((uint32_t)tiles_u);
      L.item2u_end.push_back((uint32_t)items2u);
    } else {
      if ((s = check_ptr(x.v_code, "v_code", i, 16)) || (s = check_ptr(x.v_scale, "v_scale", i, 4))) return s;
      F1D d{};
      d.hi = x.w_hi; d.lo = x.w_lo; d.g = x.grad; d.vc = x.v_code; d.vs = x.v_scale; d.n = x.numel;
      d.mc = fm ? x.m_code : nullptr;
      d.ms = fm ? x.m_scale : nullptr;
      d.tid = (uint32_t)i;
      d.nitems = (int32_t)((x.numel + kItemElems - 1) / kItemElems);
      d.v = (float*)take(sizeof(float) * (size_t)x.numel);
      d.upart = (double*)take(sizeof(double) * (size_t)d.nitems);
      d.f = (float*)take(sizeof(float));
      items += (uint64_t)d.nitems;
      if (items > 0x7FFFFFFFull) return fail(PS_ERR_SHAPE, "tensor list too large");
      L.t1.push_back(d);
      L.item_end.push_back((uint32_t)items);
    }
  }
  // the U^2 launch takes the row tiles, the flat items that are not row
  // tiles and the 1-D items in one grid
  if (rt + items2u + items > 0xFFFFFFFFull) return fail(PS_ERR_SHAPE, "tensor list too large");
  L.bytes = off;
  return PS_OK;
}

}  // namespace

ps_status factored_prepare(const ps_tensor* t, int32_t n, const ps_factored_hparams* hp, int64_t step, char* ws,
                           FactoredCall& c) {
  if (ps_status s = check_fhparams(hp)) return s;
  if (step < 1) return fail(PS_ERR_INVALID_ARG, "step must be >= 1 (got %lld)", (long long)step);
  const bool fm = hp->beta1 != 0.0;
  const bool residual = hp->split_mode != PS_SPLIT_STOCHASTIC;
  thread_local Layout W;
  W.clear();
  if (ps_status s = plan(t, n, ws, fm, residual, W)) return s;
  c.empty = W.t2.empty() && W.t1.empty();
  c.ws_bytes = W.bytes;
  // the plan image: F2D[n2] | F1D[n1] | the seven [n2] prefix-end lists |
  // item_end[n1] | seg_end[groups] | FSeg[segments]
  const size_t b2 = W.t2.size() * sizeof(F2D), b1 = W.t1.size() * sizeof(F1D);
  const size_t e2 = W.t2.size() * sizeof(uint32_t), e1 = W.t1.size() * sizeof(uint32_t);
  const size_t eg = W.seg_end.size() * sizeof(uint32_t), bs = W.segs.size() * sizeof(FSeg);
  const std::vector<uint32_t>* lists2[7] = {&W.tile_end, &W.rc_end, &W.tile_nf_end, &W.item2_end,
                                            &W.rt_end, &W.tile_u_end, &W.item2u_end};
  c.image.resize(b2 + b1 + 7 * e2 + e1 + eg + bs);
  unsigned char* p = c.image.data();
  if (b2) memcpy(p, W.t2.data(), b2);
  if (b1) memcpy(p + b2, W.t1.data(), b1);
  if (e2)
    for (int k = 0; k < 7; ++k) memcpy(p + b2 + b1 + k * e2, lists2[k]->data(), e2);
  if (e1) memcpy(p + b2 + b1 + 7 * e2, W.item_end.data(), e1);
  if (eg) memcpy(p + b2 + b1 + 7 * e2 + e1, W.seg_end.data(), eg);
  if (bs) memcpy(p + b2 + b1 + 7 * e2 + e1 + eg, W.segs.data(), bs);
  // table offsets within the image (factored_bind adds the device base)
  FPlan& pl = c.plan;
  pl.t2 = (const F2D*)0;
  pl.t1 = (const F1D*)(b2);
  pl.tile_end = (const uint32_t*)(b2 + b1);
  pl.rc_end = (const uint32_t*)(b2 + b1 + e2);
  pl.tile_nf_end = (const uint32_t*)(b2 + b1 + 2 * e2);
  pl.item2_end = (const uint32_t*)(b2 + b1 + 3 * e2);
  pl.rt_end = (const uint32_t*)(b2 + b1 + 4 * e2);
  pl.tile_u_end = (const uint32_t*)(b2 + b1 + 5 * e2);
  pl.item2u_end = (const uint32_t*)(b2 + b1 + 6 * e2);
  pl.item_end = (const uint32_t*)(b2 + b1 + 7 * e2);
  pl.seg_end = (const uint32_t*)(b2 + b1 + 7 * e2 + e1);
  pl.segs = (const FSeg*)(b2 + b1 + 7 * e2 + e1 + eg);
  pl.n_groups = (uint32_t)W.seg_end.size();
  pl.n2 = (int32_t)W.t2.size();
  pl.n1 = (int32_t)W.t1.size();
  pl.n_tiles = W.tile_end.empty() ? 0 : W.tile_end.back();
  pl.n_rc = W.rc_end.empty() ? 0 : W.rc_end.back();
  pl.n_items = W.item_end.empty() ? 0 : W.item_end.back();
  pl.n_tiles_nf = W.tile_nf_end.empty() ? 0 : W.tile_nf_end.back();
  pl.n_items2 = W.item2_end.empty() ? 0 : W.item2_end.back();
  pl.n_rt = W.rt_end.empty() ? 0 : W.rt_end.back();
  pl.n_tiles_u = W.tile_u_end.empty() ? 0 : W.tile_u_end.back();
  pl.n_items2u = W.item2u_end.empty() ? 0 : W.item2u_end.back();
  FScalars& sc = c.sc;
  const double beta2_t = hp->decay_rate != 0.0 ? 1.0 - std::pow((double)step, hp->decay_rate) : hp->beta2;
  sc.B2 = (float)beta2_t;
  sc.C2 = (float)(1.0 - beta2_t);
  sc.EPS1 = (float)hp->eps1;
  sc.CWD = (float)(hp->lr * hp->weight_decay);
  sc.B1 = (float)hp->beta1;
  sc.C1 = (float)(1.0 - hp->beta1);
  sc.lr = hp->lr;
  sc.clip = hp->clip_threshold;
  sc.wd = hp->weight_decay != 0.0;
  sc.fm = fm;
  sc.sr_seed = residual ? 0 : hp->seed;
  sc.sr_step = (uint32_t)step;
  sc.pad = 0;
  return PS_OK;
}

void factored_bind(FactoredCall& c, const void* dev_image) {
  const uintptr_t base = (uintptr_t)dev_image;
  FPlan& pl = c.plan;
  pl.t2 = (const F2D*)(base + (uintptr_t)pl.t2);
  pl.t1 = (const F1D*)(base + (uintptr_t)pl.t1);
  const uint32_t** lists[9] = {&pl.tile_end, &pl.rc_end, &pl.tile_nf_end, &pl.item2_end, &pl.rt_end,
                               &pl.tile_u_end, &pl.item2u_end, &pl.item_end, &pl.seg_end};
  for (const uint32_t** q : lists) *q = (const uint32_t*)(base + (uintptr_t)*q);
  pl.segs = (const FSeg*)(base + (uintptr_t)pl.segs);
}

}  // namespace ps

using namespace ps;

extern "C" {

ps_status ps_factored_workspace_size(const ps_tensor* tensors, int32_t n_tensors, size_t* bytes) {
  if (!bytes) return fail(PS_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  Layout L;
  if (ps_status s = plan(tensors, n_tensors, nullptr, false, false, L)) return s;
  *bytes = L.bytes;
  return PS_OK;
}

ps_status ps_factored_step(const ps_tensor* tensors, int32_t n_tensors, const ps_factored_hparams* hp, int64_t step,
                           void* workspace, size_t workspace_bytes, ps_stream_t stream) {
  thread_local FactoredCall c;
  if (ps_status s = factored_prepare(tensors, n_tensors, hp, step, nullptr, c)) return s;
  if (c.empty) return PS_OK;
  if (!workspace) return fail(PS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", c.ws_bytes);
  if (!is_aligned(workspace, 256)) return fail(PS_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  if (workspace_bytes < c.ws_bytes)
    return fail(PS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, c.ws_bytes);
  if (ps_status s = factored_prepare(tensors, n_tensors, hp, step, (char*)workspace, c)) return s;
  hipStream_t s = (hipStream_t)stream;
  const void* d = nullptr;
  TableLease lease(table_cache());   // held until the launches that read the plan are enqueued
  if (ps_status st = device_blob(c.image.data(), c.image.size(), s, &d, lease)) return st;
  factored_bind(c, d);
  return launch_factored(c.plan, c.sc, hp->split_mode, s);
}

}  // extern "C"
