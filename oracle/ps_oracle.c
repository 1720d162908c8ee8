/* ps_oracle.c - reference oracle for the fused low-precision optimizer step.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load or call this library. The HIP library under
 * precision_state_amd/ never includes, links or calls it, and it shares no
 * code with that library.
 *
 * Plain, slow, single-threaded C. Every fp32 operation is IEEE binary32 with
 * round-to-nearest-even; the build uses -O2 -ffp-contract=off (no fused
 * multiply-add except the explicit fmaf calls), no -ffast-math, and x86 SSE
 * keeps denormals. sqrtf, fmaf and '/' are correctly rounded.
 *
 * Sources (the pages this follows; cited by title and section):
 *  [KAHAN]  kohya-ss/sd-scripts PR #2159, "Kahan summation for
 *           Adafactor-optimized Flux FFT": the author's note on sending only
 *           the 16 low bits clipped off by bf16, the copy_kahan_ docstring, and
 *           the closing explanation (a 20%-of-an-ulp update moves the bf16
 *           value once every five steps).
 *  [NADAM]  kohya-ss/sd-scripts PR #2187, "(N)AdamW / Adan with fused
 *           backwards pass & CPU offloading": opening post (AdamW, Nesterov
 *           momentum, Kahan summation, lr 3.5e-6) and the second post (moments
 *           scaled, biased and pow()-companded into uint16).
 *  [ADAF]   kohya-ss/sd-scripts commit 7983d3d, "Fused backward pass",
 *           library/adafactor_fused.py, adafactor_step_param.
 *  [PRODIGY] konstmish/prodigy PR #25, "no first moment and factored second
 *           moment": beta1 = 0, factored second moment, update clipping, and
 *           the eps2 / zero-gradient NaN discussion.
 *
 * Readings the pages leave open (each one is also listed in the design doc):
 *  - Split/join: TRUNC keeps the fp32 word's upper half as the bf16 weight and
 *    its lower half as the residual, which restores the fp32 value bit for bit
 *    [KAHAN]. NEAREST_AWAY is the bijective round-to-nearest alternative.
 *  - Moment codec: exponent 1/4, one fp32 scale (the block's max |value|) per
 *    256-element block; codes round to nearest in the companded domain, with
 *    the half-way points evaluated through the decoder's own fp32 arithmetic.
 *  - NAdam: Dozat's Nesterov Adam with the momentum schedule
 *    mu_t = beta1 (1 - 0.5 * 0.96^(t * psi)); decoupled weight decay is added
 *    to the step (w - (u + lr*wd*w)).
 *  - Factored step: eps1 added to g^2 before the means, no bias correction,
 *    V^-1/2 built as (1/sqrt(r_i/mean(r))) * (1/sqrt(c_j)), RMS over the
 *    whole tensor. The update applies the fp32 U = (g * rho_i) * kap_j; the
 *    RMS that sets the clip is evaluated in double from the factored estimate
 *    itself, U_ij^2 = g_ij^2 * mean(r) / (r_i * c_j) (1-D: g^2 / v), so it is
 *    the RMS of the exact U for the stored EMAs, free of the fp32 rounding of
 *    rho, kap and U. beta2 is constant unless decay_rate < 0, which gives
 *    beta2_t = 1 - t^decay_rate [ADAF]; the optional first moment is an EMA
 *    of the clipped, lr-scaled update, taken before weight decay [ADAF].
 *  - f24 moments: bits 8..31 of the fp32 word, rounded to nearest even,
 *    3 little-endian bytes per value, no scale [NADAM, third post].
 *  - Stochastic rounding: round away from zero with probability
 *    low16(w)/2^16, the 16 random bits per element drawn from a SplitMix64
 *    stream keyed on (seed, step, tensor) [KAHAN; NADAM opening post].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLOCK 256

enum { ORC_ALGO_ADAM = 0, ORC_ALGO_NADAM = 1 };
enum { ORC_SPLIT_TRUNC = 0, ORC_SPLIT_NEAREST_AWAY = 1, ORC_SPLIT_STOCHASTIC = 2 };
enum { ORC_SIGNED = 0, ORC_UNSIGNED = 1 };

typedef struct {
  int32_t algo;
  int32_t split_mode;
  double lr, beta1, beta2, eps, weight_decay, momentum_decay;
  uint64_t seed;    /* stochastic rounding: the run's seed */
  int64_t tensor;   /* stochastic rounding: the tensor's key (its index in the step's list) */
  int64_t elem0;    /* stochastic rounding: index within the tensor of the arrays' element 0 */
} orc_hparams;

typedef struct {
  int32_t split_mode;
  int32_t reserved;
  double lr, beta2, eps1, clip_threshold, weight_decay;
  double decay_rate; /* 0: constant beta2; < 0: beta2 at update t is 1 - t^decay_rate [ADAF] */
  double beta1;      /* 0: no first moment; > 0: EMA of the clipped update, kept in the signed codec [ADAF] */
  uint64_t seed;     /* stochastic rounding: the run's seed */
  int64_t tensor;    /* stochastic rounding: the tensor's index in the step's list */
} orc_fhparams;

/* Step-dependent fp32 scalars, each computed in double and rounded once. */
typedef struct {
  float B1, C1, B2, C2, EPS, A, RS2, AG, AM, CWD;
} orc_coeffs;

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 bit pattern -> fp32 (exact widening). */
float orc_bf16_to_f32(uint16_t b) { return f_of((uint32_t)b << 16); }

/* ------------------------------------------------------------------------ */
/* Split / join of the fp32 master weight [KAHAN]                           */
/* ------------------------------------------------------------------------ */

/* Rebuild the fp32 bit pattern from the bf16 weight and the 16-bit residual. */
uint32_t orc_join1(uint16_t hi, uint16_t lo, int mode) {
  if (mode == ORC_SPLIT_TRUNC) return ((uint32_t)hi << 16) | lo;
  /* NEAREST_AWAY: hi was rounded up exactly when the residual's top bit is set */
  uint32_t h = ((uint32_t)hi - ((uint32_t)lo >> 15)) & 0xFFFFu;
  return (h << 16) | lo;
}

/* Cut the fp32 bit pattern into the bf16 weight and the 16-bit residual. */
void orc_split1(uint32_t w, uint16_t* hi, uint16_t* lo, int mode) {
  if (mode == ORC_SPLIT_TRUNC)
    *hi = (uint16_t)(w >> 16);
  else
    *hi = (uint16_t)(((w + 0x8000u) >> 16) & 0xFFFFu);
  *lo = (uint16_t)(w & 0xFFFFu);
}

void orc_join(const uint16_t* hi, const uint16_t* lo, float* w, int64_t n, int mode) {
  for (int64_t i = 0; i < n; ++i) w[i] = f_of(orc_join1(hi[i], lo[i], mode));
}

void orc_split(const float* w, uint16_t* hi, uint16_t* lo, int64_t n, int mode) {
  for (int64_t i = 0; i < n; ++i) orc_split1(u_of(w[i]), &hi[i], &lo[i], mode);
}

/* ------------------------------------------------------------------------ */
/* Stochastic rounding to bf16 without a residual [KAHAN, PR #2159 body: the */
/* default the residual replaces; NADAM opening post: "stochastic updates"] */
/* ------------------------------------------------------------------------ */

/* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): the state advances by the golden-ratio
 * increment and each output is the state passed through this finaliser. */
#define ORC_GOLDEN 0x9E3779B97F4A7C15ull
uint64_t orc_splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Output number k (0-based) of the SplitMix64 stream whose state starts at s. */
uint64_t orc_splitmix64_at(uint64_t s, uint64_t k) { return orc_splitmix64_mix(s + (k + 1) * ORC_GOLDEN); }

/* The random 16 bits of element e of tensor `tensor` at update `step` (step
 * taken modulo 2^32, tensor modulo 2^32): the stream starts at
 * mix(seed ^ mix(step << 32 | tensor)); output e/4 covers elements 4(e/4) ..
 * 4(e/4)+3, element e taking bits 16(e%4) .. 16(e%4)+15. */
uint16_t orc_sr_rand16(uint64_t seed, int64_t step, int64_t tensor, int64_t e) {
  uint64_t key = ((uint64_t)(uint32_t)step << 32) | (uint32_t)tensor;
  uint64_t s = orc_splitmix64_mix(seed ^ orc_splitmix64_mix(key));
  uint64_t word = orc_splitmix64_at(s, (uint64_t)e >> 2);
  return (uint16_t)(word >> (16 * (e & 3)));
}

/* Round x to one of its two neighbouring bf16 values: away from zero with
 * probability equal to the discarded low 16 bits / 2^16, the fractional
 * distance to the next bf16 in magnitude. With r uniform on [0, 2^16) this is
 * the upper half of bits(x) + r (a carry out of the low half is the round
 * away, across binades too). */
uint16_t orc_sr_bf16(float x, uint16_t r) { return (uint16_t)((u_of(x) + r) >> 16); }

/* Master weight and split in a given mode. STOCHASTIC has no residual: the
 * weight is the bf16 value itself and lo is neither read nor written. */
static float join_at(const uint16_t* hi, const uint16_t* lo, int64_t e, int mode) {
  if (mode == ORC_SPLIT_STOCHASTIC) return f_of((uint32_t)hi[e] << 16);
  return f_of(orc_join1(hi[e], lo[e], mode));
}

static void split_at(float w, uint16_t* hi, uint16_t* lo, int64_t e, const orc_hparams* hp, int64_t step) {
  if (hp->split_mode == ORC_SPLIT_STOCHASTIC)
    hi[e] = orc_sr_bf16(w, orc_sr_rand16(hp->seed, step, hp->tensor, hp->elem0 + e));
  else
    orc_split1(u_of(w), &hi[e], &lo[e], hp->split_mode);
}

void orc_sr_rand16_array(uint64_t seed, int64_t step, int64_t tensor, int64_t e0, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_rand16(seed, step, tensor, e0 + i);
}

/* ------------------------------------------------------------------------ */
/* Moment codec [NADAM second post]                                         */
/* ------------------------------------------------------------------------ */

static uint32_t code_q(int kind) { return kind == ORC_SIGNED ? 32767u : 65535u; }
static float code_k(int kind) { return kind == ORC_SIGNED ? (float)(1.0 / 32767.0) : (float)(1.0 / 65535.0); }

/* Companded magnitude of (possibly half-integer) code h: ((h/Q)^2)^2 with
 * 1/Q rounded to fp32 once and three fp32 multiplies. */
float orc_dec_mag(float h, int kind) {
  float a = h * code_k(kind);
  float t = a * a;
  return t * t;
}

/* Code magnitude of x in [0, 1]: the largest k in 0..Q with k == 0 or
 * x >= dec_mag(k - 1/2), i.e. round-to-nearest in the 1/4-power domain. */
uint32_t orc_code_mag(float x, int kind) {
  uint32_t lo = 0, hi = code_q(kind);
  while (lo < hi) {
    uint32_t mid = lo + (hi - lo + 1) / 2;
    if (x >= orc_dec_mag((float)mid - 0.5f, kind))
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

/* Encode one block of L <= 256 values. The scale is the block's max |value|;
 * a block whose max is below the smallest normal fp32 gets scale 0 and zero
 * codes, so 1/scale can never overflow. Signed codes are 32768 +- k. */
void orc_encode_block(const float* val, int L, int kind, uint16_t* code, float* scale) {
  float s = 0.0f;
  for (int i = 0; i < L; ++i) {
    float a = fabsf(val[i]);
    if (a > s) s = a;
  }
  uint16_t zero = kind == ORC_SIGNED ? 32768 : 0;
  if (!(s >= 0x1p-126f)) {
    *scale = 0.0f;
    for (int i = 0; i < L; ++i) code[i] = zero;
    return;
  }
  float inv = 1.0f / s;
  for (int i = 0; i < L; ++i) {
    float x = fabsf(val[i]) * inv;
    uint32_t k = orc_code_mag(x, kind);
    if (kind == ORC_SIGNED)
      code[i] = (uint16_t)(val[i] < 0.0f ? 32768u - k : 32768u + k);
    else
      code[i] = (uint16_t)k;
  }
  *scale = s;
}

float orc_decode1(uint16_t c, float s, int kind) {
  if (kind == ORC_SIGNED) {
    int32_t k = (int32_t)c - 32768;
    float v = orc_dec_mag((float)(k < 0 ? -k : k), kind) * s;
    return k < 0 ? -v : v;
  }
  return orc_dec_mag((float)c, kind) * s;
}

void orc_encode(const float* val, int64_t n, int kind, uint16_t* code, float* scale) {
  for (int64_t b = 0; b * ORC_BLOCK < n; ++b) {
    int64_t L = n - b * ORC_BLOCK;
    if (L > ORC_BLOCK) L = ORC_BLOCK;
    orc_encode_block(val + b * ORC_BLOCK, (int)L, kind, code + b * ORC_BLOCK, &scale[b]);
  }
}

void orc_decode(const uint16_t* code, const float* scale, int64_t n, int kind, float* val) {
  for (int64_t i = 0; i < n; ++i) val[i] = orc_decode1(code[i], scale[i / ORC_BLOCK], kind);
}

/* Vector helpers for the tests. */
void orc_dec_mag_array(const float* h, int64_t n, int kind, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_dec_mag(h[i], kind);
}

void orc_code_mag_array(const float* x, int64_t n, int kind, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_code_mag(x[i], kind);
}

/* ------------------------------------------------------------------------ */
/* Adam / NAdam step [NADAM opening post; ADAF for the EMA form]            */
/* ------------------------------------------------------------------------ */

/* NAdam momentum schedule: mu_i = beta1 * (1 - 0.5 * 0.96^(i * psi)). */
static double nadam_mu(double beta1, double psi, int64_t i) {
  return beta1 * (1.0 - 0.5 * pow(0.96, (double)i * psi));
}

/* Scalars for update number t (t >= 1):
 *   A   = lr / (1 - beta1^t)                     (Adam bias correction 1)
 *   RS2 = 1 / sqrt(1 - beta2^t)                  (bias correction 2 on sqrt(v))
 *   AG  = lr (1 - mu_t) / (1 - prod_{i<=t} mu_i)
 *   AM  = lr mu_{t+1} / (1 - prod_{i<=t+1} mu_i) (NAdam's two Nesterov terms)
 *   CWD = lr * wd                                (decoupled weight decay) */
void orc_coeffs_for(const orc_hparams* hp, int64_t t, orc_coeffs* c) {
  c->B1 = (float)hp->beta1;
  c->C1 = (float)(1.0 - hp->beta1);
  c->B2 = (float)hp->beta2;
  c->C2 = (float)(1.0 - hp->beta2);
  c->EPS = (float)hp->eps;
  c->A = (float)(hp->lr / (1.0 - pow(hp->beta1, (double)t)));
  c->RS2 = (float)(1.0 / sqrt(1.0 - pow(hp->beta2, (double)t)));
  double prod = 1.0;
  for (int64_t i = 1; i <= t; ++i) prod *= nadam_mu(hp->beta1, hp->momentum_decay, i);
  double mu_t = nadam_mu(hp->beta1, hp->momentum_decay, t);
  double mu_n = nadam_mu(hp->beta1, hp->momentum_decay, t + 1);
  c->AG = (float)(hp->lr * (1.0 - mu_t) / (1.0 - prod));
  c->AM = (float)(hp->lr * mu_n / (1.0 - prod * mu_n));
  c->CWD = (float)(hp->lr * hp->weight_decay);
}

/* One element: EMA of g and g^2, bias-corrected (N)Adam step, optional
 * decoupled weight decay, one subtraction from the fp32 master weight. */
static float step_elem(float w, float g, float m0, float v0, const orc_coeffs* c, int algo, int wd,
                       float* m_out, float* v_out) {
  float m = fmaf(c->B1, m0, c->C1 * g);
  float v = fmaf(c->B2, v0, c->C2 * (g * g));
  float d = fmaf(sqrtf(v), c->RS2, c->EPS);
  float u;
  if (algo == ORC_ALGO_ADAM)
    u = c->A * (m / d);
  else
    u = fmaf(c->AG, g, c->AM * m) / d;
  if (wd) u = fmaf(c->CWD, w, u);
  *m_out = m;
  *v_out = v;
  return w - u;
}

/* The step on plain fp32 state (no residual split, no moment codec): used to
 * pin the update rule against library optimizers. */
void orc_core_step(float* w, float* m, float* v, const float* g, int64_t n, const orc_hparams* hp,
                   int64_t step) {
  orc_coeffs c;
  orc_coeffs_for(hp, step, &c);
  int wd = hp->weight_decay != 0.0;
  for (int64_t i = 0; i < n; ++i) w[i] = step_elem(w[i], g[i], m[i], v[i], &c, hp->algo, wd, &m[i], &v[i]);
}

/* The full step on one tensor: join the master weight, widen the gradient,
 * decode both moments with the old block scales, update, re-encode the
 * moments from this step's fp32 values, split the new master weight. A
 * tensor without a gradient (g == NULL) is left untouched [ADAF]. */
void orc_opt_step(uint16_t* hi, uint16_t* lo, const uint16_t* g, uint16_t* mc, float* ms, uint16_t* vc,
                  float* vs, int64_t n, const orc_hparams* hp, int64_t step) {
  if (!g) return;
  orc_coeffs c;
  orc_coeffs_for(hp, step, &c);
  int wd = hp->weight_decay != 0.0;
  float mbuf[ORC_BLOCK], vbuf[ORC_BLOCK];
  for (int64_t b = 0; b * ORC_BLOCK < n; ++b) {
    int64_t base = b * ORC_BLOCK;
    int L = (int)(n - base < ORC_BLOCK ? n - base : ORC_BLOCK);
    for (int i = 0; i < L; ++i) {
      int64_t e = base + i;
      float w = join_at(hi, lo, e, hp->split_mode);
      float gf = orc_bf16_to_f32(g[e]);
      float m0 = orc_decode1(mc[e], ms[b], ORC_SIGNED);
      float v0 = orc_decode1(vc[e], vs[b], ORC_UNSIGNED);
      float w2 = step_elem(w, gf, m0, v0, &c, hp->algo, wd, &mbuf[i], &vbuf[i]);
      split_at(w2, hi, lo, e, hp, step);
    }
    orc_encode_block(mbuf, L, ORC_SIGNED, mc + base, &ms[b]);
    orc_encode_block(vbuf, L, ORC_UNSIGNED, vc + base, &vs[b]);
  }
}

/* Per-tensor precision policy [NADAM, second post: tensors of <= 4096
 * elements keep their moments in fp32; third post: the final layer trains in
 * fp32]. flags bit 0: moments are fp32 arrays m[n], v[n] (no codec, scales
 * unused); bit 1: the parameter and its gradient are fp32 arrays w[n], g[n]
 * (no residual); bit 2: moments are f24 arrays (3 bytes per value, scales
 * unused). The update is the same element step. */
enum { ORC_FP32_MOMENTS = 1, ORC_FP32_PARAM = 2, ORC_F24_MOMENTS = 4 };

/* f24 storage [NADAM, third post]: the upper three bytes of the fp32 word,
 * i.e. 8 more mantissa bits than bf16. Rounding to 24 bits is to nearest,
 * ties to even (the pages do not say). Stored little-endian, 3 bytes per
 * value. */
void orc_f24_encode1(float x, uint8_t* out) {
  uint32_t b = u_of(x);
  uint32_t r = (b + 0x7Fu + ((b >> 8) & 1u)) >> 8;
  out[0] = (uint8_t)r;
  out[1] = (uint8_t)(r >> 8);
  out[2] = (uint8_t)(r >> 16);
}

float orc_f24_decode1(const uint8_t* in) {
  return f_of(((uint32_t)in[0] << 8) | ((uint32_t)in[1] << 16) | ((uint32_t)in[2] << 24));
}

void orc_f24_encode(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) orc_f24_encode1(x[i], out + 3 * i);
}

void orc_f24_decode(const uint8_t* in, int64_t n, float* x) {
  for (int64_t i = 0; i < n; ++i) x[i] = orc_f24_decode1(in + 3 * i);
}

void orc_opt_step_flags(void* w, uint16_t* lo, const void* g, void* m, float* ms, void* v, float* vs, int64_t n,
                        uint32_t flags, const orc_hparams* hp, int64_t step) {
  if (!g) return;
  orc_coeffs c;
  orc_coeffs_for(hp, step, &c);
  int wd = hp->weight_decay != 0.0;
  float mbuf[ORC_BLOCK], vbuf[ORC_BLOCK];
  for (int64_t b = 0; b * ORC_BLOCK < n; ++b) {
    int64_t base = b * ORC_BLOCK;
    int L = (int)(n - base < ORC_BLOCK ? n - base : ORC_BLOCK);
    for (int i = 0; i < L; ++i) {
      int64_t e = base + i;
      float wf, gf, m0, v0;
      if (flags & ORC_FP32_PARAM) {
        wf = ((float*)w)[e];
        gf = ((const float*)g)[e];
      } else {
        wf = join_at((uint16_t*)w, lo, e, hp->split_mode);
        gf = orc_bf16_to_f32(((const uint16_t*)g)[e]);
      }
      if (flags & ORC_FP32_MOMENTS) {
        m0 = ((float*)m)[e];
        v0 = ((float*)v)[e];
      } else if (flags & ORC_F24_MOMENTS) {
        m0 = orc_f24_decode1((uint8_t*)m + 3 * e);
        v0 = orc_f24_decode1((uint8_t*)v + 3 * e);
      } else {
        m0 = orc_decode1(((uint16_t*)m)[e], ms[b], ORC_SIGNED);
        v0 = orc_decode1(((uint16_t*)v)[e], vs[b], ORC_UNSIGNED);
      }
      float w2 = step_elem(wf, gf, m0, v0, &c, hp->algo, wd, &mbuf[i], &vbuf[i]);
      if (flags & ORC_FP32_PARAM)
        ((float*)w)[e] = w2;
      else
        split_at(w2, (uint16_t*)w, lo, e, hp, step);
      if (flags & ORC_FP32_MOMENTS) {
        ((float*)m)[e] = mbuf[i];
        ((float*)v)[e] = vbuf[i];
      } else if (flags & ORC_F24_MOMENTS) {
        orc_f24_encode1(mbuf[i], (uint8_t*)m + 3 * e);
        orc_f24_encode1(vbuf[i], (uint8_t*)v + 3 * e);
      }
    }
    if (!(flags & (ORC_FP32_MOMENTS | ORC_F24_MOMENTS))) {
      orc_encode_block(mbuf, L, ORC_SIGNED, (uint16_t*)m + base, &ms[b]);
      orc_encode_block(vbuf, L, ORC_UNSIGNED, (uint16_t*)v + base, &vs[b]);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Factored second moment with update clipping [ADAF; PRODIGY]              */
/* ------------------------------------------------------------------------ */

/* beta2 of update t: the constant, or Adafactor's schedule 1 - t^decay_rate;
 * each of B2 and C2 = 1 - beta2 rounded once from double. */
static void f_beta2(const orc_fhparams* hp, int64_t t, float* B2, float* C2) {
  double b2 = hp->decay_rate != 0.0 ? 1.0 - pow((double)t, hp->decay_rate) : hp->beta2;
  *B2 = (float)b2;
  *C2 = (float)(1.0 - b2);
}

/* The optional first moment [ADAF]: an EMA of the clipped, lr-scaled update x
 * (before weight decay) replaces x. The block's values go to mbuf for the
 * signed-codec encode. */
static float f_first_moment(float x, const uint16_t* mc, const float* ms, int64_t e, float B1, float C1,
                            float* mbuf) {
  float m0 = orc_decode1(mc[e], ms[e / ORC_BLOCK], ORC_SIGNED);
  float m = fmaf(B1, m0, C1 * x);
  mbuf[e % ORC_BLOCK] = m;
  return m;
}

/* Master weight and split of the factored step; STOCHASTIC as in the (N)AdamW
 * step (no residual, random bits keyed on seed, update number, tensor). */
static float f_join(const uint16_t* hi, const uint16_t* lo, int64_t e, const orc_fhparams* hp) {
  return join_at(hi, lo, e, hp->split_mode);
}

static void f_split(float w, uint16_t* hi, uint16_t* lo, int64_t e, const orc_fhparams* hp, int64_t step) {
  if (hp->split_mode == ORC_SPLIT_STOCHASTIC)
    hi[e] = orc_sr_bf16(w, orc_sr_rand16(hp->seed, step, hp->tensor, e));
  else
    orc_split1(u_of(w), &hi[e], &lo[e], hp->split_mode);
}

/* Update clipping factor: lr / max(1, RMS(U) / d) with RMS over the tensor. */
static float clip_factor(double sum_sq, int64_t n, const orc_fhparams* hp) {
  double rms = sqrt(sum_sq / (double)n);
  double r = rms / hp->clip_threshold;
  return (float)(hp->lr / (r > 1.0 ? r : 1.0));
}

/* 2-D tensor [R, C] (row-major). row[R] and col[C] hold the EMAs of the row
 * and column means of g^2 + eps1. */
void orc_factored_2d(uint16_t* hi, uint16_t* lo, const uint16_t* g, float* row, float* col, uint16_t* mc, float* ms,
                     int64_t R, int64_t C, const orc_fhparams* hp, int64_t step) {
  if (!g) return;
  float B2, C2, EPS1 = (float)hp->eps1;
  f_beta2(hp, step, &B2, &C2);
  int fm = hp->beta1 != 0.0;
  float B1 = (float)hp->beta1, C1 = (float)(1.0 - hp->beta1), mbuf[ORC_BLOCK];
  float CWD = (float)(hp->lr * hp->weight_decay);
  int wd = hp->weight_decay != 0.0;
  double* rs = (double*)calloc((size_t)R, sizeof(double));
  double* cs = (double*)calloc((size_t)C, sizeof(double));
  float* rho = (float*)malloc((size_t)R * sizeof(float));
  float* kap = (float*)malloc((size_t)C * sizeof(float));
  /* 1. means of q = g^2 + eps1 over each row and column, then the EMAs */
  for (int64_t i = 0; i < R; ++i)
    for (int64_t j = 0; j < C; ++j) {
      float gf = orc_bf16_to_f32(g[i * C + j]);
      float q = gf * gf + EPS1;
      rs[i] += (double)q;
      cs[j] += (double)q;
    }
  for (int64_t i = 0; i < R; ++i) row[i] = fmaf(B2, row[i], C2 * (float)(rs[i] / (double)C));
  for (int64_t j = 0; j < C; ++j) col[j] = fmaf(B2, col[j], C2 * (float)(cs[j] / (double)R));
  /* 2. V_ij = r_i c_j / mean(r); its inverse square root as two factors */
  double rsum = 0.0;
  for (int64_t i = 0; i < R; ++i) rsum += (double)row[i];
  float rbar = (float)(rsum / (double)R);
  for (int64_t i = 0; i < R; ++i) rho[i] = 1.0f / sqrtf(row[i] / rbar);
  for (int64_t j = 0; j < C; ++j) kap[j] = 1.0f / sqrtf(col[j]);
  /* 3. the clip factor from RMS(U), U^2 = g^2 / V = g^2 * mean(r) / (r_i c_j)
   *    evaluated in double */
  double rmean = rsum / (double)R, su = 0.0;
  for (int64_t i = 0; i < R; ++i)
    for (int64_t j = 0; j < C; ++j) {
      double gd = (double)orc_bf16_to_f32(g[i * C + j]);
      su += gd * gd * rmean / ((double)row[i] * (double)col[j]);
    }
  float f = clip_factor(su, R * C, hp);
  /* 4. apply to the joined master weight and split again; with a first
   *    moment, re-encode each 256-element block of the flattened tensor */
  for (int64_t i = 0; i < R; ++i)
    for (int64_t j = 0; j < C; ++j) {
      int64_t e = i * C + j;
      float U = (orc_bf16_to_f32(g[e]) * rho[i]) * kap[j];
      float w = f_join(hi, lo, e, hp);
      float x = U * f;
      if (fm) x = f_first_moment(x, mc, ms, e, B1, C1, mbuf);
      if (wd) x = fmaf(CWD, w, x);
      f_split(w - x, hi, lo, e, hp, step);
      if (fm && (e % ORC_BLOCK == ORC_BLOCK - 1 || e == R * C - 1)) {
        int64_t b = e / ORC_BLOCK;
        orc_encode_block(mbuf, (int)(e - b * ORC_BLOCK + 1), ORC_SIGNED, mc + b * ORC_BLOCK, &ms[b]);
      }
    }
  free(rs);
  free(cs);
  free(rho);
  free(kap);
}

/* 1-D tensor: unfactored second moment kept in the uint16 codec. */
void orc_factored_1d(uint16_t* hi, uint16_t* lo, const uint16_t* g, uint16_t* vc, float* vs, uint16_t* mc,
                     float* ms, int64_t n, const orc_fhparams* hp, int64_t step) {
  if (!g) return;
  float B2, C2, EPS1 = (float)hp->eps1;
  f_beta2(hp, step, &B2, &C2);
  int fm = hp->beta1 != 0.0;
  float B1 = (float)hp->beta1, C1 = (float)(1.0 - hp->beta1), mbuf[ORC_BLOCK];
  float CWD = (float)(hp->lr * hp->weight_decay);
  int wd = hp->weight_decay != 0.0;
  float* v = (float*)malloc((size_t)n * sizeof(float));
  double su = 0.0;
  for (int64_t e = 0; e < n; ++e) {
    float gf = orc_bf16_to_f32(g[e]);
    float q = gf * gf + EPS1;
    v[e] = fmaf(B2, orc_decode1(vc[e], vs[e / ORC_BLOCK], ORC_UNSIGNED), C2 * q);
    su += (double)gf * (double)gf / (double)v[e];   /* U^2 = g^2 / v in double */
  }
  float f = clip_factor(su, n, hp);
  for (int64_t e = 0; e < n; ++e) {
    float U = orc_bf16_to_f32(g[e]) * (1.0f / sqrtf(v[e]));
    float w = f_join(hi, lo, e, hp);
    float x = U * f;
    if (fm) x = f_first_moment(x, mc, ms, e, B1, C1, mbuf);
    if (wd) x = fmaf(CWD, w, x);
    f_split(w - x, hi, lo, e, hp, step);
    if (fm && (e % ORC_BLOCK == ORC_BLOCK - 1 || e == n - 1)) {
      int64_t b = e / ORC_BLOCK;
      orc_encode_block(mbuf, (int)(e - b * ORC_BLOCK + 1), ORC_SIGNED, mc + b * ORC_BLOCK, &ms[b]);
    }
  }
  orc_encode(v, n, ORC_UNSIGNED, vc, vs);
  free(v);
}
