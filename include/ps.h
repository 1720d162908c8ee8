/* ps.h - C ABI of the MI355X (gfx950) fused low-precision optimizer step.
 *
 * One shared library, libps.so, built from precision_state_amd/csrc. Every
 * entry point is extern "C", takes plain pointers and sizes, and returns a
 * ps_status. Device pointers are HIP device memory (any allocator); calls are
 * asynchronous and ordered on the HIP stream passed in (NULL = the default
 * stream); nothing here synchronises unless stated.
 *
 * Pages this library implements (cited by title and section):
 *  [KAHAN]   kohya-ss/sd-scripts PR #2159, "Kahan summation for
 *            Adafactor-optimized Flux FFT": keep the 16 low bits that the bf16
 *            weight drops, restore the exact fp32 value before each update.
 *  [NADAM]   kohya-ss/sd-scripts PR #2187, "(N)AdamW / Adan with fused
 *            backwards pass & CPU offloading": opening post (AdamW / NAdamW
 *            with Kahan residuals, moments offloaded to host memory) and second
 *            post (moments stored as scaled, biased, pow()-companded uint16).
 *  [ADAF]    kohya-ss/sd-scripts commit 7983d3d, "Fused backward pass",
 *            library/adafactor_fused.py (factored second moment, update
 *            clipping, tensors without a gradient skipped).
 *  [PRODIGY] konstmish/prodigy PR #25, "no first moment and factored second
 *            moment" (beta1 = 0, factored v, update clipping, eps on g^2).
 *
 * Arithmetic contract (all kernels): IEEE binary32, round to nearest even,
 * fused multiply-add only where the formula below says fma, correctly
 * rounded division and square root, denormals preserved. Inputs are assumed
 * finite; results for non-finite inputs are unspecified.
 *
 * Error behaviour: every argument is validated on the host before any HIP
 * call, so a rejected call touches no device state and needs no GPU. A HIP
 * failure at launch returns PS_ERR_HIP. ps_last_error() gives a message for
 * the calling thread's most recent failure.
 */
#ifndef PS_H
#define PS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* ps_stream_t;

typedef int32_t ps_status;
enum {
  PS_OK = 0,
  PS_ERR_INVALID_ARG = 1, /* NULL where a pointer is required, bad enum, bad hyperparameter */
  PS_ERR_ALIGNMENT = 2,   /* a 16-bit or fp32 array not 16-byte aligned (scales: 4 bytes) */
  PS_ERR_SHAPE = 3,       /* numel < 0, rows * cols != numel, sizes out of range */
  PS_ERR_UNSUPPORTED = 4, /* valid but not implemented combination */
  PS_ERR_HIP = 5,         /* the HIP runtime reported an error */
  PS_ERR_NO_MEMORY = 6,   /* host or device allocation failed */
  PS_ERR_WORKSPACE = 7    /* caller workspace smaller than required */
};

enum { PS_ALGO_ADAM = 0, PS_ALGO_NADAM = 1 };
enum { PS_SPLIT_TRUNC = 0, PS_SPLIT_NEAREST_AWAY = 1, PS_SPLIT_STOCHASTIC = 2 };
enum { PS_MOMENT_SIGNED = 0, PS_MOMENT_UNSIGNED = 1 };

/* Elements per moment-scale block. */
#define PS_BLOCK 256

/* Per-tensor storage flags (ps_tensor.flags) [NADAM, second post: tensors of
 * at most 4096 elements keep fp32 moments; third post: the final layer trains
 * in fp32]. The update arithmetic is unchanged; only the storage differs.
 *   PS_TENSOR_FP32_MOMENTS  m_code and v_code point to float[numel] moments
 *                           (no codec); m_scale and v_scale are not used
 *   PS_TENSOR_FP32_PARAM    w_hi points to the float[numel] parameter and grad
 *                           to a float[numel] gradient (no residual); w_lo is
 *                           not used
 *   PS_TENSOR_F24_MOMENTS   [NADAM, third post: moments in the upper three
 *                           bytes of fp32] m_code and v_code point to
 *                           uint8[3 * numel]: value i is bytes 3i..3i+2, the
 *                           fp32 word's bits 8..31 little-endian (low byte
 *                           implied zero), rounded to nearest, ties to even;
 *                           m_scale and v_scale are not used. Excludes
 *                           PS_TENSOR_FP32_MOMENTS.
 * Supported by ps_opt_step_multi only (the factored step and the offload
 * pipeline reject non-zero flags with PS_ERR_UNSUPPORTED). */
enum { PS_TENSOR_FP32_MOMENTS = 1u << 0, PS_TENSOR_FP32_PARAM = 1u << 1, PS_TENSOR_F24_MOMENTS = 1u << 2 };

/* One parameter tensor's state. All arrays are device memory owned by the
 * caller, contiguous, `numel` elements unless noted; 16-bit and fp32 element
 * arrays must be 16-byte aligned, scale arrays 4-byte aligned.
 *   w_hi    bf16 weight bits (the model's parameter), read and written
 *   w_lo    uint16 residual: the fp32 master weight's low half [KAHAN]
 *   grad    bf16 gradient bits, read only; NULL skips the tensor [ADAF]
 *   m_code  exp_avg codes, signed kind (32768 +- k); unused by the factored step
 *   m_scale exp_avg block scales, ceil(numel / 256) floats
 *   v_code  exp_avg_sq codes, unsigned kind (k)
 *   v_scale exp_avg_sq block scales, ceil(numel / 256) floats
 *   row_ema, col_ema  factored step only: fp32[rows], fp32[cols]
 *   rows, cols        factored step only: rows * cols == numel for a 2-D
 *                     tensor (factored), both 0 for a 1-D tensor (v kept in
 *                     v_code / v_scale)
 * flags       PS_TENSOR_* storage flags (0: the formats above); reserved = 0
 * A tensor with numel == 0 is skipped and its pointers are not read. */
typedef struct ps_tensor {
  uint16_t* w_hi;
  uint16_t* w_lo;
  const uint16_t* grad;
  uint16_t* m_code;
  float* m_scale;
  uint16_t* v_code;
  float* v_scale;
  float* row_ema;
  float* col_ema;
  int64_t numel;
  int64_t rows;
  int64_t cols;
  uint32_t flags;
  uint32_t reserved;
} ps_tensor;

/* (N)AdamW hyperparameters [NADAM]. Constraints: algo in {ADAM, NADAM};
 * split_mode in {TRUNC, NEAREST_AWAY, STOCHASTIC}; lr >= 0; 0 <= beta1 < 1;
 * 0 <= beta2 < 1; eps > 0 and nonzero once rounded to fp32;
 * weight_decay >= 0; momentum_decay >= 0 (NAdam's psi, 0.004 by default);
 * all finite.
 *
 * split_mode STOCHASTIC [KAHAN, PR #2159 body: the stochastic rounding the
 * residual replaces; NADAM opening post]: no residual. w_lo is neither read
 * nor written (may be NULL); the master weight is the bf16 value itself, and
 * the updated fp32 weight w' is rounded to one of its two neighbouring bf16
 * values, away from zero with probability (low 16 bits of w') / 2^16:
 *   hi = (bits(w') + r) >> 16
 * with r the element's random 16 bits. They come from a SplitMix64 stream
 * (Steele, Lea, Flood, OOPSLA 2014; mix(z) = its output finaliser, G =
 * 0x9E3779B97F4A7C15): for the tensor at index i of the list and update
 * `step`, the stream starts at s = mix(seed ^ mix((step mod 2^32) << 32 | i));
 * element e takes bits 16*(e % 4) .. 16*(e % 4) + 15 of mix(s + (e/4 + 1) * G).
 * The same (seed, step, list position) always gives the same bits, so a
 * caller that steps one tensor per call (position 0 every time, as from a
 * gradient hook) should give each tensor a seed of its own, or all of them
 * draw the same stream. Supported by ps_opt_step_multi, the factored step
 * (ps_factored_hparams.seed) and the offload pipeline (which then moves no
 * residual); ps_split and ps_join return PS_ERR_UNSUPPORTED for it. `seed`
 * is not read in the other modes. */
typedef struct ps_hparams {
  int32_t algo;
  int32_t split_mode;
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
  double momentum_decay;
  uint64_t seed;
} ps_hparams;

/* Factored-second-moment hyperparameters [ADAF; PRODIGY]: eps1 added to g^2,
 * update clipped to RMS clip_threshold.
 *   decay_rate  0: constant beta2. < 0: Adafactor's schedule [ADAF]: beta2 of
 *               update t is 1 - t^decay_rate (beta2 is then ignored); B2 and
 *               C2 = 1 - beta2_t are each rounded once from double
 *   beta1       0: no first moment [PRODIGY]. In (0, 1): the clipped,
 *               lr-scaled update x is replaced by its EMA m = fma(B1, m0, C1*x)
 *               (B1 = fp32(beta1), C1 = fp32(1 - beta1)) before weight decay
 *               [ADAF], m kept in m_code / m_scale (signed codec, per-256
 *               blocks of the flattened tensor); 2-D tensors then need
 *               numel < 2^31 (else PS_ERR_UNSUPPORTED)
 *   split_mode  TRUNC, NEAREST_AWAY, or STOCHASTIC (no residual; the random
 *               bits exactly as for ps_hparams, from `seed`, the update
 *               number and the tensor's index in the list)
 * Constraints: lr >= 0; 0 <= beta2 < 1; eps1 > 0 and nonzero once rounded to fp32;
 * clip_threshold > 0; weight_decay >= 0; decay_rate <= 0;
 * 0 <= beta1 < 1; all finite. */
typedef struct ps_factored_hparams {
  int32_t split_mode;
  int32_t reserved; /* must be 0 */
  double lr;
  double beta2;
  double eps1;
  double clip_threshold;
  double weight_decay;
  double decay_rate;
  double beta1;
  uint64_t seed;
} ps_factored_hparams;

/* ps_opt_step_multi - one fused (N)AdamW step over a list of tensors, in ONE
 * kernel launch [NADAM; KAHAN].
 * Per element, for update number `step` (>= 1, the first update is 1 [ADAF]):
 *   w   = join(w_hi, w_lo)                      exact fp32 master weight
 *   g   = fp32(grad)
 *   m0  = decode(m_code, m_scale), v0 = decode(v_code, v_scale)
 *   m   = fma(B1, m0, C1*g);  v = fma(B2, v0, C2*(g*g))
 *   d   = fma(sqrt(v), RS2, EPS)
 *   ADAM:  u = A*(m/d)             NADAM: u = fma(AG, g, AM*m)/d
 *   if weight_decay != 0: u = fma(CWD, w, u)    (decoupled, additive form)
 *   w'  = w - u;  (w_hi, w_lo) = split(w')
 *   new block scales = max|m|, max v over each 256-element block of this
 *   step's fp32 moments; codes re-encoded with them.
 * Scalars (ps_step_scalars) are computed on the host in double and rounded
 * once. `tensors` is a host array of n_tensors records (n_tensors == 0 is a
 * no-op); it is copied during the call. Lists of up to 16 records travel in
 * the kernel arguments; for longer lists, and for the records with storage
 * flags, the library keeps a device copy of each distinct list it has seen,
 * so repeated calls with the same list upload nothing. That cache holds up
 * to 16384 lists or 64 MiB per device; when it is full, the call waits
 * until no other call is between taking a cached list and enqueueing the
 * launch that reads it, then synchronizes the device once and empties it. Tensors with storage flags go
 * to a second launch with a generic-format kernel. Calls from several host
 * threads, on their own streams and over distinct tensors, are safe.
 * Errors: PS_ERR_INVALID_ARG, PS_ERR_ALIGNMENT, PS_ERR_SHAPE (host checks,
 * before any device work); PS_ERR_HIP; PS_ERR_NO_MEMORY. */
ps_status ps_opt_step_multi(const ps_tensor* tensors, int32_t n_tensors, const ps_hparams* hp, int64_t step,
                            ps_stream_t stream);

/* ps_step_scalars - the fp32 scalars of update number `step`, as used by
 * ps_opt_step_multi: out[0..9] = B1, C1, B2, C2, EPS, A, RS2, AG, AM, CWD.
 * Host only (no GPU needed). */
ps_status ps_step_scalars(const ps_hparams* hp, int64_t step, float out[10]);

/* ps_split / ps_join - fp32 master weight <-> (bf16 weight, uint16 residual)
 * [KAHAN, copy_kahan_ docstring]. Elementwise over n >= 0 elements.
 *   TRUNC:        hi = bits >> 16, lo = bits & 0xFFFF (bf16 truncated toward 0)
 *   NEAREST_AWAY: hi = ((bits + 0x8000) >> 16) & 0xFFFF (bf16 rounded to
 *                 nearest, ties away from zero), lo = bits & 0xFFFF
 * join inverts split exactly for every 32-bit pattern in both modes. */
ps_status ps_split(const float* w32, uint16_t* hi, uint16_t* lo, int64_t n, int32_t mode, ps_stream_t stream);
ps_status ps_join(const uint16_t* hi, const uint16_t* lo, float* w32, int64_t n, int32_t mode,
                  ps_stream_t stream);

/* ps_encode_moments / ps_decode_moments - the uint16 moment codec [NADAM,
 * second post], 1/4-power companding, one fp32 scale per 256-element block
 * (the last block of the array covers n mod 256 elements).
 * Encode, per block: s = max |x|; if s < 2^-126 then scale = 0 and every
 * code is the zero code (SIGNED 32768, UNSIGNED 0); else inv = 1/s and for
 * each element x' = |x|*inv and k = the largest k in 0..Q with k == 0 or
 * x' >= D(k - 1/2), where D(h) = ((h*K)^2)^2, K = fp32(1/Q), Q = 32767
 * (SIGNED) or 65535 (UNSIGNED). SIGNED code = 32768 - k for x < 0 else 32768 + k;
 * UNSIGNED code = k (the sign of x is ignored).
 * Decode: SIGNED x = sign(c - 32768) * D(|c - 32768|) * s; UNSIGNED x = D(c) * s.
 * scale has ceil(n / 256) entries. */
ps_status ps_encode_moments(const float* x, uint16_t* code, float* scale, int64_t n, int32_t kind,
                            ps_stream_t stream);
ps_status ps_decode_moments(const uint16_t* code, const float* scale, float* x, int64_t n, int32_t kind,
                            ps_stream_t stream);

/* ps_factored_workspace_size - device workspace bytes ps_factored_step needs
 * for this tensor list (partial row/column sums and per-tensor reductions).
 * Host only. */
ps_status ps_factored_workspace_size(const ps_tensor* tensors, int32_t n_tensors, size_t* bytes);
/* (The workspace does not depend on the hyperparameters: a first moment lives
 * in the tensors' m_code / m_scale.) */

/* ps_factored_step - Adafactor-style step [ADAF; PRODIGY]. For a 2-D tensor
 * [rows, cols] (row-major):
 *   q_ij = g_ij*g_ij + EPS1
 *   r_i = fma(B2, r_i, C2*fp32(mean_j q_ij)),  c_j = fma(B2, c_j, C2*fp32(mean_i q_ij))
 *   rbar = fp32(mean_i r_i); rho_i = 1/sqrt(r_i/rbar); kap_j = 1/sqrt(c_j)
 *   U_ij = (g_ij*rho_i)*kap_j; f = fp32(lr / max(1, RMS/clip_threshold)),
 *     RMS = sqrt(mean_ij g_ij^2 * mean_i(r_i) / (r_i c_j)) in double: the RMS
 *     of the exact U for the new EMAs
 *   x = U*f; with beta1: m = fma(B1, decode(m), C1*x), x = m, m re-encoded
 *   w' = w - x after x = fma(CWD, w, x) if weight_decay != 0
 * Means and RMS are accumulated in double. A 1-D tensor keeps v in the
 * uint16 codec: v = fma(B2, decode(v), C2*q); U = g*(1/sqrt(v)); the clip's
 * RMS = sqrt(mean g^2 / v) in double.
 * workspace: device memory of at least ps_factored_workspace_size bytes,
 * 256-byte aligned, owned by the caller; its contents on entry are ignored;
 * calls that may run at the same time need distinct workspaces. The step's
 * device plan goes through the same cache as ps_opt_step_multi's lists.
 * Errors as ps_opt_step_multi, plus PS_ERR_WORKSPACE. */
ps_status ps_factored_step(const ps_tensor* tensors, int32_t n_tensors, const ps_factored_hparams* hp,
                           int64_t step, void* workspace, size_t workspace_bytes, ps_stream_t stream);

/* ps_factored_step_noalloc - for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): ps_factored_step with no workspace argument and no device
 * allocation. The plan and the workspace go to a scratch array that the
 * library keeps in each GPU's memory for the life of the process,
 * PS_NOALLOC_SCRATCH_BYTES per GPU (its address is looked up on the first
 * call on each device). The plan, rounded up to 256 bytes, plus
 * ps_factored_workspace_size must fit in it, else the call returns
 * PS_ERR_WORKSPACE before any device work; one FLUX double block (24 tensors,
 * 22.0 MiB of workspace) fits. The plan reaches the scratch through kernel
 * arguments, so the call makes no copy from host memory either. Same kernels
 * and results as ps_factored_step; the scratch's contents on entry are
 * ignored. Every call on one GPU uses that GPU's single scratch array: calls
 * ordered on one stream are safe, calls that may overlap on one GPU (other
 * streams or host threads without ordering between them) race and must not
 * be made. Errors as ps_factored_step. */
#define PS_NOALLOC_SCRATCH_BYTES (32u << 20)
ps_status ps_factored_step_noalloc(const ps_tensor* tensors, int32_t n_tensors, const ps_factored_hparams* hp,
                                   int64_t step, ps_stream_t stream);

/* Host-offload pipeline [NADAM, opening post: moments (and here the
 * residuals) live in host memory and cross PCIe every step].
 * A group is one set of tensors stepped together (e.g. one transformer
 * block). For every tensor, w_hi and grad are device pointers; w_lo, m_code,
 * m_scale, v_code and v_scale are PINNED HOST pointers (hipHostMalloc).
 * ps_offload_run steps the groups in order. In the STAGED mode group k's
 * host state is copied to a device staging slot on an upload stream, stepped,
 * and copied back on a download stream, with two slots so that uploads of
 * k+1 and downloads of k-1 overlap the step of k; in the DIRECT mode the step
 * kernel of group k works on the host arrays in place. The results are bit-identical
 * to ps_opt_step_multi on device-resident state (for stochastic rounding:
 * on the concatenation of the groups' tensor lists, whose positions key the
 * random streams).
 * Streams: STAGED makes an upload and a download stream, each created with a
 * CU mask (all CUs) so that each gets a hardware queue of its own and the two
 * directions overlap whatever other streams the process holds, and a
 * non-blocking stream for the step kernels; DIRECT makes one stream with a
 * CU mask of n_cus CUs for its kernels. Streams made with a CU mask are
 * blocking: they order themselves with the null stream of the device.
 * Stochastic rounding [NADAM, opening post: the stochastic updates used when
 * the residual does not fit in host memory]: runs with split_mode STOCHASTIC
 * move no residuals; w_lo may then be NULL, and a plan with any NULL w_lo
 * accepts only such runs (PS_ERR_INVALID_ARG otherwise). */
typedef struct ps_offload_group {
  const ps_tensor* tensors;
  int32_t n_tensors;
} ps_offload_group;

typedef struct ps_offload_plan ps_offload_plan;

/* Plan modes.
 *   PS_OFFLOAD_DIRECT  the step kernel reads and writes the host-resident
 *                      arrays in place over PCIe (through the device addresses
 *                      of the pinned allocations, hipHostGetDevicePointer), one
 *                      launch per group on a stream of the plan's own that is
 *                      restricted to n_cus compute units: no staging memory and
 *                      no copy engines; the rest of the GPU stays free for
 *                      other work
 *   PS_OFFLOAD_STAGED  two device staging slots, an upload and a download
 *                      stream (each with a hardware queue of its own) and the
 *                      step kernel on a third stream, as described above
 * Both move the same bytes over PCIe and give the same results. */
enum { PS_OFFLOAD_DIRECT = 0, PS_OFFLOAD_STAGED = 1 };
#define PS_OFFLOAD_DEFAULT_CUS 8
typedef struct ps_offload_options {
  int32_t mode;      /* PS_OFFLOAD_DIRECT or PS_OFFLOAD_STAGED */
  int32_t n_cus;     /* DIRECT: compute units the step kernels may use (0: all) */
  int32_t reserved0; /* must be 0 */
  int32_t reserved1; /* must be 0 */
} ps_offload_options;

/* Creates the plan: copies the group descriptions and builds the device
 * tables, streams and events. DIRECT also checks that every host array has a
 * device address; STAGED allocates two staging slots sized for the largest
 * group. Synchronous. options NULL: DIRECT on PS_OFFLOAD_DEFAULT_CUS compute
 * units. ps_offload_plan_create(g, n, p) is ps_offload_plan_create_ex(g, n,
 * NULL, p). */
ps_status ps_offload_plan_create(const ps_offload_group* groups, int32_t n_groups, ps_offload_plan** plan);
ps_status ps_offload_plan_create_ex(const ps_offload_group* groups, int32_t n_groups,
                                    const ps_offload_options* options, ps_offload_plan** plan);
/* Runs one optimizer step over all groups; asynchronous on `stream` (the
 * call returns once all work is queued; host state is final when `stream`
 * completes). Successive runs of one plan are ordered among themselves even
 * when given different streams; one plan must not be run from two host
 * threads at once. */
ps_status ps_offload_run(ps_offload_plan* plan, const ps_hparams* hp, int64_t step, ps_stream_t stream);
/* Bytes the most recent run moved host->device and device->host (before
 * any run: the bytes of a run with residuals). */
ps_status ps_offload_bytes(const ps_offload_plan* plan, uint64_t* h2d_bytes, uint64_t* d2h_bytes);
/* Waits for outstanding work and frees everything the plan owns. */
ps_status ps_offload_plan_destroy(ps_offload_plan* plan);

/* Static description of a status code. */
const char* ps_status_string(ps_status status);
/* Message of the calling thread's most recent failed call ("" if none). */
const char* ps_last_error(void);
/* Library version string. */
const char* ps_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PS_H */
