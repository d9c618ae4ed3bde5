/*
 * ssm_ternary.h -- C ABI of the MI355X (gfx950) ternary selective-SSM mixer forward.
 *
 * What is computed (cited by page title and section):
 *  - "Associative Recall Under Ternary Quantization ... at 5M Parameters" (TriSSM
 *    repository README), intro and BitSSM mixer paragraphs: the Delta, B, C
 *    projections of a selective SSM are BitNet b1.58 BitLinear layers (ternary
 *    weights, int8 activations); an RMSNorm precedes each ternary projection; the
 *    recurrence is evaluated with a parallel associative scan.
 *  - "Ternary Mamba: Grouped Quantization-Aware Training of W1.58A16 State Space
 *    Models", abstract: per-group ternary scales with unquantised (16-bit)
 *    activations (W1.58A16) on a Mamba-2 (SSD) model; the zero ratio of the codes.
 *  - "Ternary State-Space Models ...", Key Points / Abstract: weights in {-1,0,+1},
 *    multiply-free (add/subtract/skip) inference, SSM parallel scan.
 *  - Works cited by title in "Baseline Shape Decides the Verdict ..." (Builds on):
 *    BitNet b1.58 (absmean weight scale, absmax int8 activations) and Mamba
 *    (softplus Delta, exp(Delta A) discretisation, selective recurrence); in
 *    "SSDi8 ..." (Builds on): "Transformers are SSMs" (scalar A per head, SSD).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must be device memory of the current HIP
 *    device; the caller owns all memory (inputs, outputs, weights, workspace).  The
 *    library never allocates or frees device memory and keeps no device state.
 *  - Work is enqueued on `stream` and runs asynchronously: no entry point
 *    synchronises or copies to the host.
 *  - Activations are token-major, row-major: element (token m, column c) is at
 *    m * ld + c, token m = b * L + t for batch b and position t.
 *  - Shapes, strides, dtypes and alignments are validated on the host before
 *    anything is launched; a failing call launches nothing and returns a status
 *    other than SSM_OK, with a message in ssm_last_error().  A failure reported by
 *    the HIP runtime at launch returns SSM_ERR_DEVICE.  Nothing throws or aborts.
 *  - Outputs must not overlap inputs unless an entry point says otherwise.
 *  - Calls are thread-safe; the only global state is a thread-local error string.
 *  - Results do not depend on the launch configuration or on earlier calls: every
 *    integer stage is exact and every float reduction has a fixed order.
 */
#ifndef SSM_TERNARY_H
#define SSM_TERNARY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 7

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer is NULL */
  SSM_ERR_SHAPE = 2,       /* a size or stride is out of range or inconsistent */
  SSM_ERR_DTYPE = 3,       /* dtype not supported for this argument */
  SSM_ERR_ALIGN = 4,       /* a pointer or stride is not aligned as required */
  SSM_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the *_workspace_bytes value */
  SSM_ERR_UNSUPPORTED = 6, /* valid request this library does not implement */
  SSM_ERR_DEVICE = 7       /* the HIP runtime reported an error */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1, SSM_I8 = 2 } ssm_dtype;

/* Version of this ABI and of the packed weight format (bumps when either changes). */
int ssm_abi_version(void);
/* Static description of a status code. */
const char* ssm_status_string(int status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* ssm_last_error(void);

/*
 * Packed ternary weights (2 bits per weight).  The pages fix no storage format; this
 * is the library's: a row of k weights occupies ssm_packed_row_bytes(k) =
 * 4 * ceil(k / 16) bytes of little-endian 32-bit words, each word holding 16
 * consecutive weights of the row.  Weight i of a word (i = 4 j + p, 0 <= j, p < 4)
 * sits in byte p at bits 2j..2j+1: code 0b00 = 0, 0b01 = +1, 0b11 = -1 (0b10 is never
 * written).  Weights past k in a row's last word are 0.  A tensor [n_out, k] is
 * n_out such rows back to back, row-major.
 */
int64_t ssm_packed_row_bytes(int64_t k);

/*
 * ssm_ternary_quantize_weights -- absmean ternarisation and 2-bit packing (BitNet b1.58
 * absmean scale; per-group scales from the Ternary Mamba abstract; the zero ratio it
 * monitors).
 *   w_latent   device fp32 [n_out, k] row-major latent weights.
 *   group_size 0: one scale gamma = mean|W| for the tensor; > 0: one scale per run of
 *              group_size consecutive weights of a row (k % group_size == 0).  The sum
 *              of |w| is taken in fp64, each row (or row-group) in ascending k, the
 *              row sums of a per-tensor scale in ascending row order; gamma is the fp32
 *              rounding of sum / count.
 *   scale_in   NULL: absmean scales as above.  Else device fp32, shaped like w_scale:
 *              caller-supplied (e.g. learned) scales, used and copied as given.
 *   w_packed   device out, n_out * ssm_packed_row_bytes(k) bytes.  Codes are
 *              clamp(round_half_even(w / max(gamma, 1e-5)), -1, 1), fp32 IEEE division.
 *   w_scale    device fp32 out, [1] or [n_out, k / group_size].
 *   zero_count NULL or device int64 out: number of zero codes (overwritten).
 *   workspace  device memory of ssm_ternary_quantize_workspace_bytes() bytes (fp64 row
 *              sums); may be NULL when that size is 0.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE (n_out < 1, k < 1, k % group_size != 0),
 * SSM_ERR_WORKSPACE, SSM_ERR_DEVICE.
 */
size_t ssm_ternary_quantize_workspace_bytes(int64_t n_out, int64_t k, int64_t group_size,
                                            const float* scale_in);
ssm_status ssm_ternary_quantize_weights(const float* w_latent, int64_t n_out, int64_t k,
                                        int64_t group_size, const float* scale_in,
                                        uint8_t* w_packed, float* w_scale, int64_t* zero_count,
                                        void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * ssm_bitlinear_fwd -- RMSNorm -> activation quantisation -> ternary contraction ->
 * rescale (TriSSM README: BitLinear with ternary weights and int8 activations, an
 * RMSNorm before each ternary projection; W1.58A16 from the Ternary Mamba abstract).
 * For each row m of x (the first k columns; row stride ldx):
 *   r = 1 / sqrt(mean_k x^2 + norm_eps), fp32, summed as 64 partials (partial j takes
 *       columns j, j+64, ... in ascending order with fused multiply-adds from 0) that
 *       are then combined pairwise at distances 32, 16, 8, 4, 2, 1;
 *   xh = (x * r) * norm_weight (fp32; no multiply when norm_weight is NULL).
 *   act_bits 8 (A8): a = max|xh|; q = clamp(round_half_even(xh * (127 / max(a, 1e-5))),
 *       -128, 127) int8; acc = sum_k q * w (int32, exact: the multiply-free
 *       add/subtract/skip sum); y = (s_w * acc) * (max(a, 1e-5) / 127) evaluated in fp64
 *       (per group: the fp64 sum over groups, in order, of s[n, g] * acc_g), plus bias,
 *       plus residual, rounded once to fp32 (then to bf16 for a bf16 output).
 *   act_bits 16 (A16): y = sum_groups s[n, g] * sum_{k in g} xh * w with xh carried as
 *       bf16 (bf16 output) or as the sum of two bf16 terms (fp32 output), fp32
 *       accumulation; no activation quantisation.  Then + bias + residual.
 * x_dtype SSM_I8 (A8 only): x already holds int8 codes and x_absmax their per-row
 * absmax a; the norm and quantisation are skipped.
 * Optional stage outputs (A8 only; each NULL or a device buffer): dbg_xq int8 [m, k],
 * dbg_absmax fp32 [m], dbg_acc int32 [m, n_out] (sum over all groups).  dbg_xq and
 * dbg_absmax are written only when the norm runs (x_dtype F32 or BF16).
 * Requirements: 1 <= k <= 4096; 1 <= n_out; m >= 0 (m == 0 launches nothing);
 * ldx >= k, ldy >= n_out, ld_res >= n_out; group_size 0 or a multiple of 64 dividing k;
 * act_bits 16 requires x_dtype F32 or BF16; residual has y_dtype; w_packed 4-byte
 * aligned; int8 input needs k % 64 == 0, ldx % 16 == 0 and 16-byte alignment.
 * workspace: ssm_bitlinear_workspace_bytes() bytes, 16-byte aligned (0 for int8 input).
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_WORKSPACE,
 * SSM_ERR_UNSUPPORTED, SSM_ERR_DEVICE.
 */
typedef struct {
  const void* x;
  int32_t x_dtype; /* ssm_dtype */
  int32_t act_bits;
  int64_t m, k, ldx;
  const float* x_absmax;    /* [m], required iff x_dtype == SSM_I8 */
  const float* norm_weight; /* [k] RMSNorm gains or NULL (ones) */
  float norm_eps;
  int32_t pad0;
  const uint8_t* w_packed;  /* [n_out, ssm_packed_row_bytes(k)] */
  const float* w_scale;     /* [1] or [n_out, k / group_size] */
  int64_t n_out, group_size;
  const float* bias;        /* [n_out] or NULL */
  const void* residual;     /* [m, ld_res] of y_dtype, or NULL */
  int64_t ld_res;
  void* y;
  int32_t y_dtype;          /* SSM_F32 or SSM_BF16 */
  int32_t pad1;
  int64_t ldy;
  int8_t* dbg_xq;
  float* dbg_absmax;
  int32_t* dbg_acc;
} ssm_bitlinear_args;

size_t ssm_bitlinear_workspace_bytes(const ssm_bitlinear_args* a);
ssm_status ssm_bitlinear_fwd(const ssm_bitlinear_args* a, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/*
 * ssm_selective_scan_fwd -- the selective recurrence (Mamba; Transformers are SSMs),
 * evaluated as a chunked parallel scan with an fp32 state carried across chunks
 * (TriSSM README: parallel associative scan).  For batch b, head h, channel p of the
 * head, state n and position t:
 *   dt  = softplus(delta[b,t,h] + delta_bias[h]) if delta_softplus, else delta + bias;
 *         softplus(v) = v for v > 20, else log(1 + e^v)
 *   h_t = exp(dt * A) * h_{t-1} + (dt * x[b,t,h,p]) * B[b,t,n],  h_{-1} = h0 (or 0)
 *   y[b,t,h,p] = sum_n C[b,t,n] * h_t[n] + D[h] * x[b,t,h,p]
 * with A = A[h, n] (a_per_state = 1: Mamba-1, headdim 1, one channel per head) or
 * A = A[h] (a_per_state = 0: SSD, a scalar per head).  B and C are shared by all heads.
 * The state stays fp32 whatever act_dtype is.
 *   x     [B, L, nheads * headdim], row stride ld_x;  delta [B, L, nheads], ld_delta;
 *   Bm/Cm [B, L, d_state], ld_B / ld_C;  y [B, L, nheads * headdim], ld_y;
 *   x, delta, Bm, Cm, y have act_dtype (SSM_F32 or SSM_BF16); A, D, delta_bias, h0,
 *   h_last are fp32; h0 / h_last are [B, nheads, headdim, d_state] or NULL.
 * Optional dt projection (Mamba-1 kind; the TriSSM README's ternary Delta projection):
 * when dt_in is not NULL, delta is ignored and the pre-activation dt of channel h at token
 * m is the A8 BitLinear (as ssm_bitlinear_fwd, fp32 out, no bias) of dt_in's first dt_rank
 * columns (row stride ld_dt_in, act_dtype) with packed weights w_dt [nheads, dt_rank],
 * scale s_dt [1], RMSNorm gains g_dt [dt_rank] or NULL and epsilon dt_eps; it is computed
 * inside the scan and never stored.  dt_rank must be in [1, 64].
 * Optional gate (the gated block: Mamba's SiLU gate from a second in_proj branch): when
 * gate is not NULL ([B, L, nheads * headdim] of act_dtype, row stride ld_gate), the stored
 * y is the y above times SiLU(gate) = gate / (1 + exp(-gate)), computed in fp32.
 * Supported: a_per_state = 1 with headdim = 1 and d_state in {4, 8, 16, 32, 64};
 * a_per_state = 0 with headdim <= 256 and d_state in {16, 32, 64, 128}.
 * batch == 0 or seqlen == 0 launches nothing (h_last is then not written).
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_ALIGN, SSM_ERR_WORKSPACE,
 * SSM_ERR_UNSUPPORTED, SSM_ERR_DEVICE.
 */
typedef struct {
  int64_t batch, seqlen, nheads, headdim, d_state;
  int32_t a_per_state;
  int32_t act_dtype; /* ssm_dtype */
  const void* x;      int64_t ld_x;
  const void* delta;  int64_t ld_delta;
  const float* delta_bias;
  int32_t delta_softplus;
  int32_t pad0;
  const float* A;
  const void* Bm;     int64_t ld_B;
  const void* Cm;     int64_t ld_C;
  const float* D;
  const float* h0;
  float* h_last;
  void* y;            int64_t ld_y;
  /* optional dt projection (see above) */
  const void* dt_in;  int64_t ld_dt_in;
  int64_t dt_rank;
  const uint8_t* w_dt;
  const float* s_dt;
  const float* g_dt;
  float dt_eps;
  int32_t pad1;
  /* optional gate (see above) */
  const void* gate;   int64_t ld_gate;
  /* optional precomputed dt input codes (with dt_in): when dt_codes is not NULL, the scan reads
     the int8 codes [B L, 16 ceil(dt_rank / 16)] and fp64 factors dt_deq [B L] that
     ssm_dt_input_quantize wrote for dt_in, instead of computing them itself */
  const int8_t* dt_codes;
  const double* dt_deq;
} ssm_scan_args;

size_t ssm_selective_scan_workspace_bytes(const ssm_scan_args* a);
ssm_status ssm_selective_scan_fwd(const ssm_scan_args* a, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * ssm_selective_scan_fwd_noalloc -- ssm_selective_scan_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation): the same kernels and results, with the scratch memory (the dt input's codes,
 * the carries between time chunks or segments) in an array the library holds on each GPU,
 * SSM_NOALLOC_SCRATCH_BYTES long, instead of a caller workspace.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (concurrent
 * streams, threads) race and must be serialised by the caller.  The array holds the last
 * call's contents; each call writes what it reads.
 * Errors: as ssm_selective_scan_fwd; SSM_ERR_UNSUPPORTED when the shape needs more scratch
 * than SSM_NOALLOC_SCRATCH_BYTES (ssm_selective_scan_workspace_bytes gives the need).
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ssm_status ssm_selective_scan_fwd_noalloc(const ssm_scan_args* a, hipStream_t stream);

/*
 * ssm_dt_input_quantize -- the first step of the scan's dt projection on its own: per token
 * row m of dt_in (dt_rank values, row stride ld, act dtype `dtype`), RMSNorm with gains g_dt
 * (NULL = ones) and epsilon eps, then absmax int8 codes (TriSSM README: BitLinear with int8
 * activations; the same fixed-order arithmetic as ssm_bitlinear_fwd):
 *   codes [m, 16 ceil(dt_rank / 16)] int8 (zero past dt_rank), deq [m] fp64 = max(absmax, 1e-5) / 127.
 * Passing them to ssm_selective_scan_fwd (dt_codes, dt_deq) gives exactly the result of the
 * scan computing them itself.  dt_rank in [1, 64]; m = 0 launches nothing.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_UNSUPPORTED, SSM_ERR_DEVICE.
 */
ssm_status ssm_dt_input_quantize(const void* dt_in, int32_t dtype, int64_t m, int64_t dt_rank, int64_t ld,
                                 const float* g_dt, float eps, int8_t* codes, double* deq,
                                 hipStream_t stream);

/*
 * ssm_mixer_fwd -- one ternary selective-SSM mixer layer (TriSSM README BitSSM mixer;
 * Ternary Mamba abstract for the SSD / W1.58A16 kind), on u [B, L, d_model]:
 *  SSM_MIXER_MAMBA1:  x = BL(u; W_in) [M, d_inner];  p = BL(x; W_x) = [dr | B | C]
 *      [M, dt_rank + 2 d_state];  z = BL(dr; W_dt) [M, d_inner] (internal, fp32);
 *      y = scan(x, z, dt_bias, A [d_inner, d_state], B, C, D);  out = BL(y; W_out).
 *  SSM_MIXER_SSD:     v = BL(u; W_in) = [x (nheads*headdim) | B | C | dt (nheads)];
 *      y = scan(x, dt, dt_bias, A [nheads], B, C, D);  out = BL(y; W_out).
 *  BL is ssm_bitlinear_fwd with the configuration's act_bits, group_size and norm_eps;
 *  x, p, v, y and out are stored in act_dtype; out += u when add_residual != 0.
 *  Gated block (gated = 1; Mamba's block around the selective SSM, the gated diagonal-SSM
 *  block of "Baseline Shape Decides the Verdict ...", abstract (ii)): W_in gains d_inner
 *  rows for a gate branch zg placed last ([x | zg], or [x | B | C | dt | zg] for SSD); the
 *  SSM input channels (x; for SSD x, B and C) first go through ssm_conv1d_silu_fwd of
 *  width d_conv with weights conv_w [channels, d_conv] and bias conv_b (nullable), and
 *  the scan output is multiplied by SiLU(zg) before out_proj (the scan's gate).
 *  Full-precision projections (fp_proj; the TriSSM model keeps in_proj and out_proj in full
 *  precision and makes only Delta, B, C ternary, and compares with an fp_ssm baseline):
 *  fp_proj = 1: in_proj and out_proj are ssm_dense_fwd with fw_in / fw_out; fp_proj = 2:
 *  every projection is (for the Mamba-1 kind the dt projection output is then stored in
 *  act_dtype and read by the scan).  The SSD kind has only in_proj and out_proj, so 1 and 2
 *  mean the same there.
 * u and out have row stride d_model; out may equal u (in place) only when
 * add_residual != 0.  workspace: ssm_mixer_workspace_bytes() bytes of device memory.
 * Requirements: those of the BitLinear and scan calls above; Mamba-1 kind needs
 * act_bits 8 and dt_rank <= 64.
 * Errors: as ssm_bitlinear_fwd and ssm_selective_scan_fwd.
 */
typedef enum { SSM_MIXER_MAMBA1 = 0, SSM_MIXER_SSD = 1 } ssm_mixer_kind;

typedef struct {
  int32_t kind; /* ssm_mixer_kind */
  int32_t act_bits;
  int64_t d_model, d_inner, d_state, dt_rank, nheads, headdim, group_size;
  int32_t act_dtype; /* ssm_dtype */
  float norm_eps;
  int32_t gated;     /* 0: the mixer alone; 1: the gated block (convolution + SiLU gate) */
  int32_t d_conv;    /* width of the block's convolution, 1 .. 8 when gated, else 0 */
  int32_t fp_proj;   /* 0 all projections ternary; 1 in/out full precision; 2 all full precision */
  int32_t pad0;
} ssm_mixer_config;

typedef struct {
  const uint8_t *w_in, *w_x, *w_dt, *w_out; /* packed; w_x, w_dt unused by SSD */
  const float *s_in, *s_x, *s_dt, *s_out;   /* scales as ssm_ternary_quantize_weights writes */
  const float *g_in, *g_x, *g_dt, *g_out;   /* RMSNorm gains or NULL */
  const float *dt_bias, *A, *D;
  const float *conv_w, *conv_b;             /* gated block: [channels, d_conv], [channels] or NULL */
  const void *fw_in, *fw_x, *fw_dt, *fw_out; /* full-precision weights [n_out, k] in act_dtype
                                                (used where fp_proj asks for them) */
} ssm_mixer_weights;

size_t ssm_mixer_workspace_bytes(const ssm_mixer_config* c, int64_t batch, int64_t seqlen);
ssm_status ssm_mixer_fwd(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u,
                         void* out, int64_t batch, int64_t seqlen, int32_t add_residual,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * ssm_mixer_fwd_stages -- ssm_mixer_fwd with its intermediate stages copied out, for stage-wise
 * checks of the integer steps inside fused kernels (TriSSM README: the Delta, B, C projections
 * are BitLinear layers with ternary weights and int8 activations; their int8 codes and int32
 * sums have one correct value each).  Same launches, same results as ssm_mixer_fwd; after the
 * scan, the stages the kernels left in the workspace are copied (device to device, on `stream`)
 * into the caller's buffers, and the in-scan dt projection stores its int32 sums.
 *  stages: not NULL; each pointer NULL (not wanted) or a device buffer, written:
 *   x        [M, d_inner] act_dtype: the SSM input (in_proj output; its convolution when gated)
 *   p        [M, dt_rank + 2 d_state] act_dtype: x_proj output [dr | B | C]
 *            (SSD kind: the in_proj output v [M, d_inner + 2 d_state + nheads (+ d_inner)])
 *   dt_codes [M, dt_rank] int8: the int8 absmax codes of dr's RMSNorm (dt_proj's input)
 *   dt_deq   [M] fp64: max(absmax, 1e-5) / 127 of those rows
 *   dt_acc   [M, d_inner] int32: the dt projection's accumulators (sum of codes x ternary weights)
 *   y        [M, d_inner] act_dtype: the scan output (out_proj's input; times SiLU(zg) when gated)
 *  with M = batch * seqlen.  x and the dt stages exist for the Mamba-1 kind only, the dt stages
 *  with a ternary dt projection only (else SSM_ERR_UNSUPPORTED).
 * Errors: as ssm_mixer_fwd; SSM_ERR_NULL when stages is NULL.
 */
typedef struct {
  void* x;
  void* p;
  int8_t* dt_codes;
  double* dt_deq;
  int32_t* dt_acc;
  void* y;
} ssm_mixer_stages;

ssm_status ssm_mixer_fwd_stages(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u,
                                void* out, int64_t batch, int64_t seqlen, int32_t add_residual,
                                void* workspace, size_t ws_bytes, const ssm_mixer_stages* stages,
                                hipStream_t stream);

/*
 * ssm_mixer_bwd -- the backward pass of one Mamba-1 kind mixer layer (TriSSM README: the mixer
 * is trained end to end, its BitLinear layers with straight-through estimators; Ternary Mamba
 * abstract: quantisation-aware training with learnable scales).  Given dout, the gradient of
 * the loss with respect to out = mixer(u) (+ u with add_residual), it computes du and the
 * gradients of the layer's parameters.  The forward is run again with its intermediates kept
 * in the workspace: x = BL(u; W_in), p = BL(x; W_x) = [dr | B | C], delta = BL(dr; W_dt),
 * y = scan(x, softplus(delta + dt_bias), A, B, C, D) (the values ssm_mixer_fwd computes); then
 *   dy    = BL_bwd(W_out; y, dout)                      (+ dW_out, d s_out)
 *   dx_s, d delta, dA, dB, dC, dD, d dt_bias = ssm_selective_scan_bwd(..., dy)
 *   d dr  = BL_bwd(W_dt; dr, d delta)                   (+ dW_dt, d s_dt)
 *   dx_p  = BL_bwd(W_x; x, [d dr | dB | dC])            (+ dW_x, d s_x)
 *   du    = BL_bwd(W_in; u, dx_s + dx_p) (+ dout)       (+ dW_in, d s_in)
 * where BL_bwd is ssm_bitlinear_bwd's straight-through backward.
 * Supported: Mamba-1 kind, not gated, ternary projections (fp_proj 0), act_bits 8,
 * group_size 0, act_dtype SSM_F32 (else SSM_ERR_UNSUPPORTED).
 *  u [batch, seqlen, d_model] fp32; dout fp32, same shape; du fp32, same shape (written; may
 *  not alias u or dout).  seqlen is limited as in
 *  ssm_selective_scan_bwd.  batch * seqlen = 0 returns SSM_OK and writes nothing.  grads: NULL or a struct whose pointers are each NULL (not wanted) or
 *  device fp32 buffers, written: dw_* [n_out, k] (the latent-weight gradients; n_out, k those
 *  of the projection), ds_* [1] (scale gradients; each needs its dw_* and the latent weights
 *  lat_* [n_out, k]), dA [d_inner, d_state], dD and d_dt_bias [d_inner].
 *  workspace: ssm_mixer_bwd_workspace_bytes(c, batch, seqlen) bytes (0 for a configuration or
 *  size the call rejects), 256-byte aligned; it holds x, p, delta, y and the intermediate
 *  gradients (6 d_inner + 2 dt_rank + 6 d_state floats per token) plus the largest
 *  workspace of the steps.  Sums are taken in a fixed order (results do not depend on timing).
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_UNSUPPORTED, SSM_ERR_ALIGN,
 * SSM_ERR_WORKSPACE, SSM_ERR_DEVICE.
 */
typedef struct {
  const float *lat_in, *lat_x, *lat_dt, *lat_out; /* latent weights (for the scale gradients) */
  float *dw_in, *dw_x, *dw_dt, *dw_out;
  float *ds_in, *ds_x, *ds_dt, *ds_out;
  float *dA, *dD, *d_dt_bias;
} ssm_mixer_grads;

size_t ssm_mixer_bwd_workspace_bytes(const ssm_mixer_config* c, int64_t batch, int64_t seqlen);
ssm_status ssm_mixer_bwd(const ssm_mixer_config* c, const ssm_mixer_weights* w, const ssm_mixer_grads* g,
                         const float* u, const float* dout, float* du, int64_t batch, int64_t seqlen,
                         int32_t add_residual, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * ssm_mixer_step -- one decoding step of the mixer layer: ONE new token per sequence, the
 * recurrence carried between calls (the recurrent, linear-time inference the TernarySSM and
 * TriSSM pages describe for these models).  The result is that of ssm_mixer_fwd with
 * seqlen = 1 whose scan starts from, and ends in, state.
 *  u, out:  [batch, d_model] in act_dtype (out may equal u when add_residual != 0);
 *  state:   device fp32, [batch, d_inner, d_state] (Mamba-1 kind) or
 *           [batch, nheads, headdim, d_state] (SSD kind); read as the state before the token
 *           and overwritten with the state after it (zeros before the first token).
 *  conv_state: gated block with d_conv > 1 only (else ignored, may be NULL): device fp32
 *           [batch, d_conv - 1, channels], the previous d_conv - 1 inputs of the convolution,
 *           oldest first; read and overwritten like state (zeros before the first token).
 *  workspace: ssm_mixer_workspace_bytes(c, batch, 1) bytes of device memory.
 * Decoding a sequence token by token reproduces the outputs of ssm_mixer_fwd over the whole
 * sequence.  Errors: as ssm_mixer_fwd; SSM_ERR_NULL when state (or a needed conv_state) is
 * NULL and batch > 0.
 */
ssm_status ssm_mixer_step(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u, void* out,
                          int64_t batch, float* state, float* conv_state, int32_t add_residual,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * ssm_mixer_stack_step -- one decoding step through a stack of nlayers mixer layers of one
 * configuration c (the output of layer l is the input of layer l + 1): ONE new token per
 * sequence (the TernarySSM and TriSSM pages' recurrent inference, a whole model's layers per
 * token).  The result, and every state afterwards, is bit-identical to calling ssm_mixer_step
 * for layer 0, 1, ..., nlayers - 1 in turn.  Mamba-1 kind layers with ternary projections,
 * per-tensor scales, int8 activations and no gate run in one kernel launch per 24 layers, a
 * block per sequence keeping the activations between layers on chip and fetching each
 * layer's first weights while the previous layer runs; any other layer runs as ssm_mixer_step.
 *  w:           host array of nlayers pointers, layer l's weights (as ssm_mixer_step);
 *  states:      host array of nlayers device pointers, layer l's state (as ssm_mixer_step);
 *  conv_states: host array of nlayers pointers (gated block with d_conv > 1), or NULL;
 *  u, out:      [batch, d_model] in act_dtype (out may equal u when add_residual != 0);
 *  workspace:   ssm_mixer_stack_workspace_bytes(c, batch) bytes of device memory, 256-byte
 *               aligned (the layers' workspace and the activations between layers).
 * All device memory caller-owned; asynchronous on stream; nothing allocated.
 * Errors: SSM_ERR_SHAPE (nlayers < 1, the configuration's), SSM_ERR_NULL, SSM_ERR_WORKSPACE,
 * SSM_ERR_ALIGN, and those of ssm_mixer_step for any layer.
 */
size_t ssm_mixer_stack_workspace_bytes(const ssm_mixer_config* c, int64_t batch);
ssm_status ssm_mixer_stack_step(const ssm_mixer_config* c, const ssm_mixer_weights* const* w, int32_t nlayers,
                                const void* u, void* out, int64_t batch, float* const* states,
                                float* const* conv_states, int32_t add_residual, void* workspace,
                                size_t ws_bytes, hipStream_t stream);

/*
 * ssm_conv1d_silu_fwd -- the gated block's short causal depthwise convolution with SiLU
 * (Mamba, cited under "Builds on" of "Baseline Shape Decides the Verdict ..."):
 *   a[b, t, c] = bias[c] + sum_{j < width} w[c, j] * x[b, t - width + 1 + j, c]
 *   out[b, t, c] = a / (1 + exp(-a))
 * computed in fp64 and rounded once to dtype (the value feeds an int8 quantisation).
 *  x:   [batch, seqlen, ldx] of dtype (SSM_F32 / SSM_BF16), channels 0 .. channels-1 used;
 *  w:   fp32 [channels, width], width in [1, 8];  bias: fp32 [channels] or NULL;
 *  state_in:  fp32 [batch, width - 1, channels] or NULL: the inputs before t = 0 (oldest
 *             first; zeros when NULL);
 *  state_out: fp32 [batch, width - 1, channels] or NULL: receives the last width - 1
 *             inputs (the state after the sequence); may equal state_in;
 *  out: [batch, seqlen, ldo] of dtype; must not alias x.
 * All device pointers; caller-owned; asynchronous on stream.
 * Errors: SSM_ERR_DTYPE, SSM_ERR_SHAPE (sizes, strides, width, out == x), SSM_ERR_NULL,
 * SSM_ERR_DEVICE.
 */
/*
 * ssm_selective_scan_bwd -- the backward of the Mamba-1 kind selective scan (the mixer is
 * trained end to end; TriSSM README): the exact reverse-mode derivative of the recurrence of
 * ssm_selective_scan_fwd (a_per_state = 1, headdim = 1; the dt input given as delta, not as a
 * dt projection).  With dt = softplus(delta + bias), a_t = exp(dt A), h_t = a_t h_{t-1} +
 * dt x B, y = C . h + D x and the state adjoint g_t = C_t dy_t + a_{t+1} g_{t+1}:
 *   dx = D dy + dt sum_n g B;  d delta = sum_n g (h_{t-1} a A + x B) * softplus'(delta + bias);
 *   dA = sum_{b,t} g h_{t-1} a dt;  dB_t = sum_channels g dt x;  dC_t = sum_channels dy h_t;
 *   dD = sum dy x;  d bias = sum d delta;  dh0 = a_0 g_0.
 * Inputs as ssm_selective_scan_fwd (act_dtype x, delta, Bm, Cm; fp32 A [H, N], D, bias, h0)
 * plus dy fp32 [B, L, ld_dy].  Outputs fp32, dense: dx and ddelta [B, L, H], dA [H, N],
 * dB and dC [B, L, N]; dD, dbias [H] and dh0 [B, H, N] nullable.  Time is processed in chunks
 * of 256 / d_state steps; the workspace holds the states and adjoint carries at the chunk
 * boundaries (2 B nchunks H N fp32) and partial sums: ssm_selective_scan_bwd_workspace_bytes().
 * Sums over sequences, chunks and channel tiles are taken in a fixed order (results do not
 * depend on timing).  seqlen is limited to 65535 chunks.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_UNSUPPORTED, SSM_ERR_ALIGN,
 * SSM_ERR_WORKSPACE, SSM_ERR_DEVICE.
 */
typedef struct {
  int64_t batch, seqlen, nheads, d_state;
  int32_t act_dtype; int32_t delta_softplus;
  const void* x;      int64_t ld_x;
  const void* delta;  int64_t ld_delta;
  const float* delta_bias;
  const float* A;
  const void* Bm;     int64_t ld_B;
  const void* Cm;     int64_t ld_C;
  const float* D;
  const float* h0;
  const float* dy;    int64_t ld_dy;
  float *dx, *ddelta, *dA, *dB, *dC, *dD, *dbias, *dh0;
} ssm_scan_bwd_args;

size_t ssm_selective_scan_bwd_workspace_bytes(const ssm_scan_bwd_args* a);
ssm_status ssm_selective_scan_bwd(const ssm_scan_bwd_args* a, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * ssm_bitlinear_bwd -- the backward pass of the A8 BitLinear with straight-through
 * estimators (TriSSM README: BitLinear layers trained with straight-through estimators; the
 * estimator of "Estimating or Propagating Gradients Through Stochastic Neurons ...", cited
 * under "Builds on" of "Baseline Shape Decides the Verdict ...").  With x̂ = RMSNorm(x) g,
 * x̃ = the forward's int8 codes times max(absmax, 1e-5) / 127, W̃ = scale * codes, the forward
 * is y = x̃ W̃^T; the estimator passes gradients through both roundings (absmax and scale held
 * fixed there):
 *   dx̂ = dy W̃;  dx = r g dx̂ - x (r^3 / k) sum_j g_j dx̂_j x_j  (r = 1 / sqrt(mean x^2 + eps));
 *   dW = dy^T x̃ (the gradient of the latent weights);
 *   d_scale = sum over each scale's weights of dW (q - W/s) where |W/s| <= 1, dW q elsewhere
 *   (learnable scales, Ternary Mamba abstract; the learned-step-size rule).
 * All fp32 except x (act dtype).  The forward's codes are rebuilt from x exactly as the
 * forward computes them.  Both contractions run on the library's own matrix-core kernels:
 * with one scale per tensor dx̂ multiplies dy by the bf16 codes (the RMSNorm backward fused
 * into its epilogue) when k <= 1024, otherwise (and with grouped scales) dy W̃ is a dense fp32
 * product; dW multiplies dy by the activation codes over token chunks.
 *  x [m, ldx] (first k columns), norm_weight [k] or NULL, w_packed / w_scale / group_size as
 *  ssm_ternary_quantize_weights wrote them, w_latent [n_out, k] (for d_scale), dy [m, ld_dy],
 *  dx [m, ld_dx] (written), dw [n_out, k] or NULL, d_scale [1] or [n_out, k/group] or NULL.
 *  workspace: ssm_bitlinear_bwd_workspace_bytes(), 256-byte aligned.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_ALIGN, SSM_ERR_WORKSPACE,
 * SSM_ERR_DEVICE.
 */
typedef struct {
  const void* x; int32_t x_dtype; int32_t pad0;
  int64_t m, k, ldx;
  const float* norm_weight; float norm_eps; int32_t pad1;
  const uint8_t* w_packed; const float* w_scale;
  int64_t n_out, group_size;
  const float* w_latent;
  const float* dy; int64_t ld_dy;
  float* dx; int64_t ld_dx;
  float* dw;
  float* d_scale;
} ssm_bitlinear_bwd_args;

size_t ssm_bitlinear_bwd_workspace_bytes(const ssm_bitlinear_bwd_args* a);
ssm_status ssm_bitlinear_bwd(const ssm_bitlinear_bwd_args* a, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/*
 * ssm_qat_sgd_step -- one step of quantisation-aware training (Ternary Mamba abstract:
 * grouped QAT with learnable quantisation scales): w_latent -= lr * dw and, when d_scale is
 * given, w_scale -= lr_scale * d_scale (fp32 fused multiply-adds, in place); then the weights
 * are ternarised under the updated scales (not their absmean) into w_packed, and zero_count
 * (nullable, device int64) receives the number of zero codes -- the zero ratio that collapses
 * when learnable scales grow.  Shapes as ssm_ternary_quantize_weights.  Asynchronous.
 * Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_ALIGN, SSM_ERR_DEVICE.
 */
ssm_status ssm_qat_sgd_step(float* w_latent, float* w_scale, const float* dw, const float* d_scale,
                            int64_t n_out, int64_t k, int64_t group_size, float lr, float lr_scale,
                            uint8_t* w_packed, int64_t* zero_count, void* workspace, size_t ws_bytes,
                            hipStream_t stream);

/*
 * ssm_dense_fwd -- a full-precision linear layer, y = x W^T (+ residual): the in and out
 * projections of the TriSSM model, and every projection of its fp_ssm baseline (TriSSM
 * README).  No RMSNorm, no quantisation, no bias.  A plain dense GEMM on the library's own
 * matrix-core kernel: fp32 operands on fp32 MFMA, or bf16 operands on bf16 MFMA, fp32
 * accumulation, the residual added in fp32, one rounding to dtype.
 *  x: [m, ldx] of dtype (first k columns);  w: [n, k] of dtype, row-major;
 *  residual: [m, ld_res] of dtype or NULL (may equal y);  y: [m, ldy] of dtype, not x.
 * Allocates nothing and keeps no state; asynchronous on stream.
 * Errors: SSM_ERR_DTYPE, SSM_ERR_SHAPE (sizes, strides, sizes of 2^31 or more, y == x),
 * SSM_ERR_NULL, SSM_ERR_DEVICE.
 */
ssm_status ssm_dense_fwd(const void* x, int32_t dtype, int64_t m, int64_t k, int64_t ldx, const void* w, int64_t n,
                         const void* residual, int64_t ld_res, void* y, int64_t ldy, hipStream_t stream);

ssm_status ssm_conv1d_silu_fwd(const void* x, int32_t dtype, int64_t batch, int64_t seqlen, int64_t channels,
                               int64_t ldx, const float* w, int32_t width, const float* bias,
                               const float* state_in, float* state_out, void* out, int64_t ldo,
                               hipStream_t stream);

/*
 * ssm_mixer_fuses_front -- 1 when ssm_mixer_fwd evaluates this configuration's x = BL(u; W_in),
 * p = BL(x; W_x) and the quantisation of dr (the dt projection's input) as one fused kernel
 * (Mamba-1 kind, d_model 64..512, d_inner 128..1024 but not 512 with 1024, dt_rank + 2 d_state
 * <= 64), 0 when it issues them as separate BitLinear calls.  The results are the same either
 * way; this only tells a profiler which kernels to expect.  Host-only, no device access;
 * returns 0 for a NULL or invalid configuration.
 */
int32_t ssm_mixer_fuses_front(const ssm_mixer_config* c);

#ifdef __cplusplus
}
#endif

#endif /* SSM_TERNARY_H */
