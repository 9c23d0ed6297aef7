/* dq.h — C ABI of the DualQuant dual-scale weight-reconstruction library (MI355X, gfx950).
 *
 * DualQuant ("DualQuant: Dual-scale Calibration-free Weight-and-Activation Quantization
 * for LLMs") fits a weight matrix W (rows = output channels, cols = input channels) as
 *
 *     W ~= diag(r) . Qhat . diag(c),   Qhat = FQ_f(W ./ (r c^T)),
 *
 * where FQ_f is the block fake-quantiser of format f used as a black box, r is a row-scale
 * vector and c a column-scale vector.  It minimises the reconstruction MSE by block
 * coordinate descent with closed-form scale updates, projecting each scale onto the
 * format's admissible set after each update (listing page abstract; conference entry's
 * abstract; news summary, mechanism paragraph).  The column scales are the activation
 * rescaling beta: activation channel j is multiplied by c_j before it is quantised
 * (listing page Table 1 caption and Table 6; news summary).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or retains them; scratch memory comes in through `workspace`.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every compute call only
 *     enqueues work on it and returns; its outputs are valid once that work has completed
 *     (an event, a stream synchronisation, or later work on the same stream).
 *   - Matrices are row-major; `ld` is the row pitch in elements (ld >= cols).  Blocks of
 *     `group` consecutive elements run along a row.  Base pointers and the row pitch in
 *     bytes must be multiples of 16.  cols must be a multiple of the group and at most
 *     65536 (the solver's row pass keeps the column scales in LDS while 8 bytes per column
 *     fit a workgroup's LDS, always up to 16384 columns, and reads them from L2 beyond; the
 *     quantisers cover wider rows in several passes of 16384 columns).
 *   - Codes of the 4-bit formats: two per byte, low nibble = even column, [rows][cols/2].
 *     INT4 and MXINT4 codes are two's complement; MXFP4/NVFP4 codes are E2M1
 *     sign-magnitude (the sign of a negative value that rounds to zero is kept: code 0x8).
 *     Codes of the 8-bit formats: one byte per element, [rows][cols]; INT8 and MXINT8
 *     two's complement, MXFP8 the OCP E4M3FN / E5M2 byte.
 *     Codes of the 6-bit formats (MXFP6 E2M3 / E3M2, sign in bit 5): a little-endian bit
 *     stream, element j of a row in bits 6j .. 6j+5 of the row's 3*cols/4 bytes.
 *     The sign of a negative value that rounds to zero is kept in every float format.
 *   - Block scales: [rows][cols/group].  INT4/INT8: bf16 bit patterns (uint16), value
 *     bf16(amax/7) or bf16(amax/127).  MX formats: one E8M0 byte, value 2^(byte-127).
 *     NVFP4: one E4M3FN byte, multiplied by the fp32 tensor scale.
 *   - Dequantised value of an element: INT4/INT8 q*s; MXINT4 q*2^(e-2); MXINT8 q*2^(e-6);
 *     MXFP4 e2m1(q)*2^e; MXFP8/MXFP6 value(q)*2^e; NVFP4 e2m1(q)*(e4m3(sb)*tensor_scale).
 *     The MX shared exponent is e = floor(log2 amax) - emax of the element type (MXFP4 2,
 *     E4M3 8, E5M2 15, E2M3 2, E3M2 4; MXINT4 and MXINT8 0), elements round to nearest
 *     with ties to even and saturate at the type's largest finite value.
 *   - Errors are returned synchronously.  Every argument check happens before any GPU work
 *     is enqueued, so a call that returns an error has enqueued nothing.  Conditions that
 *     depend on the data are reported as flag bits (DQ_FLAG_*) in dq_report.
 *   - The quantisers (dq_quantize_weights, dq_rescale_quantize_acts and its _multi and
 *     _noalloc forms), the layer (dq_quantized_linear, dq_quantized_linear_ws),
 *     dq_recode_mxint4_to_mxfp6 and dq_dequantize enqueue kernel launches only: no
 *     allocation, memset, copy or host wait, and every workspace byte a kernel reads was
 *     written earlier in the same call.  They may be recorded by HIP stream capture and the
 *     graph replayed (on new input values at the same addresses).  dq_solve is not
 *     capture-safe: it clears the histories with memsets and stages its problem
 *     descriptors with a host-to-device copy.
 */
#ifndef DQ_H
#define DQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
enum {
  DQ_OK = 0,
  DQ_ERR_NULL = -1,       /* a required pointer is NULL */
  DQ_ERR_SHAPE = -2,      /* bad rows/cols/ld, cols not a multiple of the group, cols > 65536 */
  DQ_ERR_ALIGN = -3,      /* base pointer or row pitch not 16-byte aligned */
  DQ_ERR_FORMAT = -4,     /* unknown format, group or dtype */
  DQ_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required */
  DQ_ERR_HIP = -6,        /* a HIP runtime call failed */
  DQ_ERR_ARG = -7         /* other invalid argument (iteration count, problem count) */
};

/* ---------------------------------------------------------------- formats and dtypes */
enum {
  DQ_FMT_INT4 = 0,    /* symmetric INT4, per-group bf16 scale, group 64 or 128 */
  DQ_FMT_MXINT4 = 1,  /* 32-element blocks, E8M0 scale, 4-bit integers with implicit 2^-2 */
  DQ_FMT_MXFP4 = 2,   /* 32-element blocks, E8M0 scale, E2M1 elements (OCP MX v1.0) */
  DQ_FMT_NVFP4 = 3,   /* 16-element blocks, E4M3 block scale, fp32 tensor scale, E2M1 */
  DQ_FMT_INT8 = 4,    /* symmetric INT8, per-group bf16 scale, group 64 or 128 */
  DQ_FMT_MXINT8 = 5,  /* 32-element blocks, E8M0 scale, INT8 elements x 2^-6 (OCP MX v1.0) */
  DQ_FMT_MXFP8_E4M3 = 6,  /* 32-element blocks, E8M0 scale, FP8 E4M3 elements (OCP MX v1.0) */
  DQ_FMT_MXFP8_E5M2 = 7,  /* 32-element blocks, E8M0 scale, FP8 E5M2 elements */
  DQ_FMT_MXFP6_E2M3 = 8,  /* 32-element blocks, E8M0 scale, FP6 E2M3 elements */
  DQ_FMT_MXFP6_E3M2 = 9   /* 32-element blocks, E8M0 scale, FP6 E3M2 elements */
};
enum { DQ_F32 = 0, DQ_BF16 = 1 };

/* ---------------------------------------------------------------- report flags */
enum {
  DQ_FLAG_NONFINITE = 1,           /* W contained NaN or Inf (results are not meaningful) */
  DQ_FLAG_ZERO_ROW = 2,            /* a row had D = 0 in an r-step: its scale was kept */
  DQ_FLAG_ZERO_COL = 4,            /* a column had D = 0 in a c-step: its scale was kept */
  DQ_FLAG_NV_BLOCK_UNDERFLOW = 8,  /* an NVFP4 block scale rounded to zero (block zeroed) */
  DQ_FLAG_NV_TENSOR_UNDERFLOW = 16, /* NVFP4 tensor scale s_t = amax/2688 so small (about
                                      2^-119 or less) that 1/(6 s_t) or 1/(2^-9 s_t) is not a
                                      finite fp32 number: the matrix is quantised to 0 */
  DQ_FLAG_UNFINISHED = 32          /* the solve did not finish in the sweeps dq_solve queued
                                      (never expected: T iterations take T + 1 sweeps) */
};

typedef struct {
  int32_t fmt;    /* DQ_FMT_* */
  int32_t group;  /* block size; 0 = the format's default (INT4/INT8 128, MX 32, NVFP4 16) */
} dq_quant_spec;

typedef struct {
  int32_t iters;     /* BCD iterations T, 0 <= T <= 65536 */
  float tol_relchg;  /* > 0: stop after the first iteration whose relative change of Qhat is
                        <= tol_relchg; 0: run all T iterations */
  int32_t scale_steps;  /* which scale steps run: DQ_STEP_ROW | DQ_STEP_COL, 0 = both.  With
                           one bit the other scale vector stays at its initial value and its
                           trace rows stay NaN (the news summary's ablation: row scales only
                           or column scales only) */
} dq_solve_opts;

#define DQ_STEP_ROW 1
#define DQ_STEP_COL 2

typedef struct {           /* written to DEVICE memory by the solve's last kernel */
  int32_t iters_run;       /* iterations completed */
  int32_t rejected_steps;  /* Qhat-steps whose candidate was not kept (it would raise the MSE) */
  uint32_t flags;          /* DQ_FLAG_* */
  int32_t sweeps;          /* passes over W the solve made (diagnostic) */
} dq_report;

/* One matrix of a (possibly batched) solve. */
typedef struct {
  const void* W;        /* [rows][ld] fp32 or bf16 */
  int32_t w_dtype;      /* DQ_F32 or DQ_BF16 */
  int32_t reserved;
  int64_t rows, cols, ld;
  const float* r_init;  /* [rows] initial row scales, or NULL for ones */
  const float* c_init;  /* [cols] initial column scales, or NULL for ones */
  float* r;             /* out [rows]: final row scales (admissible values) */
  float* c;             /* out [cols]: final column scales = beta (admissible values) */
  uint8_t* codes;       /* out [rows*cols/2] (8-bit formats: [rows*cols]): codes of the final Qhat */
  void* block_scales;   /* out [rows*cols/group]: block scales of the final Qhat */
  float* tensor_scale;  /* out [1]: NVFP4 tensor scale of the final Qhat (ignored otherwise) */
  double* nmse_hist;    /* out [iters+1] or NULL: ||W - diag(r)Qhat diag(c)||^2 / ||W||^2 */
  double* relchg_hist;  /* out [iters+1] or NULL: ||Qhat_t - Qhat_{t-1}|| / ||Qhat_{t-1}||, [0] = 0 */
  float* r_trace;       /* out [iters][rows] or NULL: each r-step's closed form N/D before projection (NaN if D = 0) */
  float* c_trace;       /* out [iters][cols] or NULL: each c-step's closed form N/D before projection (NaN if D = 0) */
  dq_report* report;    /* DEVICE pointer (4-byte aligned) or NULL: written by the solve's
                           last kernel, valid when the solve's work on `stream` has completed */
} dq_problem;

/* Bytes of workspace dq_solve needs for this batch (0 on invalid arguments). */
size_t dq_workspace_bytes(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                          const dq_solve_opts* opts);

/* The DualQuant solve (listing page abstract: variable splitting + block coordinate
 * descent with closed-form subproblems; conference entry: quantiser as a black box,
 * scales projected onto the format's admissible set after each update; listing page
 * Fig. 2 / Fig. 3 for the statistics).  For each problem, starting from r = r_init and
 * c = c_init (ones when NULL) and Qhat_0 = FQ_f(W ./ r c^T), each iteration runs
 *   r-step  r_i <- Proj(N_i / D_i), N_i = sum_j W_ij Qhat_ij c_j, D_i = sum_j (Qhat_ij c_j)^2;
 *   c-step  c_j <- Proj(N_j / D_j), N_j = sum_i r_i W_ij Qhat_ij, D_j = sum_i (r_i Qhat_ij)^2,
 *           with the new r;  a scale whose D is 0 is kept;
 *   Qhat-step  candidate FQ_f(W ./ r c^T), kept unless it raises the MSE at the current
 *           scales (so the MSE never increases);
 * where Proj is the nearest admissible value: E4M3 values in [2^-9, 448] (NVFP4), bf16
 * values in [2^-126, max bf16] with ties to even (INT4, INT8 and the MX formats, whose
 * block scales stay E8M0 powers of two inside the quantiser: a power-of-two dual scale
 * would be absorbed by them exactly).
 * Problems are independent; count (1..65535) > 1 runs them together on one GPU.
 * Stream-ordered: the call uploads the problem descriptors (staged before it returns),
 * enqueues its T + 1 sweeps -- the INIT sweep and one per iteration; each sweep computes the
 * next r- and c-steps for both outcomes of its Qhat-step's safeguard, so a rejected
 * candidate costs no extra sweep -- and the output kernel, and returns without waiting.
 * With tol_relchg > 0 a solve can finish early; the queued sweeps that find every problem
 * finished exit at once.  `workspace` must hold
 * dq_workspace_bytes(...) bytes of device memory; its contents on entry do not matter, and
 * it must stay untouched until the solve's work has completed. */
int dq_solve(const dq_problem* problems, int32_t count, dq_quant_spec spec,
             const dq_solve_opts* opts, void* workspace, size_t workspace_bytes, void* stream);

/* Diagnostic: dq_solve with a begin/end HIP event pair attached to each pass's kernel
 * launches -- the row pass, the column pass, and the column finalize plus the safeguard
 * decision (all problems of the call) -- of each queued sweep.  Synchronises `stream` before
 * returning and writes three durations in ms per sweep to the HOST array pass_ms
 * (pass_ms_capacity sweeps at most; *pass_ms_count = sweeps written).  Sweeps beyond the
 * report's `sweeps` ran no work.  Same outputs as dq_solve. */
int dq_solve_timed(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                   const dq_solve_opts* opts, void* workspace, size_t workspace_bytes,
                   void* stream, float* pass_ms, int32_t pass_ms_capacity,
                   int32_t* pass_ms_count);

/* The same diagnostic split in two so that timing adds no wait to the stream.
 * dq_solve_timed_enqueue is dq_solve (same arguments, same outputs, asynchronous) with the
 * event pairs attached to the first `timed_sweeps` (>= 1, else DQ_ERR_ARG) queued sweeps.
 * dq_solve_timed_read, called on the same current device after the caller has waited for
 * that stream, writes the three durations per sweep of the last timed solve enqueued on the
 * device to the HOST array pass_ms (pass_ms_capacity sweeps at most; *pass_ms_count =
 * sweeps written); DQ_ERR_HIP if the stream has not run them yet.  The events belong to the
 * library, one set per device: timed solves on one device must not overlap between their
 * enqueue and their read. */
int dq_solve_timed_enqueue(const dq_problem* problems, int32_t count, dq_quant_spec spec,
                           const dq_solve_opts* opts, void* workspace, size_t workspace_bytes,
                           void* stream, int32_t timed_sweeps);
int dq_solve_timed_read(float* pass_ms, int32_t pass_ms_capacity, int32_t* pass_ms_count);

/* Bytes of workspace dq_quantize_weights / dq_rescale_quantize_acts need. */
size_t dq_quantize_workspace_bytes(int64_t rows, int64_t cols, dq_quant_spec spec);

/* The Qhat-step on its own: codes, block scales and (NVFP4) tensor scale of
 * FQ_f(W ./ (r c^T)) (conference entry: the quantiser used as a black box).  r and/or c
 * may be NULL (ones).  The NVFP4 tensor scale is max|W ./ r c^T| / 2688.  Asynchronous. */
int dq_quantize_weights(const void* W, int32_t w_dtype, int64_t rows, int64_t cols, int64_t ld,
                        const float* r, const float* c, dq_quant_spec spec, uint8_t* codes,
                        void* block_scales, float* tensor_scale, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Activation rescale + quantise (listing page abstract and Table 11, "activation
 * quantization (incl. beta)"; Table 6; news summary): x'_tj = x_tj * c_j (exact in fp32
 * for admissible c), then FQ_f along each token row.  c may be NULL (beta not applied).
 * X is [tokens][ld], fp32 or bf16.  Asynchronous. */
int dq_rescale_quantize_acts(const void* X, int32_t x_dtype, int64_t tokens, int64_t cols,
                             int64_t ld, const float* c, dq_quant_spec spec, uint8_t* codes,
                             void* block_scales, float* tensor_scale, void* workspace,
                             size_t workspace_bytes, void* stream);

/* dq_rescale_quantize_acts for callers that cannot allocate memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments without the workspace; same outputs, bit for bit.  The call allocates nothing.
 * The scratch it needs (NVFP4: the amax pre-pass partials; the other formats need none) is a
 * fixed array of DQ_NOALLOC_SCRATCH_BYTES bytes that the library keeps on every GPU it runs
 * on until the process ends; its address is looked up on the first call on each device.
 * Every call on one GPU shares that array and leaves its contents behind: calls that may
 * overlap on one GPU (issued to different streams without ordering between them) race and
 * give wrong results.  The stream must belong to the current device (DQ_ERR_ARG otherwise).
 * Returns DQ_ERR_WORKSPACE if a call would need more scratch than the array holds (no input
 * size does: the partials never exceed 1024 floats), DQ_ERR_HIP if the array's device
 * address cannot be obtained, and otherwise what dq_rescale_quantize_acts returns.
 * Asynchronous. */
#define DQ_NOALLOC_SCRATCH_BYTES 4096
int dq_rescale_quantize_acts_noalloc(const void* X, int32_t x_dtype, int64_t tokens,
                                     int64_t cols, int64_t ld, const float* c,
                                     dq_quant_spec spec, uint8_t* codes, void* block_scales,
                                     float* tensor_scale, void* stream);

/* Activation rescale + quantise for several projections that read the same activations
 * (q/k/v of an attention block, gate/up of an MLP block), each with its own solved column
 * scales c_k (same passages as dq_rescale_quantize_acts: beta is applied per consuming
 * weight, so each projection needs its own copy of the quantised activations).  Output k is
 * exactly what dq_rescale_quantize_acts(X, ..., c[k], spec, codes[k], block_scales[k],
 * tensor_scales[k], ...) writes; X is read once per pass instead of once per output.
 *   count          1..DQ_MAX_MULTI outputs.
 *   c              HOST array of `count` device pointers (an entry may be NULL: no beta);
 *                  c itself may be NULL (no beta for any output).
 *   codes, block_scales, tensor_scales
 *                  HOST arrays of `count` device pointers, each laid out as for the
 *                  single-output call (tensor_scales only read for NVFP4; may be NULL
 *                  otherwise).
 *   workspace      dq_quantize_multi_workspace_bytes(...) bytes of device memory.
 * Returns DQ_ERR_ARG for count outside 1..DQ_MAX_MULTI, otherwise the single-output call's
 * statuses.  Asynchronous. */
#define DQ_MAX_MULTI 8
size_t dq_quantize_multi_workspace_bytes(int64_t tokens, int64_t cols, int32_t count,
                                         dq_quant_spec spec);
int dq_rescale_quantize_acts_multi(const void* X, int32_t x_dtype, int64_t tokens,
                                   int64_t cols, int64_t ld, int32_t count,
                                   const float* const* c, dq_quant_spec spec,
                                   uint8_t* const* codes, void* const* block_scales,
                                   float* const* tensor_scales, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Quantised linear layer on the matrix cores (listing page Table 11, "quantized linears",
 * and Table 12's packed 4-bit weights; news summary: beta folds into the activation
 * quantiser, the row scales into the layer output):
 *     Y[m][n] = r[n] * sum_k Aq[m][k] * Q[n][k],
 * the product of the activation codes (dq_rescale_quantize_acts with the solved c, so
 * Aq = FQ(X diag(c))) and the weight codes (dq_solve or dq_quantize_weights), each element
 * dequantised with its block scale (and, for NVFP4, its tensor scale).  With
 * W ~ diag(r) Q diag(c) this is Y ~ X W^T.
 *   spec       DQ_FMT_MXFP4, DQ_FMT_MXFP6_E2M3/E3M2, DQ_FMT_MXFP8_E4M3/E5M2 (group 32) on
 *              the block-scaled cores, DQ_FMT_NVFP4 (group 16) on the f16 cores: its
 *              elements e2m1 * e4m3 are exact in fp16 and the tensor scales multiply the
 *              fp32 result; or DQ_FMT_INT4 (group 64 or 128, bf16 scales) on the int8 cores:
 *              each group's integer dot product is exact in int32, then multiplied by the
 *              two bf16 scales' product (exact in fp32) and added in fp32.  The same format
 *              for both operands (MXINT4: see dq_recode_mxint4_to_mxfp6).
 *   a_codes    [M][K] activation codes in the format's layout (row pitch K*bits/8 bytes),
 *              16-byte aligned; a_scales [M][K/group] scale bytes (INT4: bf16 values, 2-byte
 *              aligned); a_tensor_scale [1] fp32 (NVFP4 only, else ignored and may be NULL).
 *   b_codes    [N][K] weight codes, 16-byte aligned; b_scales [N][K/group]; b_tensor_scale.
 *   K          a multiple of 32 (INT4: of the group; 0 gives Y = 0).
 *   r          [N] fp32 row scales of the weights, or NULL (ones).
 *   y          [M][ldy] output, fp32 (y_dtype DQ_F32) or bf16 (DQ_BF16, round to nearest
 *              even); ldy >= N.
 * Accumulation is fp32 in the matrix cores.  For E2M1 and E2M3 elements every product and
 * partial sum of one instruction is exact, so only the fp32 accumulation rounds; the f16
 * products of NVFP4 are exact too, but its tensor scales are applied once to the sum (the
 * per-element dequantisation rounds e4m3 * s_t instead).  For E4M3, E5M2 and E3M2 the cores'
 * internal sum keeps fewer bits than fp32 (measured: about 2^-12 of sum |a b| over
 * 128-element random-code dot products).  Fastest with 4-byte-aligned scale arrays and K
 * a multiple of 256 (FP4), 128 (FP8, NVFP4); other inputs take a register-staged kernel.
 * Returns DQ_ERR_FORMAT for other formats, DQ_ERR_SHAPE for bad sizes, DQ_ERR_ALIGN for
 * misaligned codes or output.  Asynchronous. */
int dq_quantized_linear(dq_quant_spec spec, const uint8_t* a_codes, const uint8_t* a_scales,
                        const float* a_tensor_scale, int64_t M, const uint8_t* b_codes,
                        const uint8_t* b_scales, const float* b_tensor_scale, int64_t N,
                        int64_t K, const float* r, void* y, int32_t y_dtype, int64_t ldy,
                        void* stream);

/* The same layer with a caller workspace, which lets an INT4 layer with few output tiles
 * (few tokens: the listing page's Table 11 forwards of 82 tokens, and decoding) split K
 * over several workgroups per tile: each writes unscaled fp32 partial sums to the
 * workspace and a second kernel adds them in split order and applies 2^-8 and r.  The sum
 * order differs from the unsplit kernel's (one more fp32 rounding per split: the bound is
 * (K/group + splits + 3) 2^-24 sum |a b| |r|); a given shape always splits the same way, so
 * results are reproducible.  Other formats, and INT4 shapes that fill the GPU without it,
 * ignore the workspace.
 *   workspace         16-byte-aligned device memory of at least
 *                     dq_quantized_linear_workspace_bytes(spec, M, N, K) bytes, or NULL (no
 *                     split: the same as dq_quantized_linear).
 * Returns DQ_ERR_WORKSPACE when a non-NULL workspace is smaller than required, DQ_ERR_ALIGN
 * when it is misaligned; otherwise as dq_quantized_linear.  Asynchronous. */
int dq_quantized_linear_ws(dq_quant_spec spec, const uint8_t* a_codes, const uint8_t* a_scales,
                           const float* a_tensor_scale, int64_t M, const uint8_t* b_codes,
                           const uint8_t* b_scales, const float* b_tensor_scale, int64_t N,
                           int64_t K, const float* r, void* y, int32_t y_dtype, int64_t ldy,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dq_quantized_linear_ws uses for this shape (0: it does not split); at most
 * K (N + 3), twice the weight codes' bytes: the splits are capped so. */
size_t dq_quantized_linear_workspace_bytes(dq_quant_spec spec, int64_t M, int64_t N, int64_t K);

/* Exact re-encoding of MXINT4 codes as MXFP6 E2M3 codes, so that MXINT4 activations and
 * weights can run through dq_quantized_linear (whose matrix cores take FP4/FP6/FP8 elements
 * under E8M0 scales, not integers).  Each MXINT4 element q * 2^(e-2), q in [-7, 7], is the
 * E2M3 value q under the scale 2^(e-2); when e - 2 is below the smallest E8M0 scale 2^-127
 * it becomes q/2 or q/4 under 2^-127, still exact.  The dequantised values of the output
 * equal those of the input bit for bit.
 *   codes        [rows][cols/2] MXINT4 nibbles, 16-byte aligned;  block_scales [rows][cols/32].
 *   out_codes    [rows][3*cols/4] MXFP6 E2M3 codes (the 6-bit stream layout), 8-byte aligned;
 *   out_scales   [rows][cols/32] E8M0 bytes.
 * cols must be a multiple of 32.  Asynchronous. */
int dq_recode_mxint4_to_mxfp6(const uint8_t* codes, const uint8_t* block_scales, int64_t rows,
                              int64_t cols, uint8_t* out_codes, uint8_t* out_scales,
                              void* stream);

/* Decode codes + block scales (+ tensor scale) into fp32 values [rows][cols].  When r and/or
 * c are given the output is diag(r) Qhat diag(c) (the reconstruction), else Qhat.
 * Asynchronous. */
int dq_dequantize(dq_quant_spec spec, const uint8_t* codes, const void* block_scales,
                  const float* tensor_scale, int64_t rows, int64_t cols, const float* r,
                  const float* c, float* out, void* stream);

/* Human-readable text of a status code. */
const char* dq_status_string(int status);

/* ---------------------------------------------------------------- diagnostics
 * Apply one of the library's scalar device rounding routines elementwise (n values):
 *   DQ_ROUND_E2M1      x -> E2M1 code byte (ties to even, saturating, sign kept)
 *   DQ_ROUND_E4M3      x >= 0 -> E4M3FN code byte (ties to even, saturating at 448)
 *   DQ_ROUND_BF16      x -> nearest bf16 value (fp32 out)
 *   DQ_ROUND_INT4      x -> nearest integer in [-7, 7], ties to even (int8 out)
 *   DQ_PROJ_MX / DQ_PROJ_E4M3 / DQ_PROJ_BF16     x > 0 -> projected dual scale of the MX
 *                      formats (bf16 values), NVFP4 (E4M3 values), INT4/INT8 (bf16 values)
 * Used to check the device routines against an independent implementation. */
enum { DQ_ROUND_E2M1 = 0, DQ_ROUND_E4M3 = 1, DQ_ROUND_BF16 = 2, DQ_ROUND_INT4 = 3,
       DQ_PROJ_MX = 4, DQ_PROJ_E4M3 = 5, DQ_PROJ_BF16 = 6 };
int dq_debug_round(int32_t fn, const float* x, void* out, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DQ_H */
