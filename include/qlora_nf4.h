/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) NF4 / double-quant / QLoRA-linear library.
 *
 * Sources (web pages on QLoRA/NF4):
 *   [QE] "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs"
 *   [LQ] "LoRA vs QLoRA: Efficient Fine-Tuning Explained"
 *   [WQ] "What is QLoRA, and how does it enable fine-tuning on consumer hardware?"
 *
 * General conventions (every entry point):
 *   - Every device buffer is allocated and owned by the caller.  The library
 *     allocates no device memory and keeps no device state between calls.
 *   - All arrays are dense and row-major.  bf16 is the IEEE-754 binary32 top half
 *     (1-8-7); f32 is IEEE binary32.  Element counts are int64_t.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work
 *     is enqueued asynchronously on it; the call returns once it is enqueued.
 *     Results are deterministic: no floating-point atomics, fixed reduction order.
 *   - Calls on different streams may run concurrently if their outputs do not
 *     overlap.  The library is thread-safe.
 *   - Return value is a qn_status.  Argument validation happens on the host
 *     before anything is enqueued; a non-QN_OK return from validation means
 *     nothing was launched and no output was touched.  QN_ERR_HIP reports a
 *     failed launch (hipGetLastError).  No C++ exception crosses the ABI.
 *   - Device pointers must be 16-byte aligned unless stated otherwise
 *     (QN_ERR_ALIGN).  Weight matrices are 2-D only ([QE] "Turn a LoRA script
 *     into a QLoRA script ...": the 4-bit kernels take two-dimensional weights).
 *
 * Format constants, fixed by [QE]: block of 64 weights per absmax ("Why the
 * groups are small"); group of 256 absmaxes per fp32 constant ("Shrink the
 * scale factors too, and total up the real bill").
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QN_BLOCK 64
#define QN_GROUP 256
#define QN_MAX_RANK 64   /* [LQ] "How LoRA Works": r is commonly 8 to 64 */
#define QN_MAX_GROUP 8   /* linears per grouped launch (a layer has 7)   */

typedef enum {
  QN_OK = 0,
  QN_ERR_NULL = 1,       /* a required pointer is NULL                           */
  QN_ERR_SHAPE = 2,      /* a size is <= 0, too large, or inconsistent            */
  QN_ERR_DTYPE = 3,      /* unknown qn_dtype                                      */
  QN_ERR_ALIGN = 4,      /* a device pointer is not 16-byte aligned               */
  QN_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than qlora_workspace_size() */
  QN_ERR_HIP = 6,        /* the HIP runtime reported an error on launch           */
  QN_ERR_VALUE = 7,      /* a scalar argument is not finite                       */
  QN_ERR_SCRATCH = 8,    /* the no-allocation entry point's static scratch is too */
                         /* small for this problem                                */
  QN_ERR_MEMORY = 9      /* a buffer is neither device memory nor pinned host     */
                         /* memory mapped for the device                          */
} qn_status;

typedef enum { QN_F32 = 0, QN_BF16 = 1 } qn_dtype;

/* 4-bit types: the table a weight's codes index.  [QE] "Turn a LoRA script
 * into a QLoRA script with one config object": bnb_4bit_quant_type picks NF4,
 * the quantile table; the library's other option is a small floating-point
 * layout at the same memory.  QN_FP4 reads that as the E2M1 float (sign, two
 * exponent bits, one mantissa bit; 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 * negatives) divided by 6 so the table spans [-1, 1] like NF4; code c has
 * sign bit 3, exponent bits 2..1, mantissa bit 0; +0 (code 0) is the code
 * written for zero. */
#define QN_NF4 0
#define QN_FP4 1

/* One frozen weight W[N, K] in quantised form.  Caller-owned device buffers.
 *   codes    uint8[ceil(N*K/2)]: element e of the row-major flattening has its
 *            4-bit row index in byte e/2, low nibble for even e, high nibble for
 *            odd e ([QE] "Store a weight in 4 bits ...": the pattern is a row
 *            index; [WQ] "How it actually works": N*b/8 bytes).
 *   absmax   fp32[ceil(N*K/64)]: largest |w| of each block of 64 consecutive
 *            elements.  Used when absmax_q is NULL.
 *   absmax_q uint8[ceil(N*K/64)]: double-quantised block scales, or NULL.
 *   scale2   fp32[ceil(nb/256)]: grid step of each group of 256 blocks; required
 *            when absmax_q is non-NULL.  The scale of block b is then
 *            fl32(absmax_q[b] * scale2[b/256]).
 *   quant_type QN_NF4 (0, the default of a zero-initialised struct) or QN_FP4:
 *            the table the codes index.
 * codes 16-byte aligned; absmax, absmax_q and scale2 4-byte aligned.
 */
typedef struct {
  const uint8_t *codes;
  const float *absmax;
  const uint8_t *absmax_q;
  const float *scale2;
  int64_t N;
  int64_t K;
  int32_t quant_type;
} qn_nf4_weight;

/* The NF4 table, written to host memory out[16] (index 0 = -1, 7 = 0, 15 = +1).
 * [QE] "Put the rows where the weights are", "That is NF4": sixteen values at
 * quantiles of a standard normal, one of them exactly zero, fixed once (not
 * calibrated on a model).  Derived on the host in fp64 (evenly spaced
 * probabilities per half, 7 rows below zero and 8 above, outermost rows at tail
 * probability 31/960, scaled to end at exactly -1 and +1) and rounded to fp32.
 * No device work.  Returns QN_ERR_NULL if out is NULL. */
int qn_codebook(float out[16]);

/* The table of a 4-bit type (QN_NF4 or QN_FP4) in host memory out[16], by
 * code.  QN_ERR_NULL if out is NULL, QN_ERR_DTYPE for an unknown type. */
int qn_table(int quant_type, float out[16]);

/* Blockwise NF4 quantisation of W[N, K] ([QE] "The table, and the number that
 * stretches it", "Why the groups are small", "That is NF4").
 *   W       device, N*K elements of w_dtype (QN_F32 or QN_BF16), row-major.
 *   codes   device out, uint8[ceil(N*K/2)] (layout as in qn_nf4_weight; an odd
 *           element count leaves the last high nibble 0).
 *   absmax  device out, fp32[ceil(N*K/64)]; the last block may be partial.
 * Per block: a = max|w|; rho = fl32(1/a) (correctly rounded; 0 when a = 0);
 * n = fl32(w*rho), or n = fl32(w/a) when 1/a overflows fp32 (a < 2^-128);
 * code = index of the closest table row to n, an exact tie
 * going to the lower index.  Inputs must be finite (non-finite inputs give
 * unspecified codes).  Any N, K >= 1.  W 16-byte aligned; codes 8-byte aligned;
 * absmax 4-byte aligned. */
int nf4_quantize(const void *W, int w_dtype, int64_t N, int64_t K,
                 uint8_t *codes, float *absmax, void *stream);

/* Blockwise quantisation to either 4-bit type, with the block scales'
 * double quantisation optionally in the same launch ([QE] "Shrink the scale
 * factors too, and total up the real bill").
 *   quant_type  QN_NF4 or QN_FP4 (QN_ERR_DTYPE otherwise).
 *   codes, absmax  as nf4_quantize (same values for QN_NF4).
 *   absmax_q, scale2  both NULL (no double quantisation), or both device
 *       outputs as nf4_double_quant writes them from absmax (same values):
 *       uint8[ceil(N*K/64)] and fp32[ceil(N*K/64/256)].
 * For FP4 the closest of the fifteen distinct values is found as for NF4 (an
 * exact tie goes to the lower value) and written as its code; zero is code 0.
 * Alignment as nf4_quantize; absmax_q 4-byte aligned. */
int qn_quantize_4bit(const void *W, int w_dtype, int64_t N, int64_t K, int quant_type,
                     uint8_t *codes, float *absmax, uint8_t *absmax_q, float *scale2,
                     void *stream);

/* Double quantisation of nb block scales ([QE] "Shrink the scale factors too,
 * and total up the real bill": 8 bits per scale, one 32-bit constant per 256).
 *   absmax    device, fp32[nb], values >= 0 (as written by nf4_quantize).
 *   absmax_q  device out, uint8[nb].
 *   scale2    device out, fp32[ceil(nb/256)].
 * Per group g of 256 consecutive blocks (the last may be partial):
 * c = max absmax; step = fl32(c/255); k_b = clamp(ceil(fl32(a_b/step) - 1/2), 0, 255)
 * (nearest grid point of the quotient, ties down); step = 0 gives all k = 0.
 * 4-byte alignment suffices. */
int nf4_double_quant(const float *absmax, int64_t nb, uint8_t *absmax_q,
                     float *scale2, void *stream);

/* Dequantisation of a whole weight ([QE] "The table, and the number ..." step 4,
 * "Predict the throughput tax before you pay it": look up the row, multiply by
 * the block scale).
 *   out  device, N*K elements of out_dtype: fp32 w = fl32(table[q] * A_b), or
 *        bf16 = round-to-nearest-even of that fp32.
 * Bit-exact with that definition.  out 16-byte aligned. */
int nf4_dequant(const qn_nf4_weight *W, void *out, int out_dtype, void *stream);

/* Merge a trained adapter into the frozen weight, for export ([LQ] "How LoRA
 * Works": W + (alpha/r) B A, folded in once; its FAQ: a QLoRA adapter is merged
 * into a dequantised full-precision copy of the base; [QE] "Ship the result,
 * and plan for the merge before you need it": save a 16-bit checkpoint; merged
 * into the 4-bit codes, an update smaller than the gap between rows would be
 * lost).  With w = fl32(table[q] * A_b) (as nf4_dequant, fp32) and s = fl32(alpha/r):
 *     acc = sum_j B[n][j] * A[j][k]   in fp32, j increasing, rounded each step
 *     out[n][k] = fl32(w + fl32(s * acc))       (QN_F32), or its bf16 RNE (QN_BF16)
 *   W    the weight [N, K]; K % 64 == 0, K <= 2^25, N <= 2097120.
 *   A    device bf16 [r, K];  B device bf16 [N, r];  1 <= r <= QN_MAX_RANK.
 *   out  device [N, K] of out_dtype, 16-byte aligned; A, B 16-byte aligned.
 * Bit-exact with that definition whenever no product B[n][j] * A[j][k] falls
 * into fp32's subnormal range (a product of two bf16 values is otherwise exact
 * in fp32, and the kernel adds it with one fused multiply-add).  Asynchronous
 * on `stream`; QN_ERR_* as elsewhere. */
int qlora_merge(const qn_nf4_weight *W, const void *A, const void *B, int64_t r,
                float alpha, void *out, int out_dtype, void *stream);

/* One AdamW step on a bf16 adapter tensor (A or B of a linear) with 8-bit
 * block-wise optimizer state.  [QE] "Why the groups are small": block-wise
 * quantisation (blocks of 64, a scale each) is what makes 8-bit optimizer
 * state work; "Turn a LoRA script into a QLoRA script with one config object":
 * the optimizer is an 8-bit AdamW, its state belongs to the adapter only.
 * The AdamW rule is the published one (decoupled weight decay, bias-corrected
 * moments, step t >= 1); in fp32, each operation rounded once in this order:
 *   m = k_m step_m,  u = k_u step_u,  v = u u            (state read back)
 *   m' = b1 m + (1-b1) g,   v' = b2 v + (1-b2) (g g)
 *   p' = bf16(p - lr ((m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps) + wd p))
 * with 1-b1, 1-b2, 1-b1^t, 1-b2^t formed in double from the fp32 betas and
 * rounded once.  The new state, per block of 64 consecutive parameters: the
 * first moment signed, step_m = max|m'|/127, k_m = clamp(ceil(m'/step_m - 1/2),
 * -127, 127); the second through its square root u' = sqrt(v'), step_u =
 * max u'/255, k_u = clamp(ceil(u'/step_u - 1/2), 0, 255); a zero block has step
 * 0 and codes 0.  2.125 bytes of state per parameter.
 *   param  bf16 [n], updated in place;  grad bf16 [n].
 *   m_q    int8 [n];  m_step fp32 [ceil(n/64)];
 *   u_q    uint8 [n]; u_step fp32 [ceil(n/64)]: read and rewritten;
 *          all zero before the first step.
 * param, grad 16-byte aligned; m_q, u_q, m_step, u_step 4-byte aligned.
 * Placement ([QE] "Turn a memory spike into a slowdown with a paged
 * optimizer": optimizer state that does not fit next to the model can live
 * in host memory, at the price of a slower step).  Each of the six buffers
 * may be device memory (or managed memory), or pinned host memory mapped for
 * the device (hipHostMalloc; torch's pin_memory=True): the kernel then reads
 * and writes it across the host link, the state's bytes never occupying
 * device memory.  Host memory that is not pinned and mapped (pageable
 * memory, an unknown pointer) returns QN_ERR_MEMORY, checked with
 * hipPointerGetAttributes and hipHostGetDevicePointer before any launch.  The
 * library allocates none of it.
 * QN_ERR_VALUE for step < 1, lr, eps or weight_decay not finite, a beta
 * outside [0, 1) or eps <= 0. */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} qn_adamw_config;
int qn_adamw8_step(void *param, const void *grad, int64_t n, int8_t *m_q, float *m_step,
                   uint8_t *u_q, float *u_step, const qn_adamw_config *cfg, void *stream);

/* The same step over several tensors (the A and B of every adapted linear of
 * a layer or a model: [QE] "Turn a LoRA script into a QLoRA script with one
 * config object", the adapter on every linear) in as few launches as possible:
 * one per QN_ADAMW_MULTI tensors.  Each tensor's arguments, layout and
 * alignment as in qn_adamw8_step; all share cfg.  Results are bit-identical to
 * qn_adamw8_step on each tensor in turn.  QN_ERR_SHAPE for n_tensors < 1 or a
 * tensor with n <= 0; QN_ERR_NULL, QN_ERR_ALIGN, QN_ERR_MEMORY and
 * QN_ERR_VALUE as there; nothing is launched unless every tensor passes. */
typedef struct {
  void *param;
  const void *grad;
  int64_t n;
  int8_t *m_q;
  float *m_step;
  uint8_t *u_q;
  float *u_step;
} qn_adamw_tensor;
#define QN_ADAMW_MULTI 32
int qn_adamw8_step_multi(int n_tensors, const qn_adamw_tensor *tensors, const qn_adamw_config *cfg,
                         void *stream);

/* Workspace size in bytes for op = QN_OP_FWD or QN_OP_BWD at the given shape.
 * Returns 0 for an invalid op or shape. */
#define QN_OP_FWD 0
#define QN_OP_BWD 1
size_t qlora_workspace_size(int op, int64_t M, int64_t N, int64_t K, int64_t r);

/* QLoRA linear forward ([LQ] "How LoRA Works": W' = W + (alpha/r) B A; [QE] "That
 * is NF4": the 4-bit base is expanded to bf16 before the multiply, the adapter is
 * bf16; "Turn a LoRA script ...": no bias):
 *     Y = X * bf16(dequant(W))^T + (alpha/r) * (X * A^T) * B^T
 *   X   device bf16 [M, K]      A  device bf16 [r, K]      B  device bf16 [N, r]
 *   Y   device bf16 [M, N] out (fp32 accumulation, rounded to nearest even once)
 *   H_out  device fp32 [M, r] out, X*A^T (unscaled), or NULL.  Keeping it for
 *       the backward saves that call a second pass over X.
 *   workspace  device, >= qlora_workspace_size(QN_OP_FWD, M, N, K, r) bytes.
 * Requires M >= 1, N % 64 == 0, K % 64 == 0 (whole blocks per row; whole
 * contraction steps of 64 over K in the forward and over N in dX),
 * N*K/2 <= INT32_MAX (the kernels address the codes with 32-bit byte offsets),
 * K <= 2^23 and N <= 2^23 (a 128-row slab of X or dY is addressed with 32-bit
 * byte offsets), 1 <= r <= QN_MAX_RANK, finite alpha; workspace 256-byte aligned, H_out 4-byte
 * aligned.  Any other shape returns QN_ERR_SHAPE before anything is launched.
 * M <= 8 runs the streaming decode path (weights read once at HBM rate); larger
 * M runs the MFMA path (tiles dequantised into LDS, bf16 MFMA). */
int qlora_linear_fwd(const void *X, int64_t M, const qn_nf4_weight *W,
                     const void *A, const void *B, int64_t r, float alpha,
                     void *Y, float *H_out, void *workspace, size_t ws_bytes,
                     void *stream);

/* Grouped forward: several independent QLoRA linear forwards in one call
 * ([QE] "Turn a LoRA script into a QLoRA script with one config object":
 * target_modules="all-linear" puts an adapter on every linear of a layer).
 * Problem g computes exactly what qlora_linear_fwd computes with its fields
 * (bit-identical results).  The problems with M > 8 share one low-rank launch
 * and one dequant-GEMM launch per scale source (double-quantised or fp32
 * scales) whose tiles cover all of them, the longest contractions first, so
 * that linears too small to fill the GPU on their own (a layer's k and v
 * projections) run beside the others; problems with M <= 8 run the decode
 * path one after the other.  The problems must be independent: no output may
 * overlap another problem's input or output.
 *   n          1 <= n <= QN_MAX_GROUP.
 *   problems   host array of n descriptors; each follows qlora_linear_fwd's
 *              rules (QN_ERR_* of the first failing problem).
 *   workspace  device, >= qlora_workspace_size_grouped(n, problems) bytes,
 *              256-byte aligned. */
typedef struct {
  const void *X;        /* bf16 [M, K]                                 */
  int64_t M;
  qn_nf4_weight W;      /* [N, K]                                      */
  const void *A;        /* bf16 [r, K]                                 */
  const void *B;        /* bf16 [N, r]                                 */
  int64_t r;
  float alpha;
  void *Y;              /* bf16 [M, N] out                             */
  float *H_out;         /* fp32 [M, r] out, or NULL                    */
} qlora_fwd_problem;
size_t qlora_workspace_size_grouped(int n, const qlora_fwd_problem *problems);
int qlora_linear_fwd_grouped(int n, const qlora_fwd_problem *problems, void *workspace,
                             size_t ws_bytes, void *stream);

/* No-allocation variant of qlora_linear_fwd, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and shape rules as qlora_linear_fwd (identical kernels, bit-identical
 * output), without the workspace arguments: the workspace is a static device
 * array of QN_NOALLOC_SCRATCH_BYTES in the library, one per device, kept until
 * the process ends.  The call uses the current device's copy (the device that
 * is current must be the stream's).  Returns QN_ERR_SCRATCH, before anything is
 * launched, when qlora_workspace_size(QN_OP_FWD, M, N, K, r) exceeds it (16 MiB
 * covers decode, M <= 8, at every configured shape and the MFMA path up to
 * M = 43690 at r = 64 or M = 104856 at r = 16).  The first call on a device
 * looks the array's address up (hipGetSymbolAddress); no call allocates or
 * frees memory.  Calls that overlap
 * in time on one device (different streams, or host threads without ordering)
 * share the array and race: the caller serialises them. */
#define QN_NOALLOC_SCRATCH_BYTES (16u << 20)
int qlora_linear_fwd_noalloc(const void *X, int64_t M, const qn_nf4_weight *W,
                             const void *A, const void *B, int64_t r, float alpha,
                             void *Y, float *H_out, void *stream);

/* QLoRA linear backward: gradients reach the adapter only; the frozen base gets
 * none ([QE] "Name the one memory cost LoRA could not remove"; "Turn a LoRA
 * script ...": gradients flow through the frozen 4-bit layers to the adapters).
 * With G = dY, s = alpha/r, H = X A^T:
 *     dH = s G B,  dB = s G^T H,  dA = dH^T X,  dX = G bf16(dequant(W)) + dH A
 *   dY  device bf16 [M, N]; X, A, B as in the forward.
 *   H   device fp32 [M, r]: X A^T as the forward wrote it to H_out, or NULL,
 *       in which case it is recomputed from X and A (one more read of X).
 *       With H given, dB uses bf16(s H) of these values; 4-byte aligned.
 *   dX  device bf16 [M, K] out, or NULL to skip it.
 *   dA  device bf16 [r, K] out;  dB device bf16 [N, r] out.
 *   workspace  device, >= qlora_workspace_size(QN_OP_BWD, M, N, K, r) bytes.
 * Same shape rules as the forward. */
int qlora_linear_bwd(const void *dY, const void *X, const float *H, int64_t M,
                     const qn_nf4_weight *W, const void *A, const void *B,
                     int64_t r, float alpha, void *dX, void *dA, void *dB,
                     void *workspace, size_t ws_bytes, void *stream);

/* Kernel-level timing log, for measurement (off by default; costs nothing when
 * off).  While enabled, each call brackets its dominant kernel with two HIP
 * events recorded on the call's own stream and logs them under one of the
 * QN_TRACE_* kinds below.  qn_trace_enable(1) clears the log and starts
 * logging, qn_trace_enable(0) stops.  qn_trace_read() waits for the logged
 * events, writes up to `cap` (kind, milliseconds) entries to host arrays,
 * clears the log and returns the number written (negative qn_status on error).
 * Not for use under HIP graph capture. */
#define QN_TRACE_QUANTIZE 1      /* nf4_quantize kernel                          */
#define QN_TRACE_DOUBLE_QUANT 2  /* nf4_double_quant kernel                      */
#define QN_TRACE_DEQUANT 3       /* nf4_dequant kernel                           */
#define QN_TRACE_GEMV 4          /* decode-path streaming kernel (fwd, M <= 8)   */
#define QN_TRACE_GEMM_FWD 5      /* forward dequant-GEMM tile kernel (M > 8)     */
#define QN_TRACE_GEMM_DX 6       /* backward dX dequant-GEMM tile kernel         */
#define QN_TRACE_GEMM_DB 7       /* backward dA and dB contractions over M (one  */
                                 /* launch carries both)                         */
#define QN_TRACE_GEMM_DA 8       /* reserved (dA shares the launch of kind 7)    */
#define QN_TRACE_LOWRANK 9       /* X A^T or dY B low-rank product               */
#define QN_TRACE_MERGE 10        /* qlora_merge kernel                           */
#define QN_TRACE_ADAMW8 11       /* qn_adamw8_step(_multi) kernel                */
int qn_trace_enable(int on);
int qn_trace_read(int *kinds, float *ms, int cap);

/* Tiling of the dequant-GEMMs (forward and the backward's dX) for the calls
 * that follow, process-wide (for measurement and tests; results are the same
 * either way up to the order of fp32 accumulation within a tile, which the
 * tilings share; dX has tilings 1 and 2 only, and 3 selects 2 there):
 *   0  automatic (the default): per launch, the tiling whose rounds of tiles
 *      over the compute units, weighted by the measured time of one tile,
 *      finish first (256 x 256 tiles for large launches, 256 x 128 for small
 *      ones or where the wide tiles leave a partial round);
 *   1  256 x 128 tiles: four MFMA waves and four dequantising waves;
 *   2  256 x 256 tiles: eight waves that all multiply and dequantise;
 *   3  256 x 256 tiles: four such waves, 128 x 128 each.
 * QN_ERR_VALUE for any other value. */
int qn_set_gemm_variant(int variant);

/* Human-readable name of a qn_status (static storage). */
const char *qn_status_string(int status);

/* Library version string (static storage). */
const char *qn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
