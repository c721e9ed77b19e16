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

typedef enum {
  QN_OK = 0,
  QN_ERR_NULL = 1,       /* a required pointer is NULL                           */
  QN_ERR_SHAPE = 2,      /* a size is <= 0, too large, or inconsistent            */
  QN_ERR_DTYPE = 3,      /* unknown qn_dtype                                      */
  QN_ERR_ALIGN = 4,      /* a device pointer is not 16-byte aligned               */
  QN_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than qlora_workspace_size() */
  QN_ERR_HIP = 6,        /* the HIP runtime reported an error on launch           */
  QN_ERR_VALUE = 7       /* a scalar argument is not finite                       */
} qn_status;

typedef enum { QN_F32 = 0, QN_BF16 = 1 } qn_dtype;

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
 * codes 16-byte aligned; absmax, absmax_q and scale2 4-byte aligned.
 */
typedef struct {
  const uint8_t *codes;
  const float *absmax;
  const uint8_t *absmax_q;
  const float *scale2;
  int64_t N;
  int64_t K;
} qn_nf4_weight;

/* The NF4 table, written to host memory out[16] (index 0 = -1, 7 = 0, 15 = +1).
 * [QE] "Put the rows where the weights are", "That is NF4": sixteen values at
 * quantiles of a standard normal, one of them exactly zero, fixed once (not
 * calibrated on a model).  Derived on the host in fp64 (evenly spaced
 * probabilities per half, 7 rows below zero and 8 above, outermost rows at tail
 * probability 31/960, scaled to end at exactly -1 and +1) and rounded to fp32.
 * No device work.  Returns QN_ERR_NULL if out is NULL. */
int qn_codebook(float out[16]);

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
 *   H_out  device fp32 [M, r] out, X*A^T (unscaled), or NULL.
 *   workspace  device, >= qlora_workspace_size(QN_OP_FWD, M, N, K, r) bytes.
 * Requires M >= 1, N % 64 == 0, K % 64 == 0 (whole blocks per row, whole
 * contraction steps in both directions), 1 <= r <= QN_MAX_RANK, finite alpha;
 * workspace 256-byte aligned.
 * M <= 8 runs the streaming decode path (weights read once at HBM rate); larger
 * M runs the MFMA path (tiles dequantised into LDS, bf16 MFMA). */
int qlora_linear_fwd(const void *X, int64_t M, const qn_nf4_weight *W,
                     const void *A, const void *B, int64_t r, float alpha,
                     void *Y, float *H_out, void *workspace, size_t ws_bytes,
                     void *stream);

/* QLoRA linear backward: gradients reach the adapter only; the frozen base gets
 * none ([QE] "Name the one memory cost LoRA could not remove"; "Turn a LoRA
 * script ...": gradients flow through the frozen 4-bit layers to the adapters).
 * With G = dY, s = alpha/r, H = X A^T:
 *     dH = s G B,  dB = s G^T H,  dA = dH^T X,  dX = G bf16(dequant(W)) + dH A
 *   dY  device bf16 [M, N]; X, A, B as in the forward.
 *   dX  device bf16 [M, K] out, or NULL to skip it.
 *   dA  device bf16 [r, K] out;  dB device bf16 [N, r] out.
 *   workspace  device, >= qlora_workspace_size(QN_OP_BWD, M, N, K, r) bytes.
 * Same shape rules as the forward. */
int qlora_linear_bwd(const void *dY, const void *X, int64_t M,
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
int qn_trace_enable(int on);
int qn_trace_read(int *kinds, float *ms, int cap);

/* Human-readable name of a qn_status (static storage). */
const char *qn_status_string(int status);

/* Library version string (static storage). */
const char *qn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
