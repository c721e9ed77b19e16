// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora_nf4.h"

namespace qn {

// Tables handed to the codec kernels by value (they live in the kernel argument
// segment; kernels copy what they index dynamically into LDS).
//   code[16]      the NF4 rows (fp32).
//   thr[32], base[32]  bucket table for the nearest-row search: a normalised
//   value n in [-1, 1] falls into bucket b = clamp(int(16 n + 16), 0, 31); the
//   row index is base[b] + (n >= thr[b]).  Built on the host so that each bucket
//   holds at most one decision threshold and every threshold lies far (>1e-4)
//   from a bucket edge, which makes the bucket's own rounding irrelevant.
struct CodecTables {
  float code[16];
  float thr[32];
  uint32_t base[32];
};

// Host: the NF4 table and the bucket table (codebook.cpp).  Idempotent, thread-safe.
const CodecTables &codec_tables();
// False if the bucket table failed its self-check (never expected).
bool codec_tables_ok();

// Host: fp64 NF4 rows before rounding (exposed for the library's own checks).
void nf4_rows_f64(double out[16]);

// Kernel-level timing (trace.cpp).  While tracing is enabled, an object of this
// type records a start event on construction and a stop event on destruction,
// on the given stream, and logs the pair under `kind` (QN_TRACE_* codes).
class TraceScope {
 public:
  TraceScope(int kind, hipStream_t s);
  ~TraceScope();
  TraceScope(const TraceScope &) = delete;
  TraceScope &operator=(const TraceScope &) = delete;

 private:
  int kind_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// Kernel launchers (return hipError_t of the launch).
hipError_t launch_quantize(const void *W, int w_is_bf16, int64_t n, uint8_t *codes,
                           float *absmax, hipStream_t s);
hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *absmax_q,
                               float *scale2, hipStream_t s);
hipError_t launch_dequant(const qn_nf4_weight &W, void *out, int out_bf16, hipStream_t s);

// Scale of block b: fl32(k_b * step_g) with double quantisation, else absmax[b].
struct ScaleSrc {
  const float *absmax;
  const uint8_t *absmax_q;
  const float *scale2;
};

// The 16 NF4 rows passed by value to kernels that build LDS tables from them.
struct Code16 {
  float v[16];
};
Code16 code16();

// Dequant-GEMM (k_qgemm.hip).  out[M, Nout] (bf16) =
//   sum_k L[m, k] * W_hat(k, n)  +  sum_{j<r} L2[m, j] * R2(j, n)
// where W_hat(k, n) = bf16(fl32(table[q] * scale)) of weight element
//   (n, k) of codes [Nout, Kc]   (forward, "NK"), or
//   (k, n) of codes [Kc, Nout]   (dX, "KN"),
// and R2(j, n) = R2[n*ldr2 + j] (forward) or R2[j*ldr2 + n] (dX).
// Requires Kc % 64 == 0 and Nout % 64 == 0.
struct QGemmArgs {
  const uint16_t *L;
  int64_t ldl;
  int64_t M, Nout, Kc;
  const uint8_t *codes;
  const float *absmax;
  const uint8_t *absmax_q;
  const float *scale2;
  const uint16_t *L2;
  int64_t ldl2;
  const uint16_t *R2;
  int64_t ldr2;
  int64_t r;
  uint16_t *out;
  int64_t ldo;
  int tiles_m, tiles_n, group_m;
};
hipError_t launch_qgemm_fwd(const QGemmArgs &a, hipStream_t s);
hipError_t launch_qgemm_dx(const QGemmArgs &a, hipStream_t s);

// Low-rank product (k_lowrank.hip): C[M, R] = L[M, Kc] * P[R, Kc]^T, R <= 64,
// Kc % 32 == 0.  Writes any of: out_f32 [M, R] (unscaled), out_b [M, ldb] =
// bf16(scale * C) zero beyond R, out_t [ldt_rows, Mp] = bf16(scale * C)^T zero
// beyond R and beyond M (Mp >= M).
struct LowRankArgs {
  const uint16_t *L;
  int64_t ldl, M, Kc;
  const uint16_t *P;
  int64_t ldp, R;
  float scale;
  float *out_f32;
  uint16_t *out_b;
  int64_t ldb;
  uint16_t *out_t;
  int64_t ldt_rows, Mp;
};
hipError_t launch_lowrank(const LowRankArgs &a, hipStream_t s);
// Two independent products with the same rank bucket in one launch (b may be null).
hipError_t launch_lowrank2(const LowRankArgs &a, const LowRankArgs *b, hipStream_t s);

// Column-streaming reduction over rows (k_lowrank.hip): out = bf16(sum_m
// Lt[j][m] * Q[m][c]) for j < R <= 64, as [R][Ncols] or transposed [Ncols][R].
// Lt is [>= R rows, Mp] bf16 zero beyond M; Q is [M, Ncols] bf16, leading dim
// ldq.  `part` holds colred_splits(M) * R * Ncols floats.
struct ColRedArgs {
  const uint16_t *Lt;
  int64_t Mp;
  const uint16_t *Q;
  int64_t ldq, M, Ncols, R;
  float *part;
  uint16_t *out;
  bool transpose;
};
int colred_splits(int64_t M);
hipError_t launch_colred(const ColRedArgs &a, hipStream_t s, int trace_kind);
// Two independent reductions over the same M in one launch (b may be null);
// each needs its own `part`.
hipError_t launch_colred2(const ColRedArgs &a, const ColRedArgs *b, hipStream_t s, int trace_kind);

// Forward pieces.
struct FwdArgs {
  const uint16_t *X;     // bf16 [M,K]
  int64_t M, N, K, r;
  const uint8_t *codes;
  ScaleSrc sc;
  const uint16_t *A;     // bf16 [r,K]
  const uint16_t *B;     // bf16 [N,r]
  float s;               // alpha / r
  uint16_t *Y;           // bf16 [M,N]
  float *H_out;          // fp32 [M,r] or null
  void *ws;
  size_t ws_bytes;
};
size_t fwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r);
hipError_t run_fwd(const FwdArgs &a, hipStream_t s);

struct BwdArgs {
  const uint16_t *dY;    // bf16 [M,N]
  const uint16_t *X;     // bf16 [M,K]
  int64_t M, N, K, r;
  const uint8_t *codes;
  ScaleSrc sc;
  const uint16_t *A;     // bf16 [r,K]
  const uint16_t *B;     // bf16 [N,r]
  float s;
  uint16_t *dX;          // bf16 [M,K] or null
  uint16_t *dA;          // bf16 [r,K]
  uint16_t *dB;          // bf16 [N,r]
  void *ws;
  size_t ws_bytes;
};
size_t bwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r);
hipError_t run_bwd(const BwdArgs &a, hipStream_t s);

}  // namespace qn
