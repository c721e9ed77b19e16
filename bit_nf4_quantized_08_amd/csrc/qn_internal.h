// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora_nf4.h"

namespace qn {

// Tables handed to the codec kernels by value (they live in the kernel argument
// segment; kernels copy what they index dynamically into LDS), one per 4-bit
// type (QN_NF4, QN_FP4).
//   code[16]      the table's values by code (fp32).
//   thr[33], base[33], lohi[33]  bucket table for the nearest-value search: a
//   normalised value n in [-1, 1 + 2^-23] falls into bucket b = floor(16 n +
//   16) (0 .. 32; bucket 32 holds n >= 1); its level is base[b] + (n >=
//   thr[b]) among the distinct values in ascending order, and its code is
//   byte (n >= thr[b]) of lohi[b].  For NF4 the code of a level is the level
//   itself.
constexpr int kBuckets = 33;
struct CodecTables {
  float code[16];
  float thr[kBuckets];
  uint32_t base[kBuckets];
  uint32_t lohi[kBuckets];
};

// Host: the tables of a 4-bit type (codebook.cpp).  Idempotent, thread-safe.
const CodecTables &codec_tables(int qtype = QN_NF4);
// False if a decision table failed its self-check (never expected).
bool codec_tables_ok();

// Host: fp64 NF4 rows before rounding (exposed for the library's own checks).
void nf4_rows_f64(double out[16]);

// Compute units of the current device (device.cpp); cached per device, thread-safe.
int device_cus();

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
// Quantise n weights; with absmax_q and scale2 non-null the same launch also
// double-quantises the block scales (a workgroup per group of 256 blocks).
hipError_t launch_quantize(const void *W, int w_is_bf16, int64_t n, int qtype, uint8_t *codes,
                           float *absmax, uint8_t *absmax_q, float *scale2, hipStream_t s);
hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *absmax_q,
                               float *scale2, hipStream_t s);
hipError_t launch_dequant(const qn_nf4_weight &W, void *out, int out_bf16, hipStream_t s);
// One 8-bit AdamW step (k_adamw8.hip): the fp32 constants of the step, with
// c1 = 1 - b1, c2 = 1 - b2, bc1 = 1 - b1^t, bc2 = 1 - b2^t formed in fp64 and
// rounded once on the host.
struct AdamConsts {
  float lr, b1, b2, eps, wd, c1, c2, bc1, bc2;
};
hipError_t launch_adamw8(uint16_t *p, const uint16_t *g, int64_t n, int8_t *mq, float *ms, uint8_t *uq, float *us,
                         const AdamConsts &c, hipStream_t s);
// The same step over up to QN_ADAMW_MULTI tensors in one launch: tensor i owns
// spans (of 256 parameters) [first[i], first[i + 1]).
struct AdamTensor {
  uint16_t *p;
  const uint16_t *g;
  int64_t n;
  int8_t *mq;
  float *ms;
  uint8_t *uq;
  float *us;
};
struct AdamMulti {
  AdamTensor t[QN_ADAMW_MULTI];
  int64_t first[QN_ADAMW_MULTI + 1];
  int n;
};
hipError_t launch_adamw8_multi(const AdamMulti &mt, const AdamConsts &c, hipStream_t s);

// Adapter merged into the dequantised base (k_merge.hip).  W.K % 64 == 0, 1 <= r <= 64.
hipError_t launch_merge(const qn_nf4_weight &W, const uint16_t *A, const uint16_t *B, int64_t r, float alpha,
                        void *out, int out_bf16, hipStream_t s);

// Scale of block b: fl32(k_b * step_g) with double quantisation, else
// absmax[b]; qtype names the table the codes index.
struct ScaleSrc {
  const float *absmax;
  const uint8_t *absmax_q;
  const float *scale2;
  int qtype;
};

// The 16 values of a 4-bit table, passed by value to kernels that build LDS
// tables from them.
struct Code16 {
  float v[16];
};
Code16 code16(int qtype = QN_NF4);

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
  int qtype;
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
// Several independent forward products in one launch (n <= QN_MAX_GROUP); the
// problems must agree on the scale source (all double-quantised or none) and
// on the 4-bit type.
hipError_t launch_qgemm_fwd_group(const QGemmArgs *a, int n, hipStream_t s);
// Tiling choice of the dequant-GEMMs (forward and dX) for all later launches: 0 automatic, 1 256 x 128, 2 256 x 256.
void set_gemm_variant(int v);

// Problems of one grouped launch, passed by value in the kernel arguments.
// Workgroups [start[g], start[g+1]) run problem g; each range is a multiple of
// 8 workgroups (the XCD count), the tail ones past the problem's tiles exit.
struct QGemmGroup {
  QGemmArgs p[QN_MAX_GROUP];
  int start[QN_MAX_GROUP + 1];
  int n;
};

// Low-rank product (k_lowrank.hip): C[M, R] = L[M, Kc] * P[R, Kc]^T, R <= 64,
// Kc % 64 == 0.  Writes any of: out_f32 [M, R] (unscaled), out_b [M, ldb] =
// bf16(scale * C) zero beyond R, out_t [ldt_rows, Mp] = bf16(scale * C)^T zero
// beyond R and beyond M (Mp >= M).  The contraction is cut into
// lowrank_splits(M, Kc) ranges whose fp32 partial products go to `part`
// (lowrank_part_bytes(M, Kc, R) bytes of workspace) and are then added in
// range order, so the result depends on the shape alone.
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
  float *part;
  int splits;   // set by the launcher
};
int lowrank_splits(int64_t M, int64_t Kc);
size_t lowrank_part_bytes(int64_t M, int64_t Kc, int64_t R);
hipError_t launch_lowrank(const LowRankArgs &a, hipStream_t s);
// Two independent products with the same rank bucket in one launch (b may be null).
hipError_t launch_lowrank2(const LowRankArgs &a, const LowRankArgs *b, hipStream_t s);
// Up to QN_MAX_GROUP independent products in one launch (blockIdx.y picks one).
hipError_t launch_lowrank_n(const LowRankArgs *a, int n, hipStream_t s);

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
// Several forwards: decode-path problems (M <= 8) as in run_fwd, the others
// with one low-rank launch and one dequant-GEMM launch per scale source.  Each
// problem's workspace is a[g].ws (carved by the caller).
hipError_t run_fwd_group(const FwdArgs *a, int n, hipStream_t s);
// Device address of the current device's static scratch array (k_linear.hip),
// looked up once per device.
hipError_t noalloc_scratch(void **ptr);

struct BwdArgs {
  const uint16_t *dY;    // bf16 [M,N]
  const uint16_t *X;     // bf16 [M,K]
  const float *H;        // fp32 [M,r] = X A^T from the forward, or null (recomputed)
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
