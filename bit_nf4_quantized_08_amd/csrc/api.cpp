// C ABI entry points: argument validation (host only, before any launch) and
// dispatch to the kernels.  Declared in include/qlora_nf4.h.

#include <cmath>
#include <cstdint>
#include <cstring>

#include "qn_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // far above any HBM size; guards overflow

int check_weight(const qn_nf4_weight *W) {
  if (!W || !W->codes) return QN_ERR_NULL;
  if (W->N <= 0 || W->K <= 0 || W->N > kMaxElems / W->K) return QN_ERR_SHAPE;
  if (W->absmax_q) {
    if (!W->scale2) return QN_ERR_NULL;
    if (!aligned(W->absmax_q, 4) || !aligned(W->scale2, 4)) return QN_ERR_ALIGN;
  } else {
    if (!W->absmax) return QN_ERR_NULL;
    if (!aligned(W->absmax, 4)) return QN_ERR_ALIGN;
  }
  if (!aligned(W->codes, 16)) return QN_ERR_ALIGN;
  return QN_OK;
}

int check_linear_shapes(int64_t M, const qn_nf4_weight *W, int64_t r, float alpha) {
  if (M <= 0 || r < 1 || r > QN_MAX_RANK) return QN_ERR_SHAPE;
  if (W->K % QN_BLOCK != 0 || W->N % QN_BLOCK != 0) return QN_ERR_SHAPE;
  if (M > kMaxElems / W->K || M > kMaxElems / W->N) return QN_ERR_SHAPE;
  if (M > INT32_MAX / 64 || W->N > INT32_MAX / 64) return QN_ERR_SHAPE;
  if (!std::isfinite(alpha)) return QN_ERR_VALUE;
  return QN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QN_OK : QN_ERR_HIP; }

}  // namespace

extern "C" {

int qn_codebook(float out[16]) {
  if (!out) return QN_ERR_NULL;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  std::memcpy(out, qn::codec_tables().code, 16 * sizeof(float));
  return QN_OK;
}

int nf4_quantize(const void *W, int w_dtype, int64_t N, int64_t K, uint8_t *codes, float *absmax,
                 void *stream) {
  if (!W || !codes || !absmax) return QN_ERR_NULL;
  if (w_dtype != QN_F32 && w_dtype != QN_BF16) return QN_ERR_DTYPE;
  if (N <= 0 || K <= 0 || N > kMaxElems / K) return QN_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(codes, 8) || !aligned(absmax, 4)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  return hip_status(qn::launch_quantize(W, w_dtype == QN_BF16, N * K, codes, absmax,
                                        static_cast<hipStream_t>(stream)));
}

int nf4_double_quant(const float *absmax, int64_t nb, uint8_t *absmax_q, float *scale2, void *stream) {
  if (!absmax || !absmax_q || !scale2) return QN_ERR_NULL;
  if (nb <= 0 || nb > kMaxElems / QN_BLOCK) return QN_ERR_SHAPE;
  if ((nb + QN_GROUP - 1) / QN_GROUP > (int64_t)INT32_MAX) return QN_ERR_SHAPE;
  if (!aligned(absmax, 4) || !aligned(scale2, 4)) return QN_ERR_ALIGN;
  return hip_status(qn::launch_double_quant(absmax, nb, absmax_q, scale2, static_cast<hipStream_t>(stream)));
}

int nf4_dequant(const qn_nf4_weight *W, void *out, int out_dtype, void *stream) {
  int st = check_weight(W);
  if (st != QN_OK) return st;
  if (!out) return QN_ERR_NULL;
  if (out_dtype != QN_F32 && out_dtype != QN_BF16) return QN_ERR_DTYPE;
  if (!aligned(out, 16)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  return hip_status(qn::launch_dequant(*W, out, out_dtype == QN_BF16, static_cast<hipStream_t>(stream)));
}

size_t qlora_workspace_size(int op, int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 1 || r > QN_MAX_RANK) return 0;
  if (K % QN_BLOCK != 0 || N % QN_BLOCK != 0) return 0;
  if (M > kMaxElems / K || M > kMaxElems / N) return 0;
  if (op == QN_OP_FWD) return qn::fwd_workspace(M, N, K, r);
  if (op == QN_OP_BWD) return qn::bwd_workspace(M, N, K, r);
  return 0;
}

int qlora_linear_fwd(const void *X, int64_t M, const qn_nf4_weight *W, const void *A, const void *B, int64_t r,
                     float alpha, void *Y, float *H_out, void *workspace, size_t ws_bytes, void *stream) {
  int st = check_weight(W);
  if (st != QN_OK) return st;
  if (!X || !A || !B || !Y) return QN_ERR_NULL;
  st = check_linear_shapes(M, W, r, alpha);
  if (st != QN_OK) return st;
  if (!aligned(X, 16) || !aligned(A, 16) || !aligned(B, 16) || !aligned(Y, 16)) return QN_ERR_ALIGN;
  if (H_out && !aligned(H_out, 4)) return QN_ERR_ALIGN;
  const size_t need = qn::fwd_workspace(M, W->N, W->K, r);
  if (!workspace || ws_bytes < need) return QN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  qn::FwdArgs a{};
  a.X = static_cast<const uint16_t *>(X);
  a.M = M; a.N = W->N; a.K = W->K; a.r = r;
  a.codes = W->codes;
  a.sc = qn::ScaleSrc{W->absmax, W->absmax_q, W->scale2};
  a.A = static_cast<const uint16_t *>(A);
  a.B = static_cast<const uint16_t *>(B);
  a.s = alpha / (float)r;
  a.Y = static_cast<uint16_t *>(Y);
  a.H_out = H_out;
  a.ws = workspace; a.ws_bytes = ws_bytes;
  return hip_status(qn::run_fwd(a, static_cast<hipStream_t>(stream)));
}

int qlora_linear_bwd(const void *dY, const void *X, int64_t M, const qn_nf4_weight *W, const void *A,
                     const void *B, int64_t r, float alpha, void *dX, void *dA, void *dB, void *workspace,
                     size_t ws_bytes, void *stream) {
  int st = check_weight(W);
  if (st != QN_OK) return st;
  if (!dY || !X || !A || !B || !dA || !dB) return QN_ERR_NULL;
  st = check_linear_shapes(M, W, r, alpha);
  if (st != QN_OK) return st;
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(A, 16) || !aligned(B, 16) || !aligned(dA, 16) ||
      !aligned(dB, 16) || (dX && !aligned(dX, 16)))
    return QN_ERR_ALIGN;
  const size_t need = qn::bwd_workspace(M, W->N, W->K, r);
  if (!workspace || ws_bytes < need) return QN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  qn::BwdArgs a{};
  a.dY = static_cast<const uint16_t *>(dY);
  a.X = static_cast<const uint16_t *>(X);
  a.M = M; a.N = W->N; a.K = W->K; a.r = r;
  a.codes = W->codes;
  a.sc = qn::ScaleSrc{W->absmax, W->absmax_q, W->scale2};
  a.A = static_cast<const uint16_t *>(A);
  a.B = static_cast<const uint16_t *>(B);
  a.s = alpha / (float)r;
  a.dX = static_cast<uint16_t *>(dX);
  a.dA = static_cast<uint16_t *>(dA);
  a.dB = static_cast<uint16_t *>(dB);
  a.ws = workspace; a.ws_bytes = ws_bytes;
  return hip_status(qn::run_bwd(a, static_cast<hipStream_t>(stream)));
}

const char *qn_status_string(int status) {
  switch (status) {
    case QN_OK: return "ok";
    case QN_ERR_NULL: return "null pointer";
    case QN_ERR_SHAPE: return "invalid shape";
    case QN_ERR_DTYPE: return "invalid dtype";
    case QN_ERR_ALIGN: return "misaligned pointer";
    case QN_ERR_WORKSPACE: return "workspace missing or too small";
    case QN_ERR_HIP: return "HIP launch error";
    case QN_ERR_VALUE: return "invalid scalar value";
    default: return "unknown status";
  }
}

const char *qn_version(void) { return "qlora_nf4 0.1 (gfx950)"; }

}  // extern "C"
