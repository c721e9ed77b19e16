// C ABI entry points: argument validation (host only, before any launch) and
// dispatch to the kernels.  Declared in include/qlora_nf4.h.

#include <algorithm>
#include <vector>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "qn_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // far above any HBM size; guards overflow

int check_weight(const qn_nf4_weight *W) {
  if (!W || !W->codes) return QN_ERR_NULL;
  if (W->quant_type != QN_NF4 && W->quant_type != QN_FP4) return QN_ERR_DTYPE;
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
  // The GEMM kernels address the code array with 32-bit byte offsets (the
  // transposed reader of the backward spans all of it): N*K/2 bytes must fit.
  if (W->N * W->K / 2 > (int64_t)INT32_MAX) return QN_ERR_SHAPE;
  // The low-rank kernels address 128 rows of X (or dY) with 32-bit offsets.
  if (W->K > (int64_t)1 << 23 || W->N > (int64_t)1 << 23) return QN_ERR_SHAPE;
  if (M > kMaxElems / W->K || M > kMaxElems / W->N) return QN_ERR_SHAPE;
  if (M > INT32_MAX / 64 || W->N > INT32_MAX / 64) return QN_ERR_SHAPE;
  if (!std::isfinite(alpha)) return QN_ERR_VALUE;
  return QN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QN_OK : QN_ERR_HIP; }

// The address a kernel uses for a buffer the caller placed in device memory,
// managed memory, or pinned host memory mapped for the device (the optimizer
// state's host placement); nullptr for anything else, pageable host memory
// included, which a kernel could not reach.
template <typename T>
T *device_view(T *p) {
  void *vp = const_cast<void *>(static_cast<const void *>(p));
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, vp) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return p;
  if (at.type != hipMemoryTypeHost) return nullptr;
  void *dp = nullptr;
  if (hipHostGetDevicePointer(&dp, vp, 0) != hipSuccess || !dp) {
    (void)hipGetLastError();
    return nullptr;
  }
  return static_cast<T *>(dp);
}

int check_adam_tensor(const qn_adamw_tensor &t) {
  if (!t.param || !t.grad || !t.m_q || !t.m_step || !t.u_q || !t.u_step) return QN_ERR_NULL;
  if (t.n <= 0 || t.n > kMaxElems) return QN_ERR_SHAPE;
  if (!aligned(t.param, 16) || !aligned(t.grad, 16) || !aligned(t.m_q, 4) || !aligned(t.u_q, 4) ||
      !aligned(t.m_step, 4) || !aligned(t.u_step, 4))
    return QN_ERR_ALIGN;
  return QN_OK;
}

// Replaces each of a validated tensor's pointers by the address the kernel
// uses (the last check before a launch: it asks the HIP runtime).
int place_adam_tensor(qn_adamw_tensor &t) {
  qn_adamw_tensor d{device_view(t.param), device_view(t.grad), t.n, device_view(t.m_q), device_view(t.m_step),
                    device_view(t.u_q), device_view(t.u_step)};
  if (!d.param || !d.grad || !d.m_q || !d.m_step || !d.u_q || !d.u_step) return QN_ERR_MEMORY;
  t = d;
  return QN_OK;
}

// The step's fp32 constants, 1 - beta and 1 - beta^t formed in double.
int adam_consts(const qn_adamw_config &h, qn::AdamConsts &c) {
  if (h.step < 1 || !std::isfinite(h.lr) || !std::isfinite(h.eps) || !(h.eps > 0.0f) ||
      !std::isfinite(h.weight_decay) || !(h.beta1 >= 0.0f && h.beta1 < 1.0f) || !(h.beta2 >= 0.0f && h.beta2 < 1.0f))
    return QN_ERR_VALUE;
  c.lr = h.lr; c.b1 = h.beta1; c.b2 = h.beta2; c.eps = h.eps; c.wd = h.weight_decay;
  c.c1 = (float)(1.0 - (double)h.beta1);
  c.c2 = (float)(1.0 - (double)h.beta2);
  c.bc1 = (float)(1.0 - std::pow((double)h.beta1, (double)h.step));
  c.bc2 = (float)(1.0 - std::pow((double)h.beta2, (double)h.step));
  return QN_OK;
}

}  // namespace

extern "C" {

int qn_codebook(float out[16]) {
  if (!out) return QN_ERR_NULL;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  std::memcpy(out, qn::codec_tables().code, 16 * sizeof(float));
  return QN_OK;
}

int qn_table(int quant_type, float out[16]) {
  if (!out) return QN_ERR_NULL;
  if (quant_type != QN_NF4 && quant_type != QN_FP4) return QN_ERR_DTYPE;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  std::memcpy(out, qn::codec_tables(quant_type).code, 16 * sizeof(float));
  return QN_OK;
}

int qn_quantize_4bit(const void *W, int w_dtype, int64_t N, int64_t K, int quant_type, uint8_t *codes,
                     float *absmax, uint8_t *absmax_q, float *scale2, void *stream) {
  if (!W || !codes || !absmax) return QN_ERR_NULL;
  if ((absmax_q == nullptr) != (scale2 == nullptr)) return QN_ERR_NULL;
  if (w_dtype != QN_F32 && w_dtype != QN_BF16) return QN_ERR_DTYPE;
  if (quant_type != QN_NF4 && quant_type != QN_FP4) return QN_ERR_DTYPE;
  if (N <= 0 || K <= 0 || N > kMaxElems / K) return QN_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(codes, 8) || !aligned(absmax, 4)) return QN_ERR_ALIGN;
  if (absmax_q && (!aligned(absmax_q, 4) || !aligned(scale2, 4))) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  return hip_status(qn::launch_quantize(W, w_dtype == QN_BF16, N * K, quant_type, codes, absmax, absmax_q, scale2,
                                        static_cast<hipStream_t>(stream)));
}

int nf4_quantize(const void *W, int w_dtype, int64_t N, int64_t K, uint8_t *codes, float *absmax,
                 void *stream) {
  return qn_quantize_4bit(W, w_dtype, N, K, QN_NF4, codes, absmax, nullptr, nullptr, stream);
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

int qlora_merge(const qn_nf4_weight *W, const void *A, const void *B, int64_t r, float alpha, void *out,
                int out_dtype, void *stream) {
  int st = check_weight(W);
  if (st != QN_OK) return st;
  if (!A || !B || !out) return QN_ERR_NULL;
  if (out_dtype != QN_F32 && out_dtype != QN_BF16) return QN_ERR_DTYPE;
  if (r < 1 || r > QN_MAX_RANK || W->K % QN_BLOCK != 0 || W->N > 2097120 || W->K > (1 << 25)) return QN_ERR_SHAPE;
  if (!std::isfinite(alpha)) return QN_ERR_VALUE;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(out, 16)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  return hip_status(qn::launch_merge(*W, static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(B), r,
                                     alpha, out, out_dtype == QN_BF16, static_cast<hipStream_t>(stream)));
}

int qn_adamw8_step(void *param, const void *grad, int64_t n, int8_t *m_q, float *m_step, uint8_t *u_q,
                   float *u_step, const qn_adamw_config *cfg, void *stream) {
  if (!cfg) return QN_ERR_NULL;
  qn_adamw_tensor t{param, grad, n, m_q, m_step, u_q, u_step};
  int st = check_adam_tensor(t);
  if (st != QN_OK) return st;
  qn::AdamConsts c{};
  st = adam_consts(*cfg, c);
  if (st != QN_OK) return st;
  st = place_adam_tensor(t);
  if (st != QN_OK) return st;
  return hip_status(qn::launch_adamw8(static_cast<uint16_t *>(t.param), static_cast<const uint16_t *>(t.grad), n,
                                      t.m_q, t.m_step, t.u_q, t.u_step, c, static_cast<hipStream_t>(stream)));
}

int qn_adamw8_step_multi(int n_tensors, const qn_adamw_tensor *tensors, const qn_adamw_config *cfg, void *stream) {
  if (!tensors || !cfg) return QN_ERR_NULL;
  if (n_tensors < 1) return QN_ERR_SHAPE;
  for (int i = 0; i < n_tensors; ++i) {
    const int st = check_adam_tensor(tensors[i]);
    if (st != QN_OK) return st;
  }
  qn::AdamConsts c{};
  const int st = adam_consts(*cfg, c);
  if (st != QN_OK) return st;
  std::vector<qn_adamw_tensor> dev(tensors, tensors + n_tensors);   // the kernel's addresses
  for (auto &t : dev) {
    const int sp = place_adam_tensor(t);
    if (sp != QN_OK) return sp;
  }
  for (int b = 0; b < n_tensors; b += QN_ADAMW_MULTI) {
    qn::AdamMulti mt{};
    mt.n = std::min(QN_ADAMW_MULTI, n_tensors - b);
    int64_t spans = 0;
    for (int i = 0; i < mt.n; ++i) {
      const qn_adamw_tensor &t = dev[b + i];
      mt.t[i] = qn::AdamTensor{static_cast<uint16_t *>(t.param), static_cast<const uint16_t *>(t.grad), t.n, t.m_q,
                               t.m_step, t.u_q, t.u_step};
      mt.first[i] = spans;
      spans += (t.n + 255) / 256;
    }
    mt.first[mt.n] = spans;
    const int e = hip_status(qn::launch_adamw8_multi(mt, c, static_cast<hipStream_t>(stream)));
    if (e != QN_OK) return e;
  }
  return QN_OK;
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
  a.sc = qn::ScaleSrc{W->absmax, W->absmax_q, W->scale2, W->quant_type};
  a.A = static_cast<const uint16_t *>(A);
  a.B = static_cast<const uint16_t *>(B);
  a.s = alpha / (float)r;
  a.Y = static_cast<uint16_t *>(Y);
  a.H_out = H_out;
  a.ws = workspace; a.ws_bytes = ws_bytes;
  return hip_status(qn::run_fwd(a, static_cast<hipStream_t>(stream)));
}

size_t qlora_workspace_size_grouped(int n, const qlora_fwd_problem *problems) {
  if (n < 1 || n > QN_MAX_GROUP || !problems) return 0;
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    const size_t w = qlora_workspace_size(QN_OP_FWD, problems[i].M, problems[i].W.N, problems[i].W.K, problems[i].r);
    if (w == 0) return 0;
    total += w;   // each piece is a multiple of 256 bytes
  }
  return total;
}

int qlora_linear_fwd_grouped(int n, const qlora_fwd_problem *problems, void *workspace, size_t ws_bytes,
                             void *stream) {
  if (!problems) return QN_ERR_NULL;
  if (n < 1 || n > QN_MAX_GROUP) return QN_ERR_SHAPE;
  qn::FwdArgs args[QN_MAX_GROUP];
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const qlora_fwd_problem &p = problems[i];
    int st = check_weight(&p.W);
    if (st != QN_OK) return st;
    if (!p.X || !p.A || !p.B || !p.Y) return QN_ERR_NULL;
    st = check_linear_shapes(p.M, &p.W, p.r, p.alpha);
    if (st != QN_OK) return st;
    if (!aligned(p.X, 16) || !aligned(p.A, 16) || !aligned(p.B, 16) || !aligned(p.Y, 16)) return QN_ERR_ALIGN;
    if (p.H_out && !aligned(p.H_out, 4)) return QN_ERR_ALIGN;
    qn::FwdArgs &a = args[i];
    a = qn::FwdArgs{};
    a.X = static_cast<const uint16_t *>(p.X);
    a.M = p.M; a.N = p.W.N; a.K = p.W.K; a.r = p.r;
    a.codes = p.W.codes;
    a.sc = qn::ScaleSrc{p.W.absmax, p.W.absmax_q, p.W.scale2, p.W.quant_type};
    a.A = static_cast<const uint16_t *>(p.A);
    a.B = static_cast<const uint16_t *>(p.B);
    a.s = p.alpha / (float)p.r;
    a.Y = static_cast<uint16_t *>(p.Y);
    a.H_out = p.H_out;
    const size_t need = qn::fwd_workspace(p.M, p.W.N, p.W.K, p.r);
    a.ws = workspace ? static_cast<char *>(workspace) + off : nullptr;
    a.ws_bytes = need;
    off += need;
  }
  if (!workspace || ws_bytes < off) return QN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  return hip_status(qn::run_fwd_group(args, n, static_cast<hipStream_t>(stream)));
}

int qlora_linear_fwd_noalloc(const void *X, int64_t M, const qn_nf4_weight *W, const void *A, const void *B,
                             int64_t r, float alpha, void *Y, float *H_out, void *stream) {
  int st = check_weight(W);
  if (st != QN_OK) return st;
  if (!X || !A || !B || !Y) return QN_ERR_NULL;
  st = check_linear_shapes(M, W, r, alpha);
  if (st != QN_OK) return st;
  if (!aligned(X, 16) || !aligned(A, 16) || !aligned(B, 16) || !aligned(Y, 16)) return QN_ERR_ALIGN;
  if (H_out && !aligned(H_out, 4)) return QN_ERR_ALIGN;
  const size_t need = qn::fwd_workspace(M, W->N, W->K, r);
  if (need > (size_t)QN_NOALLOC_SCRATCH_BYTES) return QN_ERR_SCRATCH;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  void *scratch = nullptr;
  if (qn::noalloc_scratch(&scratch) != hipSuccess) return QN_ERR_HIP;
  qn::FwdArgs a{};
  a.X = static_cast<const uint16_t *>(X);
  a.M = M; a.N = W->N; a.K = W->K; a.r = r;
  a.codes = W->codes;
  a.sc = qn::ScaleSrc{W->absmax, W->absmax_q, W->scale2, W->quant_type};
  a.A = static_cast<const uint16_t *>(A);
  a.B = static_cast<const uint16_t *>(B);
  a.s = alpha / (float)r;
  a.Y = static_cast<uint16_t *>(Y);
  a.H_out = H_out;
  a.ws = scratch; a.ws_bytes = QN_NOALLOC_SCRATCH_BYTES;
  return hip_status(qn::run_fwd(a, static_cast<hipStream_t>(stream)));
}

int qlora_linear_bwd(const void *dY, const void *X, const float *H, int64_t M, const qn_nf4_weight *W,
                     const void *A, const void *B, int64_t r, float alpha, void *dX, void *dA, void *dB,
                     void *workspace, size_t ws_bytes, void *stream) {
  int st = check_weight(W);
  if (st != QN_OK) return st;
  if (!dY || !X || !A || !B || !dA || !dB) return QN_ERR_NULL;
  st = check_linear_shapes(M, W, r, alpha);
  if (st != QN_OK) return st;
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(A, 16) || !aligned(B, 16) || !aligned(dA, 16) ||
      !aligned(dB, 16) || (dX && !aligned(dX, 16)) || (H && !aligned(H, 4)))
    return QN_ERR_ALIGN;
  const size_t need = qn::bwd_workspace(M, W->N, W->K, r);
  if (!workspace || ws_bytes < need) return QN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QN_ERR_ALIGN;
  if (!qn::codec_tables_ok()) return QN_ERR_VALUE;
  qn::BwdArgs a{};
  a.dY = static_cast<const uint16_t *>(dY);
  a.X = static_cast<const uint16_t *>(X);
  a.H = H;
  a.M = M; a.N = W->N; a.K = W->K; a.r = r;
  a.codes = W->codes;
  a.sc = qn::ScaleSrc{W->absmax, W->absmax_q, W->scale2, W->quant_type};
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
    case QN_ERR_SCRATCH: return "problem needs more scratch than the static buffer holds";
    case QN_ERR_MEMORY: return "buffer is neither device memory nor pinned host memory mapped for the device";
    default: return "unknown status";
  }
}

int qn_set_gemm_variant(int variant) {
  if (variant < 0 || variant > 3) return QN_ERR_VALUE;
  qn::set_gemm_variant(variant);
  return QN_OK;
}

const char *qn_version(void) { return "qlora_nf4 0.1 (gfx950)"; }

}  // extern "C"
