// Merge of a trained adapter into the dequantised base weight, for export.
//
// "LoRA vs QLoRA: Efficient Fine-Tuning Explained", "How LoRA Works": the
// adapter folds into the base as W + (alpha/r) B A; its FAQ: a QLoRA adapter is
// merged into a dequantised, full-precision copy of the base.  "QLoRA
// Explained: A 4-Bit Base, NF4, and What It Really Costs", "Ship the result,
// and plan for the merge before you need it": the result is a 16-bit
// checkpoint (folding into the 4-bit codes would lose the update).
//
//   w        = fl32(table[q] * A_b)                      (the fp32 dequantisation)
//   acc      = sum_j B[n][j] * A[j][k] in fp32, j increasing, one rounding per
//              step (each product of two bf16 values is exact in fp32, so a
//              fused multiply-add rounds exactly like the product-then-add of
//              the definition)
//   W_m      = fl32(w + fl32(s * acc)),  s = fl32(alpha / r)
//   out      = W_m (fp32) or its bf16 round-to-nearest-even.
//
// Work layout: a workgroup of 4 waves owns 32 rows x 512 columns; a wave owns 8
// rows, a lane 8 consecutive columns (one 16-byte load of each adapter row A[j]
// serves the wave's 8 rows).  The workgroup's 32 rows of B sit in LDS and are
// read as broadcasts.  The contraction costs r fused multiply-adds per output
// element, so for r beyond about 16 the kernel is bound by vector arithmetic
// rather than by HBM.

#pragma clang fp contract(off)

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;
constexpr int ROWS = 32, COLS = 512, WROWS = 8, LCOLS = 8;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0xFFFFFFF0LL;
  const int n = (int)(uint32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

struct MergeArgs {
  const uint8_t *codes;
  ScaleSrc sc;
  int64_t N, K;
  const uint16_t *A;   // [r, K]
  const uint16_t *B;   // [N, r]
  int64_t r;
  float s;
  void *out;           // [N, K] fp32 or bf16
};

template <bool OUT_BF16, bool DQ>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a, Code16 cb) {
  __shared__ __attribute__((aligned(16))) uint16_t Bs[ROWS][64];
  __shared__ float table[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.y * ROWS, k0 = (int64_t)blockIdx.x * COLS;
  if (tid < 16) table[tid] = cb.v[tid];
  for (int idx = tid; idx < ROWS * 64; idx += kThreads) {
    const int row = idx >> 6, j = idx & 63;
    const int64_t n = n0 + row;
    Bs[row][j] = (n < a.N && j < a.r) ? a.B[n * a.r + j] : (uint16_t)0;
  }
  __syncthreads();

  const int64_t k = k0 + lane * LCOLS;
  const bool kin = k < a.K;
  // Adapter rows: lanes past K and rows past r read zeros (out-of-range offsets).
  const rsrc_t ra = make_rsrc(a.A, a.r * a.K * 2);
  float acc[WROWS][LCOLS];
#pragma unroll
  for (int i = 0; i < WROWS; ++i)
#pragma unroll
    for (int c = 0; c < LCOLS; ++c) acc[i][c] = 0.0f;
  const int wr = __builtin_amdgcn_readfirstlane(wave) * WROWS;
  for (int j0 = 0; j0 < a.r; j0 += 8) {
    u32x4 av[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int64_t j = j0 + jj;
      const uint32_t off = (kin && j < a.r) ? (uint32_t)((j * a.K + k) * 2) : kOutOfRange;
      av[jj] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
    }
    u32x4 bv[WROWS];
#pragma unroll
    for (int i = 0; i < WROWS; ++i) bv[i] = *reinterpret_cast<const u32x4 *>(&Bs[wr + i][j0]);
    // Terms j0 .. j0+7 in increasing j; beyond r both factors are zero, and
    // adding +0 leaves the sum unchanged (it starts at +0 and never becomes -0).
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t aw[4] = {av[jj].x, av[jj].y, av[jj].z, av[jj].w};
      float x[LCOLS];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * q] = bf16_lo(aw[q]);
        x[2 * q + 1] = bf16_hi(aw[q]);
      }
#pragma unroll
      for (int i = 0; i < WROWS; ++i) {
        const uint32_t bw[4] = {bv[i].x, bv[i].y, bv[i].z, bv[i].w};
        const float b = (jj & 1) ? bf16_hi(bw[jj >> 1]) : bf16_lo(bw[jj >> 1]);
#pragma unroll
        for (int c = 0; c < LCOLS; ++c) acc[i][c] = __builtin_fmaf(b, x[c], acc[i][c]);
      }
    }
  }
  if (!kin) return;

  // Base weight of each row: 8 codes (4 bytes) in one block of 64.
#pragma unroll
  for (int i = 0; i < WROWS; ++i) {
    const int64_t n = n0 + wr + i;
    if (n >= a.N) break;
    const int64_t e = n * a.K + k;
    const uint32_t cw = *reinterpret_cast<const uint32_t *>(a.codes + e / 2);
    const int64_t blk = e / QN_BLOCK;
    const float A = DQ ? (float)a.sc.absmax_q[blk] * a.sc.scale2[blk / QN_GROUP] : a.sc.absmax[blk];
    float m[LCOLS];
#pragma unroll
    for (int c = 0; c < LCOLS; ++c) {
      const float w = table[(cw >> (4 * c)) & 15] * A;
      const float d = a.s * acc[i][c];
      m[c] = w + d;
    }
    if constexpr (OUT_BF16) {
      st_stream(static_cast<uint16_t *>(a.out) + e,
                u32x4{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]), pack_bf16x2(m[4], m[5]),
                      pack_bf16x2(m[6], m[7])});
    } else {
      float *o = static_cast<float *>(a.out) + e;
      st_stream_f4(o, f32x4{m[0], m[1], m[2], m[3]});
      st_stream_f4(o + 4, f32x4{m[4], m[5], m[6], m[7]});
    }
  }
}

}  // namespace

hipError_t launch_merge(const qn_nf4_weight &W, const uint16_t *A, const uint16_t *B, int64_t r, float alpha,
                        void *out, int out_bf16, hipStream_t st) {
  MergeArgs a{W.codes, ScaleSrc{W.absmax, W.absmax_q, W.scale2, W.quant_type}, W.N, W.K, A, B, r, alpha / (float)r, out};
  const dim3 grid((unsigned)((W.K + COLS - 1) / COLS), (unsigned)((W.N + ROWS - 1) / ROWS));
  const Code16 cb = code16(W.quant_type);
  const bool dq = W.absmax_q != nullptr;
  TraceScope tr(QN_TRACE_MERGE, st);
  if (out_bf16) {
    if (dq) hipLaunchKernelGGL((merge_kernel<true, true>), grid, dim3(kThreads), 0, st, a, cb);
    else hipLaunchKernelGGL((merge_kernel<true, false>), grid, dim3(kThreads), 0, st, a, cb);
  } else {
    if (dq) hipLaunchKernelGGL((merge_kernel<false, true>), grid, dim3(kThreads), 0, st, a, cb);
    else hipLaunchKernelGGL((merge_kernel<false, false>), grid, dim3(kThreads), 0, st, a, cb);
  }
  return hipGetLastError();
}

}  // namespace qn
