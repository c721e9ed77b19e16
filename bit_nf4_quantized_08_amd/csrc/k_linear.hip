// QLoRA linear layer kernels for gfx950: forward and backward.
//
// "LoRA vs QLoRA: Efficient Fine-Tuning Explained", "How LoRA Works": the layer
// is the frozen W plus (alpha/r) B A.  "QLoRA Explained: A 4-Bit Base, NF4, and
// What It Really Costs", "Predict the throughput tax before you pay it": the
// matrix unit cannot read a row index, so each multiply first reads the 4-bit
// codes, looks each one up in the table, scales it by its block's scale, and
// writes bf16 values to on-chip memory for the matrix unit; "Why it is ever
// worth paying": a pass must read every weight, which makes small-batch decode
// bound by weight bandwidth.
//
// Kernels in this file (the dequant-GEMMs are in k_qgemm.hip, the low-rank
// products and column reductions in k_lowrank.hip):
//   gemv_kernel           decode path (M <= 8): streams codes at HBM rate,
//                         expands byte pairs through an LDS table and
//                         accumulates with v_dot2_f32_bf16; per-block scale
//                         applied to partial sums.  Its first blocks compute
//                         the adapter's H partials.
//   gemv_epilogue_kernel  adds the split partials and the adapter term.
//   transpose_bf16_kernel B^T for the backward's dH = dY B.

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;        // contraction step: one NF4 block along K
__device__ __forceinline__ float scale_of(const ScaleSrc &sc, int64_t b) {
  if (sc.absmax_q) return (float)sc.absmax_q[b] * sc.scale2[b / QN_GROUP];
  return sc.absmax[b];
}

// Transpose a small bf16 matrix: out[c][r] = in[r][c] for c < C, rows of out
// beyond C (up to out_rows) zero.  in is [R, C] with leading dim ldi.
__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(const uint16_t *__restrict__ in, int64_t R,
                                                                  int64_t C, int64_t ldi,
                                                                  uint16_t *__restrict__ out, int64_t out_rows) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // over out_rows * R
  if (idx >= out_rows * R) return;
  const int64_t c = idx / R, r = idx % R;
  out[c * R + r] = (c < C) ? in[r * ldi + c] : (uint16_t)0;
}

// ================================================================ GEMV (decode)
// y_part[split][m][n] = sum over this split's K-range of x[m][k] * W_hat[n][k],
// the block scale applied to each 32-weight partial sum.  Lane l of a wave owns
// 32 consecutive k of every 2048-wide chunk (16 bytes of codes).  A wave works on
// RPW rows at once so that each lane's x registers are reused RPW times.
// The first h_blocks blocks instead compute H partials,
// h_part[split][m][j] = sum over the split's K-range of x[m][k] * A[j][k]:
// block b takes K-range b % hsplits and adapter rows 4 (b / hsplits) .. +3,
// one per wave, so that every wave makes a single pass and H is spread over
// many short blocks that start first.
constexpr int GEMV_RPW = 4;                       // rows per wave
constexpr int GEMV_ROWS = GEMV_RPW * (kThreads / 64);  // rows per workgroup

struct GemvArgs {
  const uint16_t *X;  // [M, K]
  int64_t M, N, K;
  const uint8_t *codes;
  ScaleSrc sc;
  const uint16_t *A;  // [r, K]
  int64_t r;
  float *y_part;      // [splits][M][N]
  float *h_part;      // [hsplits][M][64]
  int64_t k_per_split;   // multiple of 2048 (or K)
  int splits;
  int h_blocks;       // hsplits * ceil(r / 4)
  int hsplits;
  int64_t hk_per_split;  // H partial K-range per block (multiple of 2048 or K)
};

template <int MM>
__device__ __forceinline__ void load_x_chunk(const GemvArgs &a, int64_t k, bool valid, uint32_t (&x)[MM][16]) {
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    if (valid && m < a.M) {
      const u32x4 *p = reinterpret_cast<const u32x4 *>(a.X + m * a.K + k);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 v = p[c];
        x[m][4 * c] = v.x; x[m][4 * c + 1] = v.y; x[m][4 * c + 2] = v.z; x[m][4 * c + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) x[m][c] = 0;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int MM>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a, Code16 cb) {
  __shared__ uint32_t pairs[256];  // byte -> bf16(row lo) | bf16(row hi) << 16
  {
    const uint32_t v = threadIdx.x;
    pairs[v] = pack_bf16x2(cb.v[v & 15], cb.v[v >> 4]);
  }
  __syncthreads();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if ((int)blockIdx.x < a.h_blocks) {
    // ---- H partials (see above).
    const int hb = (int)blockIdx.x % a.hsplits;
    const int64_t kb = (int64_t)hb * a.hk_per_split;
    const int64_t ke = min(a.K, kb + a.hk_per_split);
    const int j = 4 * ((int)blockIdx.x / a.hsplits) + wave;
    if (j < a.r) {
      float hm[MM];
#pragma unroll
      for (int m = 0; m < MM; ++m) hm[m] = 0.0f;
      for (int64_t k = kb + lane * 32; k < ke; k += 2048) {
        uint32_t x[MM][16];
        load_x_chunk<MM>(a, k, true, x);
        const u32x4 *pa = reinterpret_cast<const u32x4 *>(a.A + j * a.K + k);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 av = pa[c];
          const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int m = 0; m < MM; ++m)
              hm[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[q]),
                                                      __builtin_bit_cast(bf16x2, x[m][4 * c + q]), hm[m], false);
        }
      }
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const float t = wave_sum(hm[m]);
        if (lane == 0 && m < a.M) a.h_part[((int64_t)hb * a.M + m) * 64 + j] = t;
      }
    }
    return;
  }

  const int gb = (int)blockIdx.x - a.h_blocks;
  const int rb = gb / a.splits;
  const int split = gb % a.splits;
  const int64_t n_base = (int64_t)rb * GEMV_ROWS + wave * GEMV_RPW;
  const int64_t kb = (int64_t)split * a.k_per_split;
  const int64_t ke = min(a.K, kb + a.k_per_split);

  float acc[GEMV_RPW][MM];
#pragma unroll
  for (int i = 0; i < GEMV_RPW; ++i)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[i][m] = 0.0f;

  for (int64_t kc = kb; kc < ke; kc += 2048) {
    const int64_t k = kc + lane * 32;
    const bool kvalid = k < ke;
    uint32_t x[MM][16];
    load_x_chunk<MM>(a, k, kvalid, x);
#pragma unroll
    for (int i = 0; i < GEMV_RPW; ++i) {
      const int64_t n = n_base + i;
      if (!kvalid || n >= a.N) continue;
      const int64_t e = n * a.K + k;
      const u32x4 cw = ld_stream(a.codes + (e >> 1));
      const float A = scale_of(a.sc, e >> 6);
      const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
      float p[MM];
#pragma unroll
      for (int m = 0; m < MM; ++m) p[m] = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t pr = pairs[(w[q] >> (8 * b)) & 0xFF];
#pragma unroll
          for (int m = 0; m < MM; ++m)
            p[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr),
                                                   __builtin_bit_cast(bf16x2, x[m][4 * q + b]), p[m], false);
        }
#pragma unroll
      for (int m = 0; m < MM; ++m) acc[i][m] = __builtin_fmaf(A, p[m], acc[i][m]);
    }
  }
#pragma unroll
  for (int i = 0; i < GEMV_RPW; ++i) {
    const int64_t n = n_base + i;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float t = wave_sum(acc[i][m]);
      if (lane == 0 && n < a.N && m < a.M) a.y_part[((int64_t)split * a.M + m) * a.N + n] = t;
    }
  }
}

// y[m][n] = sum_s y_part[s][m][n] + s_lora * sum_j H[m][j] * B[n][j], H summed
// from its partials; rounded to bf16.  Optionally writes H (fp32, unscaled).
__global__ __launch_bounds__(kThreads) void gemv_epilogue_kernel(const float *__restrict__ y_part, int splits,
                                                                 const float *__restrict__ h_part, int hsplits,
                                                                 int64_t M, int64_t N, int64_t r,
                                                                 const uint16_t *__restrict__ B, float s_lora,
                                                                 uint16_t *__restrict__ Y, float *H_out) {
  __shared__ float Hs[8 * 64];
  for (int idx = threadIdx.x; idx < M * 64; idx += kThreads) {
    const int m = idx / 64, j = idx % 64;
    float v = 0.0f;
    if (j < r)
      for (int s = 0; s < hsplits; ++s) v += h_part[((int64_t)s * M + m) * 64 + j];
    Hs[idx] = v;
    if (H_out && blockIdx.x == 0 && j < r) H_out[m * r + j] = v;
  }
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float y = 0.0f;
  for (int s = 0; s < splits; ++s) y += y_part[((int64_t)s * M + m) * N + n];
  float l = 0.0f;
  for (int j = 0; j < r; ++j) l = __builtin_fmaf(Hs[m * 64 + j], bf16_to_f32(B[n * r + j]), l);
  Y[m * N + n] = f32_to_bf16(__builtin_fmaf(s_lora, l, y));
}

// ================================================================ host side
int num_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) cus = p.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return cus;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// A bump allocator over the caller's workspace (256-B aligned pieces).
struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *p) : base(static_cast<char *>(p)) {}
  template <typename T>
  T *take(int64_t count) {
    T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
    off += (size_t)align_up((int64_t)(count * (int64_t)sizeof(T)), 256);
    return p;
  }
};

// Decode path sizing.
constexpr int64_t GEMV_MAX_M = 8;

void gemv_plan(int64_t M, int64_t N, int64_t K, int &splits, int64_t &kps, int &hsplits, int64_t &hkps) {
  (void)M;
  const int64_t row_blocks = cdiv(N, GEMV_ROWS);
  const int64_t chunks = cdiv(K, 2048);
  const int64_t target = 4LL * num_cus();
  int64_t sp = 1;
  while (row_blocks * sp < target && sp * 2 <= chunks) sp *= 2;
  splits = (int)sp;
  kps = cdiv(chunks, sp) * 2048;
  splits = (int)cdiv(K, kps);
  hkps = 2048 * cdiv(chunks, std::min<int64_t>(chunks, 64));
  hsplits = (int)cdiv(K, hkps);
}

#define QN_TRY(x)                      \
  do {                                 \
    hipError_t e_ = (x);               \
    if (e_ != hipSuccess) return e_;   \
  } while (0)

}  // namespace

// ---------------------------------------------------------------- forward
size_t fwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r) {
  Carve c(nullptr);
  if (M <= GEMV_MAX_M) {
    int splits, hsplits;
    int64_t kps, hkps;
    gemv_plan(M, N, K, splits, kps, hsplits, hkps);
    c.take<float>((int64_t)splits * M * N);
    c.take<float>((int64_t)hsplits * M * 64);
  } else {
    c.take<uint16_t>(M * align_up(r, 8));
  }
  return c.off;
}

hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
  Carve c(a.ws);
  if (a.M <= GEMV_MAX_M) {
    int splits, hsplits;
    int64_t kps, hkps;
    gemv_plan(a.M, a.N, a.K, splits, kps, hsplits, hkps);
    float *y_part = c.take<float>((int64_t)splits * a.M * a.N);
    float *h_part = c.take<float>((int64_t)hsplits * a.M * 64);
    const int row_blocks = (int)cdiv(a.N, GEMV_ROWS);
    const int h_blocks = hsplits * (int)cdiv(a.r, 4);
    GemvArgs ga{a.X, a.M, a.N, a.K, a.codes, a.sc, a.A, a.r, y_part, h_part, kps, splits,
                h_blocks, hsplits, hkps};
    dim3 grid((unsigned)(h_blocks + row_blocks * splits));
    const Code16 cb = code16();
    TraceScope tr(QN_TRACE_GEMV, st);
    if (a.M == 1) hipLaunchKernelGGL(gemv_kernel<1>, grid, dim3(kThreads), 0, st, ga, cb);
    else if (a.M <= 2) hipLaunchKernelGGL(gemv_kernel<2>, grid, dim3(kThreads), 0, st, ga, cb);
    else if (a.M <= 4) hipLaunchKernelGGL(gemv_kernel<4>, grid, dim3(kThreads), 0, st, ga, cb);
    else hipLaunchKernelGGL(gemv_kernel<8>, grid, dim3(kThreads), 0, st, ga, cb);
    QN_TRY(hipGetLastError());
    hipLaunchKernelGGL(gemv_epilogue_kernel, dim3((unsigned)cdiv(a.M * a.N, kThreads)), dim3(kThreads), 0, st,
                       y_part, splits, h_part, hsplits, a.M, a.N, a.r, a.B, a.s, a.Y, a.H_out);
    return hipGetLastError();
  }
  // MFMA path: H = X A^T (low-rank kernel) -> sH bf16 -> tile GEMM with the
  // adapter term as extra contraction steps.
  const int64_t rp = align_up(a.r, 8);
  uint16_t *sH = c.take<uint16_t>(a.M * rp);
  {
    LowRankArgs la{};
    la.L = a.X; la.ldl = a.K; la.M = a.M; la.Kc = a.K;
    la.P = a.A; la.ldp = a.K; la.R = a.r; la.scale = a.s;
    la.out_f32 = a.H_out; la.out_b = sH; la.ldb = rp; la.out_t = nullptr; la.Mp = a.M;
    QN_TRY(launch_lowrank(la, st));
  }
  QGemmArgs g{};
  g.L = a.X; g.ldl = a.K; g.M = a.M; g.Nout = a.N; g.Kc = a.K;
  g.codes = a.codes; g.absmax = a.sc.absmax; g.absmax_q = a.sc.absmax_q; g.scale2 = a.sc.scale2;
  g.L2 = sH; g.ldl2 = rp; g.R2 = a.B; g.ldr2 = a.r; g.r = a.r;
  g.out = a.Y; g.ldo = a.N;
  return launch_qgemm_fwd(g, st);
}

// ---------------------------------------------------------------- backward

size_t bwd_workspace(int64_t M, int64_t N, int64_t K, int64_t r) {
  Carve c(nullptr);
  const int64_t rp = align_up(r, 32);
  const int64_t Mp = align_up(M, BK);
  c.take<uint16_t>(rp * N);                 // B^T
  c.take<uint16_t>(M * rp);                 // dH bf16 [M, rp]
  c.take<uint16_t>(rp * Mp);                // dH^T bf16 [rp, Mp]
  c.take<uint16_t>(rp * Mp);                // (sH)^T bf16 [rp, Mp]
  c.take<float>((int64_t)colred_splits(M) * r * N);   // dB partials
  c.take<float>((int64_t)colred_splits(M) * r * K);   // dA partials
  return c.off;
}

hipError_t run_bwd(const BwdArgs &a, hipStream_t st) {
  Carve c(a.ws);
  const int64_t rp = align_up(a.r, 32);
  const int64_t Mp = align_up(a.M, BK);
  uint16_t *Bt = c.take<uint16_t>(rp * a.N);
  uint16_t *dHb = c.take<uint16_t>(a.M * rp);
  uint16_t *dHt = c.take<uint16_t>(rp * Mp);
  uint16_t *sHt = c.take<uint16_t>(rp * Mp);
  float *bpart = c.take<float>((int64_t)colred_splits(a.M) * a.r * a.N);
  float *apart = c.take<float>((int64_t)colred_splits(a.M) * a.r * a.K);

  // B^T [rp, N] (rows >= r zero) so that dH = dY (B^T)^T runs on the low-rank kernel.
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)cdiv(rp * a.N, kThreads)), dim3(kThreads), 0, st,
                     a.B, a.N, a.r, a.r, Bt, rp);
  QN_TRY(hipGetLastError());
  // One launch: dH = s dY B -> dHb [M, rp], dHt [rp, Mp]; H = X A^T -> (sH)^T [rp, Mp].
  {
    LowRankArgs ld{}, lh{};
    ld.L = a.dY; ld.ldl = a.N; ld.M = a.M; ld.Kc = a.N;
    ld.P = Bt; ld.ldp = a.N; ld.R = a.r; ld.scale = a.s;
    ld.out_b = dHb; ld.ldb = rp; ld.out_t = dHt; ld.ldt_rows = rp; ld.Mp = Mp;
    lh.L = a.X; lh.ldl = a.K; lh.M = a.M; lh.Kc = a.K;
    lh.P = a.A; lh.ldp = a.K; lh.R = a.r; lh.scale = a.s;
    lh.out_t = sHt; lh.ldt_rows = rp; lh.Mp = Mp;
    QN_TRY(launch_lowrank2(ld, &lh, st));
  }

  // One launch: dB [N, r] = ((sH)^T dY)^T and dA [r, K] = dH^T X, contractions over M.
  {
    ColRedArgs cb{}, ca{};
    cb.Lt = sHt; cb.Mp = Mp; cb.Q = a.dY; cb.ldq = a.N; cb.M = a.M; cb.Ncols = a.N; cb.R = a.r;
    cb.part = bpart; cb.out = a.dB; cb.transpose = true;
    ca.Lt = dHt; ca.Mp = Mp; ca.Q = a.X; ca.ldq = a.K; ca.M = a.M; ca.Ncols = a.K; ca.R = a.r;
    ca.part = apart; ca.out = a.dA; ca.transpose = false;
    QN_TRY(launch_colred2(cb, &ca, st, QN_TRACE_GEMM_DB));
  }
  // dX [M, K] = dY [M, N] * W_hat [N, K] + dH [M, r] * A [r, K]
  if (a.dX) {
    QGemmArgs g{};
    g.L = a.dY; g.ldl = a.N; g.M = a.M; g.Nout = a.K; g.Kc = a.N;
    g.codes = a.codes; g.absmax = a.sc.absmax; g.absmax_q = a.sc.absmax_q; g.scale2 = a.sc.scale2;
    g.L2 = dHb; g.ldl2 = rp; g.R2 = a.A; g.ldr2 = a.K; g.r = a.r;
    g.out = a.dX; g.ldo = a.K;
    QN_TRY(launch_qgemm_dx(g, st));
  }
  return hipSuccess;
}

}  // namespace qn
