// Low-rank products of the adapter path on gfx950: C[M, R] = L[M, Kc] * P[R, Kc]^T
// with R <= 64.  Used for H = X A^T (forward and backward) and dH = dY B (with
// P = B^T).
//
// "LoRA vs QLoRA: Efficient Fine-Tuning Explained", "How LoRA Works": the
// adapter's two thin factors, B (d x r) and A (r x k), r small (8 to 64); the
// product through them is cheap next to the base weight, and this kernel
// streams the activations once at HBM rate.
//
// A workgroup of 8 waves owns 16 rows.  The contraction is cut into 32-wide
// chunks dealt round-robin to the 8 waves; each wave accumulates its chunks with
// v_mfma_f32_16x16x32_bf16 (lane group g = lane/16 takes indices [8g, 8g+8) of
// a chunk for both operands), keeping 16 / RT chunks of loads in flight.  The 8
// partial 16 x R results are summed in LDS in a fixed order, and the workgroup
// writes the requested outputs directly: fp32 unscaled, bf16 scaled
// (row-major, zero-padded to ldb columns), bf16 scaled and transposed
// (zero-padded to ldt_rows rows and Mp columns).  No split partials in global
// memory, no second pass.  One launch can carry two independent products
// (blockIdx.y selects the argument set), which the backward uses for H and dH.

#include <algorithm>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int ROWS = 16;
constexpr int CHUNK = 32;
constexpr int UNROLL = 16;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0xFFFFFFF0LL;
  const int n = (int)(uint32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

__host__ __device__ inline int64_t lowrank_rows(const LowRankArgs &a) {
  return a.out_t && a.Mp > a.M ? a.Mp : a.M;
}

struct LowRankGroup {
  LowRankArgs p[QN_MAX_GROUP];
};

template <int RT>  // 16-column tiles of the output: R <= 16 * RT
__global__ __launch_bounds__(kThreads) void lowrank_kernel(LowRankGroup grp) {
  __shared__ float red[kWaves][ROWS][RT * 16];
  const LowRankArgs a = grp.p[__builtin_amdgcn_readfirstlane((int)blockIdx.y)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * ROWS;
  if (m0 >= lowrank_rows(a)) return;   // the other product has more rows

  const rsrc_t rl = make_rsrc(a.L + m0 * a.ldl, (a.M - m0) * a.ldl * 2);
  const rsrc_t rp = make_rsrc(a.P, a.R * a.ldp * 2);
  const uint32_t lvoff = (uint32_t)(lr * a.ldl * 2 + lg * 16);
  uint32_t pvoff[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = t * 16 + lr;
    pvoff[t] = j < a.R ? (uint32_t)(j * a.ldp * 2 + lg * 16) : kOutOfRange;
  }

  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t chunks = a.Kc / CHUNK;
  constexpr int U = UNROLL / RT;   // chunks of loads in flight per wave (registers: 4 * U * (1 + RT))
  for (int64_t q0 = wave; q0 < chunks; q0 += (int64_t)kWaves * U) {
    u32x4 xv[U], pv[U][RT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q0 + (int64_t)u * kWaves;
      const bool in = q < chunks;
      const int soff = (int)(q * CHUNK * 2);
      xv[u] = in ? __builtin_amdgcn_raw_buffer_load_b128(rl, lvoff, soff, 0) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < RT; ++t)
        pv[u][t] = in ? __builtin_amdgcn_raw_buffer_load_b128(rp, pvoff[t], soff, 0) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < RT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[u]),
                                                        __builtin_bit_cast(bf16x8, pv[u][t]), acc[t], 0, 0, 0);
  }

  // acc[t][e] is row 4*lg + e, column 16*t + lr.
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * lg + e][16 * t + lr] = acc[t][e];
  __syncthreads();

  for (int idx = threadIdx.x; idx < ROWS * RT * 16; idx += kThreads) {
    const int row = idx / (RT * 16), j = idx % (RT * 16);
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[w][row][j];
    const int64_t m = m0 + row;
    const uint16_t b = (j < a.R) ? f32_to_bf16(v * a.scale) : (uint16_t)0;
    if (m < a.M) {
      if (a.out_f32 && j < a.R) a.out_f32[m * a.R + j] = v;
      if (a.out_b && j < a.ldb) a.out_b[m * a.ldb + j] = b;
    }
    if (a.out_t && j < a.ldt_rows && m < a.Mp) a.out_t[(int64_t)j * a.Mp + m] = b;
  }
  // Columns of out_b between RT*16 and ldb (only when ldb > RT*16) are zero.
  if (a.out_b && a.ldb > RT * 16) {
    for (int idx = threadIdx.x; idx < ROWS * (a.ldb - RT * 16); idx += kThreads) {
      const int row = idx / (int)(a.ldb - RT * 16), j = RT * 16 + idx % (int)(a.ldb - RT * 16);
      const int64_t m = m0 + row;
      if (m < a.M) a.out_b[m * a.ldb + j] = 0;
    }
  }
  if (a.out_t && a.ldt_rows > RT * 16) {
    for (int idx = threadIdx.x; idx < ROWS * (a.ldt_rows - RT * 16); idx += kThreads) {
      const int row = idx % ROWS, j = RT * 16 + idx / ROWS;
      const int64_t m = m0 + row;
      if (m < a.Mp) a.out_t[(int64_t)j * a.Mp + m] = 0;
    }
  }
}

}  // namespace

hipError_t launch_lowrank_n(const LowRankArgs *a, int n, hipStream_t st) {
  if (n < 1 || n > QN_MAX_GROUP) return hipErrorInvalidValue;
  LowRankGroup grp{};
  int64_t rows = 0, R = 0;
  for (int i = 0; i < n; ++i) {
    grp.p[i] = a[i];
    rows = std::max(rows, lowrank_rows(a[i]));
    R = std::max(R, a[i].R);
  }
  const dim3 grid((unsigned)((rows + ROWS - 1) / ROWS), (unsigned)n);
  TraceScope tr(QN_TRACE_LOWRANK, st);
  if (R <= 16) hipLaunchKernelGGL(lowrank_kernel<1>, grid, dim3(kThreads), 0, st, grp);
  else if (R <= 32) hipLaunchKernelGGL(lowrank_kernel<2>, grid, dim3(kThreads), 0, st, grp);
  else hipLaunchKernelGGL(lowrank_kernel<4>, grid, dim3(kThreads), 0, st, grp);
  return hipGetLastError();
}

hipError_t launch_lowrank2(const LowRankArgs &a, const LowRankArgs *b, hipStream_t st) {
  const LowRankArgs two[2] = {a, b ? *b : a};
  return launch_lowrank_n(two, b ? 2 : 1, st);
}

hipError_t launch_lowrank(const LowRankArgs &a, hipStream_t st) { return launch_lowrank2(a, nullptr, st); }

}  // namespace qn

// ----------------------------------------------------------------------------
// Column-streaming reduction over rows: out[j][c] = sum_m Lt[j][m] * Q[m][c] for
// j < R (R <= 64), used for dA = dH^T X and dB^T = (s H)^T dY, where the
// contraction runs down the rows of the row-major activations.  Lt is [Rp, Mp]
// bf16, zero beyond R and M.
//
// A workgroup (4 waves) owns 128 columns (2 per lane) and a range of RB rows;
// each wave takes every fourth pair of rows.  Two rows of Q are paired per
// column with one byte permute and multiplied by the pair (Lt[j][m],
// Lt[j][m+1]) with v_dot2_f32_bf16, so Q is read exactly once.  The factor
// slice for the row range sits in LDS as [row pair][j] dwords (broadcast
// reads).  Per-split partial sums go to `part`; a second kernel adds the
// splits in order and rounds to bf16.  Like the low-rank product, one launch
// can carry two independent reductions over the same rows (blockIdx.z).
namespace qn {
namespace {

constexpr int CR_THREADS = 256;
constexpr int CR_COLS = 128;
constexpr int CR_RB = 128;        // rows per split
constexpr int CR_PAIRS = CR_RB / 2;

template <int R>
__global__ __launch_bounds__(CR_THREADS) void colred_kernel(ColRedArgs a0, ColRedArgs a1) {
  constexpr int RJ = R < 16 ? R : 16;            // rows of the output reduced per pass
  __shared__ uint32_t lt[CR_PAIRS * R];          // (Lt[j][2p], Lt[j][2p+1]) at [p][j]
  __shared__ float red[4][RJ][CR_COLS];
  const ColRedArgs &a = blockIdx.z ? a1 : a0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * CR_COLS;
  if (c0 >= a.Ncols) return;                     // the other reduction is wider
  const int split = blockIdx.y;
  const int64_t mb = (int64_t)split * CR_RB;

  // Activation loads first (all of this wave's row pairs), so their latency
  // overlaps the factor preload below.
  const rsrc_t rq = make_rsrc(a.Q + mb * a.ldq, (a.M - mb) * a.ldq * 2);
  const int64_t c = c0 + 2 * lane;
  const bool cin = c < a.Ncols;
  const uint32_t qoff = cin ? (uint32_t)(c * 2) : kOutOfRange;
  constexpr int U = CR_PAIRS / 4;
  uint32_t q[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = wave + 4 * u;
    const uint32_t r0 = (uint32_t)(2 * p) * (uint32_t)(a.ldq * 2);
    q[u][0] = cin ? __builtin_amdgcn_raw_buffer_load_b32(rq, qoff + r0, 0, 0) : 0u;
    q[u][1] = cin ? __builtin_amdgcn_raw_buffer_load_b32(rq, qoff + r0 + (uint32_t)(a.ldq * 2), 0, 0) : 0u;
  }

  // Factor slice: rows j < R, columns [mb, mb + RB) of Lt (always inside Mp).
  for (int idx = tid; idx < CR_PAIRS * R; idx += CR_THREADS) {
    const int j = idx / CR_PAIRS, p = idx % CR_PAIRS;
    const int64_t m = mb + 2 * p;
    uint32_t v = 0;
    if (j < a.R && m < a.Mp) v = *reinterpret_cast<const uint32_t *>(a.Lt + (int64_t)j * a.Mp + m);
    lt[p * R + j] = v;
  }
  __syncthreads();

  float acc0[R], acc1[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc0[j] = acc1[j] = 0.0f;
  {
    const int p0 = wave;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + 4 * u;
      // (Q[m][c], Q[m+1][c]) and (Q[m][c+1], Q[m+1][c+1])
      const uint32_t pc0 = __builtin_amdgcn_perm(q[u][1], q[u][0], 0x05040100u);
      const uint32_t pc1 = __builtin_amdgcn_perm(q[u][1], q[u][0], 0x07060302u);
      const uint32_t *lrow = &lt[p * R];
#pragma unroll
      for (int j4 = 0; j4 < R; j4 += 4) {
        const u32x4 l4 = *reinterpret_cast<const u32x4 *>(lrow + j4);
        const uint32_t lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc0[j4 + t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lv[t]), __builtin_bit_cast(bf16x2, pc0),
                                                         acc0[j4 + t], false);
          acc1[j4 + t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lv[t]), __builtin_bit_cast(bf16x2, pc1),
                                                         acc1[j4 + t], false);
        }
      }
    }
  }

  // Add the 4 waves' partials in a fixed order, RJ output rows per pass.
#pragma unroll
  for (int jb = 0; jb < R; jb += RJ) {
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      red[wave][j][2 * lane] = acc0[jb + j];
      red[wave][j][2 * lane + 1] = acc1[jb + j];
    }
    __syncthreads();
    for (int idx = tid; idx < RJ * CR_COLS; idx += CR_THREADS) {
      const int j = idx / CR_COLS, cc = idx % CR_COLS;
      const int64_t col = c0 + cc;
      if (jb + j < a.R && col < a.Ncols) {
        const float v = red[0][j][cc] + red[1][j][cc] + red[2][j][cc] + red[3][j][cc];
        a.part[((int64_t)split * a.R + jb + j) * a.Ncols + col] = v;
      }
    }
    __syncthreads();
  }
}

// out = bf16(sum over splits of part), as [R][Ncols] or transposed [Ncols][R].
// One thread per output element, columns fastest: the partial reads are
// coalesced; the splits are added in order.
__global__ __launch_bounds__(256) void colred_reduce_kernel(ColRedArgs a0, ColRedArgs a1, int splits) {
  const ColRedArgs &a = blockIdx.y ? a1 : a0;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.R * a.Ncols) return;
  const int64_t j = idx / a.Ncols, col = idx % a.Ncols;
  const int64_t stride = a.R * a.Ncols;
  const float *p = a.part + idx;
  float v = 0.0f;
  int s = 0;
  for (; s + 4 <= splits; s += 4) {
    const float x0 = p[(s + 0) * stride], x1 = p[(s + 1) * stride], x2 = p[(s + 2) * stride], x3 = p[(s + 3) * stride];
    v += x0;
    v += x1;
    v += x2;
    v += x3;
  }
  for (; s < splits; ++s) v += p[s * stride];
  a.out[a.transpose ? col * a.R + j : idx] = f32_to_bf16(v);
}

}  // namespace

int colred_splits(int64_t M) { return (int)((M + CR_RB - 1) / CR_RB); }

hipError_t launch_colred2(const ColRedArgs &a, const ColRedArgs *b, hipStream_t st, int trace_kind) {
  const int splits = colred_splits(a.M);
  const int64_t ncols = std::max(a.Ncols, b ? b->Ncols : 0);
  const int64_t R = std::max(a.R, b ? b->R : 0);
  const ColRedArgs &a1 = b ? *b : a;
  const dim3 grid((unsigned)((ncols + CR_COLS - 1) / CR_COLS), (unsigned)splits, b ? 2u : 1u);
  {
    TraceScope tr(trace_kind, st);
    if (R <= 8) hipLaunchKernelGGL(colred_kernel<8>, grid, dim3(CR_THREADS), 0, st, a, a1);
    else if (R <= 16) hipLaunchKernelGGL(colred_kernel<16>, grid, dim3(CR_THREADS), 0, st, a, a1);
    else if (R <= 32) hipLaunchKernelGGL(colred_kernel<32>, grid, dim3(CR_THREADS), 0, st, a, a1);
    else hipLaunchKernelGGL(colred_kernel<64>, grid, dim3(CR_THREADS), 0, st, a, a1);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t elems = std::max(a.R * a.Ncols, b ? b->R * b->Ncols : 0);
  hipLaunchKernelGGL(colred_reduce_kernel, dim3((unsigned)((elems + 255) / 256), b ? 2u : 1u), dim3(256), 0, st, a,
                     a1, splits);
  return hipGetLastError();
}

hipError_t launch_colred(const ColRedArgs &a, hipStream_t st, int trace_kind) {
  return launch_colred2(a, nullptr, st, trace_kind);
}

}  // namespace qn
