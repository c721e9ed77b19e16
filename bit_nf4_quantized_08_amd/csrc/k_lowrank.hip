// Low-rank products of the adapter path on gfx950: C[M, R] = L[M, Kc] * P[R, Kc]^T
// with R <= 64.  Used for H = X A^T (forward and backward) and dH = dY B (with
// P = B^T).
//
// "LoRA vs QLoRA: Efficient Fine-Tuning Explained", "How LoRA Works": the
// adapter's two thin factors, B (d x r) and A (r x k), r small (8 to 64); the
// product through them is cheap next to the base weight, and this kernel
// streams the activations once at HBM rate.
//
// Work layout.  A workgroup of 4 waves owns 128 rows of L (32 per wave) and one
// range of the contraction; the ranges (lowrank_splits of them) give the GPU
// enough workgroups when M is small.  Per 64-deep step each wave loads its own
// 32 x 64 slab of L into registers with whole-line loads, LR_DEPTH steps ahead,
// and passes it through its own LDS region into the MFMA layout, while the
// R x 64 slab of the factor is loaded once for the workgroup, LR_DEPTH steps
// ahead as well, and staged in
// LDS (row pitch 144 bytes: sixteen consecutive rows read at one 16-byte
// column fall on 16 distinct 4-bank groups).  v_mfma_f32_32x32x16_bf16 takes
// both operands with the same permutation of the step's 64 contraction
// indices (lane half h, sub-step i: indices 32h + 8i .. 32h + 8i + 7), which
// leaves the sum unchanged.  The fp32 partial product of each range goes to a
// workspace; a second kernel adds the ranges in order and writes the requested
// outputs: fp32 unscaled, bf16 scaled (row-major, zero-padded to ldb
// columns), bf16 scaled and transposed (zero-padded to ldt_rows rows and Mp
// columns).  One launch carries up to QN_MAX_GROUP independent products
// (blockIdx.y selects one).

#include <algorithm>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0xFFFFFFF0LL;
  const int n = (int)(uint32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

constexpr int LR_THREADS = 256;   // 4 waves
constexpr int LR_BM = 128;        // rows of L per workgroup
constexpr int LR_CK = 64;         // contraction depth of one step
constexpr int LR_DEPTH = 4;       // steps of loads in flight
constexpr int LR_PITCH = 144;     // LDS bytes per factor row
constexpr int LR_TARGET_WGS = 256;
constexpr int LR_MAX_SPLITS = 16;
constexpr int LR_MIN_RANGE = 256; // contraction depth of the shortest range
constexpr int FIN_ROWS = 16;      // rows per workgroup of the finishing kernel

__host__ __device__ inline int64_t lowrank_rows(const LowRankArgs &a) {
  return a.out_t && a.Mp > a.M ? a.Mp : a.M;
}
__host__ __device__ inline int64_t align32(int64_t v) { return (v + 31) / 32 * 32; }

struct LowRankGroup {
  LowRankArgs p[QN_MAX_GROUP];
};

template <int RT>   // 32-column tiles of the factor: R <= 32 * RT
__global__ __launch_bounds__(LR_THREADS) void lowrank_part_kernel(LowRankGroup grp) {
  __shared__ __attribute__((aligned(16))) uint8_t ps[2][32 * RT * LR_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t xs[LR_THREADS / 64][32 * 128];   // each wave's L slab
  const LowRankArgs a = grp.p[__builtin_amdgcn_readfirstlane((int)blockIdx.y)];
  const int S = a.splits;
  const int64_t rb = blockIdx.x / S;
  const int s = (int)(blockIdx.x % S);
  const int64_t m0 = rb * LR_BM;
  if (m0 >= a.M) return;   // another product of the launch has more rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;

  const int64_t steps = a.Kc / LR_CK;
  const int64_t per = (steps + S - 1) / S;
  const int64_t c0 = std::min<int64_t>(steps, (int64_t)s * per), c1 = std::min<int64_t>(steps, c0 + per);

  // L: load i of a step brings rows 8i .. 8i + 7 of the wave's 32, eight lanes
  // per row reading its whole 128-byte line (rows past M read zeros); a wave
  // whose lanes each read a 16-byte piece of a different row would touch 32
  // lines per load and fetch each line four times.  The wave writes the slab
  // to its own LDS region, chunk k of row rho at slot k ^ ((rho >> 1) & 7), and
  // reads the MFMA fragments back: lane (lr, lh) reads row lr, chunk 4 lh + i in
  // sub-step i (16 consecutive lanes hit 16 distinct 4-bank groups).  Offsets
  // stay below 2^32: 128 rows of at most 2^24 elements.
  const rsrc_t rl = make_rsrc(a.L + m0 * a.ldl, (a.M - m0) * a.ldl * 2);
  uint32_t lvo[4], xw[4], xrd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rho = 8 * i + (lane >> 3), k = lane & 7;
    lvo[i] = (uint32_t)((32 * wave + rho) * a.ldl * 2 + 16 * k);
    xw[i] = (uint32_t)(rho * 128 + 16 * (k ^ ((rho >> 1) & 7)));
    xrd[i] = (uint32_t)(lr * 128 + 16 * ((4 * lh + i) ^ ((lr >> 1) & 7)));
  }
  uint8_t *xslab = xs[wave];
  // P: thread t moves 16-byte unit (t & 7) of rows t / 8 + 32 i, i < RT (rows
  // past R read zeros).
  const rsrc_t rp = make_rsrc(a.P, a.R * a.ldp * 2);
  uint32_t pvoff[RT], pls[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int j = tid / 8 + 32 * i, u = tid & 7;
    pvoff[i] = j < a.R ? (uint32_t)(j * a.ldp * 2 + 16 * u) : kOutOfRange;
    pls[i] = (uint32_t)(j * LR_PITCH + 16 * u);
  }

  u32x4 xr[LR_DEPTH][4];
  u32x4 pr[LR_DEPTH][RT];
  // Loads of step c (steps at or past c1 read zeros and move no data).
  auto load_step = [&](int slot, int64_t c) {
    const bool in = c < c1;
    const int soff = in ? (int)(c * LR_CK * 2) : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xr[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rl, in ? lvo[i] : kOutOfRange, soff, 0);
#pragma unroll
    for (int i = 0; i < RT; ++i)
      pr[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rp, in ? pvoff[i] : kOutOfRange, soff, 0);
  };
  auto stage = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < RT; ++i) *reinterpret_cast<u32x4 *>(&ps[buf][pls[i]]) = pr[slot][i];
  };

  f32x16 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  // The step loop runs a whole number of LR_DEPTH-step groups with no branch
  // inside a group (the padding steps multiply zeros), so that the loads of
  // the next LR_DEPTH - 1 steps stay in flight across the loop's back edge.
  // Step cb + d reads register slot d and LDS buffer d & 1 (LR_DEPTH is even).
  static_assert(LR_DEPTH % 2 == 0, "LDS buffer parity follows the slot");
  const int64_t n = c1 - c0;
  if (n > 0) {
    const int64_t np = (n + LR_DEPTH - 1) / LR_DEPTH * LR_DEPTH;
#pragma unroll
    for (int d = 0; d < LR_DEPTH; ++d) load_step(d, c0 + d);
    stage(0, 0);
    __syncthreads();
    for (int64_t cb = 0; cb < np; cb += LR_DEPTH) {
#pragma unroll
      for (int d = 0; d < LR_DEPTH; ++d) {
        const uint8_t *pb = ps[d & 1];
        // The wave's slab through its LDS region (its own rows only: LDS
        // operations of one wave complete in order, no barrier needed).
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4 *>(xslab + xw[i]) = xr[d][i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 xa = *reinterpret_cast<const bf16x8 *>(xslab + xrd[i]);
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            const u32x4 pf = *reinterpret_cast<const u32x4 *>(pb + (32 * t + lr) * LR_PITCH + 16 * (4 * lh + i));
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, __builtin_bit_cast(bf16x8, pf), acc[t], 0, 0, 0);
          }
        }
        load_step(d, c0 + cb + d + LR_DEPTH);
        stage((d + 1) % LR_DEPTH, (d + 1) & 1);
        __syncthreads();
      }
    }
  }

  // acc[t][e] is row 32 wave + 8 (e / 4) + 4 lh + e % 4, column 32 t + lr.
  const int64_t Rp = align32(a.R);
  float *part = a.part + (int64_t)s * a.M * Rp;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = 32 * t + lr;
    if (j >= Rp) break;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + 32 * wave + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (m < a.M) part[m * Rp + j] = acc[t][e];
    }
  }
}

// Adds the ranges' partial products in range order and writes the outputs.  A
// workgroup owns FIN_ROWS rows x RW columns (RW: the launch's largest rank
// rounded up to 16, 32 or 64); thread t owns elements t, t + 256, ... of that
// tile, and every range's partial of all of them is loaded before the first
// sum, so that the workgroup waits for memory once.  The sums are staged in
// LDS so that both the row-major and the transposed outputs are written along
// their rows.
template <int RW>
__global__ __launch_bounds__(256) void lowrank_finish_kernel(LowRankGroup grp) {
  constexpr int E = FIN_ROWS * RW / 256;   // elements per thread
  static_assert(E >= 1 && FIN_ROWS * RW == 256 * E && RW <= 64, "finish tile");
  __shared__ float tile[FIN_ROWS][65];
  const LowRankArgs a = grp.p[__builtin_amdgcn_readfirstlane((int)blockIdx.y)];
  const int64_t m0 = (int64_t)blockIdx.x * FIN_ROWS;
  if (m0 >= lowrank_rows(a)) return;
  const int tid = threadIdx.x;
  const int64_t Rp = align32(a.R), plane = a.M * Rp;
  const int S = a.splits;
  // The loads carry no condition, so that they all issue before the first
  // wait: lanes outside the problem read the first element of each range, and
  // slots past the last range re-read the last one; both are discarded.
  float pv[E][LR_MAX_SPLITS];
  bool in[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = tid + 256 * i, r = e / RW, j = e % RW;
    const int64_t m = m0 + r;
    in[i] = m < a.M && j < a.R;
    const float *p = a.part + (in[i] ? m * Rp + j : 0);
#pragma unroll
    for (int s = 0; s < LR_MAX_SPLITS; ++s) pv[i][s] = p[(int64_t)min(s, S - 1) * plane];
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int e = tid + 256 * i, r = e / RW, j = e % RW;
    float v = 0.0f;
#pragma unroll
    for (int s = 0; s < LR_MAX_SPLITS; ++s)
      if (s < S) v += pv[i][s];
    tile[r][j] = in[i] ? v : 0.0f;
  }
  __syncthreads();
  for (int idx = tid; idx < FIN_ROWS * 64; idx += 256) {
    const int r = idx >> 6, jj = idx & 63;
    const int64_t m = m0 + r;
    if (m >= a.M) continue;
    const float v = tile[r][jj];
    if (a.out_f32 && jj < a.R) a.out_f32[m * a.R + jj] = v;
    if (a.out_b && jj < a.ldb) a.out_b[m * a.ldb + jj] = jj < a.R ? f32_to_bf16(v * a.scale) : (uint16_t)0;
  }
  if (a.out_t) {
    for (int idx = tid; idx < FIN_ROWS * 64; idx += 256) {
      const int jj = idx / FIN_ROWS, r = idx % FIN_ROWS;
      const int64_t m = m0 + r;
      if (jj < a.ldt_rows && m < a.Mp)
        a.out_t[(int64_t)jj * a.Mp + m] = (jj < a.R && m < a.M) ? f32_to_bf16(tile[r][jj] * a.scale) : (uint16_t)0;
    }
  }
}

}  // namespace

int lowrank_splits(int64_t M, int64_t Kc) {
  const int64_t rb = (M + LR_BM - 1) / LR_BM;
  const int64_t want = (LR_TARGET_WGS + rb - 1) / rb;
  const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(LR_MAX_SPLITS, Kc / LR_MIN_RANGE));
  return (int)std::max<int64_t>(1, std::min(want, cap));
}

size_t lowrank_part_bytes(int64_t M, int64_t Kc, int64_t R) {
  return (size_t)lowrank_splits(M, Kc) * (size_t)M * (size_t)align32(R) * sizeof(float);
}

hipError_t launch_lowrank_n(const LowRankArgs *a, int n, hipStream_t st) {
  if (n < 1 || n > QN_MAX_GROUP) return hipErrorInvalidValue;
  LowRankGroup grp{};
  int64_t wgs = 0, fin = 0, R = 0;
  for (int i = 0; i < n; ++i) {
    grp.p[i] = a[i];
    grp.p[i].splits = lowrank_splits(a[i].M, a[i].Kc);
    wgs = std::max<int64_t>(wgs, (a[i].M + LR_BM - 1) / LR_BM * grp.p[i].splits);
    fin = std::max<int64_t>(fin, (lowrank_rows(a[i]) + FIN_ROWS - 1) / FIN_ROWS);
    R = std::max(R, a[i].R);
  }
  {
    TraceScope tr(QN_TRACE_LOWRANK, st);
    const dim3 grid((unsigned)wgs, (unsigned)n);
    if (R <= 32) hipLaunchKernelGGL(lowrank_part_kernel<1>, grid, dim3(LR_THREADS), 0, st, grp);
    else hipLaunchKernelGGL(lowrank_part_kernel<2>, grid, dim3(LR_THREADS), 0, st, grp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid((unsigned)fin, (unsigned)n);
  if (R <= 16) hipLaunchKernelGGL(lowrank_finish_kernel<16>, fgrid, dim3(256), 0, st, grp);
  else if (R <= 32) hipLaunchKernelGGL(lowrank_finish_kernel<32>, fgrid, dim3(256), 0, st, grp);
  else hipLaunchKernelGGL(lowrank_finish_kernel<64>, fgrid, dim3(256), 0, st, grp);
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

  // The factor slice (rows j < R, columns [mb, mb + RB) of Lt) is loaded
  // first and the activations (all of this wave's row pairs) after it, so
  // that waiting for the slice leaves the activation loads in flight.  The
  // slice loads have no condition (an index outside Lt is clamped into it and
  // its value replaced by zero), so they all issue before the first wait.
  constexpr int LTN = CR_PAIRS * R / CR_THREADS;
  static_assert(LTN * CR_THREADS == CR_PAIRS * R, "factor slice thread map");
  uint32_t ltv[LTN];
#pragma unroll
  for (int i = 0; i < LTN; ++i) {
    const int idx = tid + i * CR_THREADS, j = idx / CR_PAIRS, p = idx % CR_PAIRS;
    const int64_t m = mb + 2 * p;
    const int64_t jc = j < a.R ? j : a.R - 1, mc = m < a.Mp ? m : a.Mp - 2;
    ltv[i] = *reinterpret_cast<const uint32_t *>(a.Lt + jc * a.Mp + mc);
  }
  const rsrc_t rq = make_rsrc(a.Q + mb * a.ldq, (a.M - mb) * a.ldq * 2);
  const int64_t c = c0 + 2 * lane;
  const bool cin = c < a.Ncols;
  constexpr int U = CR_PAIRS / 4;
  uint32_t q[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // Columns past the end read zero through the out-of-range offset (the
    // offset is selected, not the load, so that no load sits in a branch).
    const int p = wave + 4 * u;
    const uint32_t r0 = (uint32_t)(2 * p) * (uint32_t)(a.ldq * 2) + (uint32_t)(c * 2);
    q[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rq, cin ? r0 : kOutOfRange, 0, 0);
    q[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rq, cin ? r0 + (uint32_t)(a.ldq * 2) : kOutOfRange, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < LTN; ++i) {
    const int idx = tid + i * CR_THREADS, j = idx / CR_PAIRS, p = idx % CR_PAIRS;
    lt[p * R + j] = (j < a.R && mb + 2 * p < a.Mp) ? ltv[i] : 0u;
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
  // Batches of splits loaded with no condition (slots past the last split
  // re-read it and are discarded), so that each batch waits for memory once.
  constexpr int BATCH = 16;
  float v = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += BATCH) {
    float x[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) x[q] = p[(int64_t)min(s0 + q, splits - 1) * stride];
#pragma unroll
    for (int q = 0; q < BATCH; ++q)
      if (s0 + q < splits) v += x[q];
  }
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
