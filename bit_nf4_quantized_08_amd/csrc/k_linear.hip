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
// Kernels in this file:
//   gemm_kernel     bf16 MFMA (v_mfma_f32_32x32x16_bf16) tile GEMM.  The right
//                   operand is NF4 codes dequantised into LDS (row-major [N,K]
//                   for the forward, or read transposed for dX), or a bf16
//                   matrix.  Extra contraction steps after the main K-loop add
//                   the rank-r adapter term with the same MFMA accumulators.
//   skinny_kernel   C[M, R<=64] = L[M, Kc] * P[R, Kc]^T with split-K partials:
//                   H = X A^T, dH = dY B.  Streams L once from HBM.
//   gemv_kernel     decode path (M <= 8): streams codes at HBM rate, expands
//                   byte pairs through an LDS table and accumulates with
//                   v_dot2_f32_bf16; per-block scale applied to partial sums.
//   small kernels   split reductions, transposes, epilogues.

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;        // contraction step: one NF4 block along K
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row: 16 B of padding keeps ds_read_b128 conflict-free

__device__ __forceinline__ float scale_of(const ScaleSrc &sc, int64_t b) {
  if (sc.absmax_q) return (float)sc.absmax_q[b] * sc.scale2[b / QN_GROUP];
  return sc.absmax[b];
}

// Byte -> (row of low nibble, row of high nibble) as fp32, in LDS.
__device__ __forceinline__ void build_pair_table(float2 *pair, const Code16 &cb) {
  for (int v = threadIdx.x; v < 256; v += blockDim.x) pair[v] = make_float2(cb.v[v & 15], cb.v[v >> 4]);
}

// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8 XCDs
// (hardware id h lands on XCD h % 8).  Give each XCD a contiguous range of
// logical tiles, and order logical tiles in groups of GM row-tiles so that the
// tiles an XCD runs together share operand rows/columns in its L2.
__device__ __forceinline__ void tile_coords(int h, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int T = tiles_m * tiles_n;
  int L = h;
  if ((T & 7) == 0) L = (h & 7) * (T >> 3) + (h >> 3);
  constexpr int GM = 8;
  const int group_size = GM * tiles_n;
  const int g = L / group_size;
  const int first_m = g * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in = L - g * group_size;
  tm = first_m + in % gm;
  tn = in / gm;
}

// ================================================================ main GEMM
enum RKind { R_NF4_NK = 0, R_NF4_KN = 1, R_BF16_KN = 2 };
enum EKind { E_NONE = 0, E_NK = 1, E_KN = 2 };

struct GemmArgs {
  const uint16_t *L;   // bf16 [Mrows, Kc] row-major, leading dim ldl
  int64_t ldl;
  int64_t Mrows;       // valid rows of L and of the output
  int64_t Nout;        // output columns (multiple of 64)
  int64_t Kc;          // contraction length (multiple of 64)
  int64_t Kvalid;      // rows k >= Kvalid of a bf16 KN right operand read as zero
  const uint8_t *codes;  // NF4 right operand
  ScaleSrc sc;
  const uint16_t *P;   // bf16 right operand, KN: P[k*ldp + n]
  int64_t ldp;
  const uint16_t *L2;  // adapter term: L2[m*ldl2 + j], j < r2
  int64_t ldl2;
  const uint16_t *R2;  // NK: R2[n*ldr2 + j]; KN: R2[j*ldr2 + n]
  int64_t ldr2;
  int64_t r2;
  uint16_t *out_bf16;  // [Mrows, Nout] (ld = ldo)
  float *out_f32;      // split partials: out_f32[split*split_stride + m*ldo + n]
  int64_t ldo;
  int64_t split_stride;
  int64_t steps_per_split;
  int tiles_m, tiles_n;
};

template <int BM, int BN, int WAVES_M, int RK, int EK, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs a, Code16 cb) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  // L tile staging: BM rows x 64 bf16 = BM*8 chunks of 16 B.
  constexpr int L_CHUNKS = BM * 8 / kThreads;
  static_assert(L_CHUNKS >= 1 || BM == 32, "tile rows");

  __shared__ __attribute__((aligned(16))) uint16_t Ls[BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Rs[BN * LDS_LD];
  __shared__ float2 pair[256];

  if constexpr (RK == R_NF4_NK || RK == R_NF4_KN) build_pair_table(pair, cb);

  int tm, tn;
  tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int split = blockIdx.y;
  const int64_t steps_main_total = a.Kc / BK;
  const int64_t s_begin = (int64_t)split * a.steps_per_split;
  const int64_t s_end = min(steps_main_total, s_begin + a.steps_per_split);
  const int64_t steps_main = max((int64_t)0, s_end - s_begin);
  const int64_t steps_epi = (EK != E_NONE && split == 0) ? (a.r2 + BK - 1) / BK : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // ---- register staging for one main step
  constexpr int LC = (BM * 8 + kThreads - 1) / kThreads;
  u32x4 lreg[LC];
  // Right operand staging.
  constexpr int NK_CHUNKS = (BN * 2 + kThreads - 1) / kThreads;  // 16-B code chunks (NF4_NK)
  constexpr int KN_UNITS = (16 * (BN / 8) + kThreads - 1) / kThreads;  // 4x8 units (KN kinds)
  u32x4 rreg[(RK == R_NF4_NK) ? NK_CHUNKS : 1];
  float rscale[(RK == R_NF4_NK) ? NK_CHUNKS : 4 * KN_UNITS];
  uint32_t kreg[(RK == R_NF4_KN) ? 4 * KN_UNITS : 1];
  u32x4 preg[(RK == R_BF16_KN) ? 4 * KN_UNITS : 1];

  auto load_step = [&](int64_t step) {
    const int64_t k0 = step * BK;
#pragma unroll
    for (int c = 0; c < LC; ++c) {
      const int idx = tid + c * kThreads;
      if (idx < BM * 8) {
        const int row = idx >> 3, col = (idx & 7) * 8;
        const int64_t gm = m0 + row;
        if (gm < a.Mrows) lreg[c] = *reinterpret_cast<const u32x4 *>(a.L + gm * a.ldl + k0 + col);
        else lreg[c] = u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (RK == R_NF4_NK) {
#pragma unroll
      for (int c = 0; c < NK_CHUNKS; ++c) {
        const int idx = tid + c * kThreads;
        if (idx < BN * 2) {
          const int row = idx >> 1, half = idx & 1;
          const int64_t gn = n0 + row;
          const int64_t e = gn * a.Kc + k0 + half * 32;
          if (gn < a.Nout) {
            rreg[c] = *reinterpret_cast<const u32x4 *>(a.codes + (e >> 1));
            rscale[c] = scale_of(a.sc, e >> 6);
          } else {
            rreg[c] = u32x4{0, 0, 0, 0};
            rscale[c] = 0.0f;
          }
        }
      }
    } else if constexpr (RK == R_NF4_KN) {
#pragma unroll
      for (int u = 0; u < KN_UNITS; ++u) {
        const int idx = tid + u * kThreads;
        if (idx < 16 * (BN / 8)) {
          const int kq = idx / (BN / 8), nc = idx % (BN / 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t gk = k0 + 4 * kq + i;
            const int64_t e = gk * a.Nout + n0 + 8 * nc;
            if (n0 + 8 * nc < a.Nout) {
              kreg[4 * u + i] = *reinterpret_cast<const uint32_t *>(a.codes + (e >> 1));
              rscale[4 * u + i] = scale_of(a.sc, e >> 6);
            } else {
              kreg[4 * u + i] = 0;
              rscale[4 * u + i] = 0.0f;
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < KN_UNITS; ++u) {
        const int idx = tid + u * kThreads;
        if (idx < 16 * (BN / 8)) {
          const int kq = idx / (BN / 8), nc = idx % (BN / 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t gk = k0 + 4 * kq + i;
            if (gk < a.Kvalid && n0 + 8 * nc < a.Nout)
              preg[4 * u + i] = *reinterpret_cast<const u32x4 *>(a.P + gk * a.ldp + n0 + 8 * nc);
            else
              preg[4 * u + i] = u32x4{0, 0, 0, 0};
          }
        }
      }
    }
  };

  auto store_step = [&]() {
#pragma unroll
    for (int c = 0; c < LC; ++c) {
      const int idx = tid + c * kThreads;
      if (idx < BM * 8) {
        const int row = idx >> 3, col = (idx & 7) * 8;
        *reinterpret_cast<u32x4 *>(&Ls[row * LDS_LD + col]) = lreg[c];
      }
    }
    if constexpr (RK == R_NF4_NK) {
#pragma unroll
      for (int c = 0; c < NK_CHUNKS; ++c) {
        const int idx = tid + c * kThreads;
        if (idx < BN * 2) {
          const int row = idx >> 1, half = idx & 1;
          const float A = rscale[c];
          const uint32_t w[4] = {rreg[c].x, rreg[c].y, rreg[c].z, rreg[c].w};
          uint32_t o[16];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float2 p = pair[(w[i] >> (8 * j)) & 0xFF];
              o[4 * i + j] = pack_bf16x2(p.x * A, p.y * A);
            }
          u32x4 *dst = reinterpret_cast<u32x4 *>(&Rs[row * LDS_LD + half * 32]);
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
        }
      }
    } else if constexpr (RK == R_NF4_KN) {
#pragma unroll
      for (int u = 0; u < KN_UNITS; ++u) {
        const int idx = tid + u * kThreads;
        if (idx < 16 * (BN / 8)) {
          const int kq = idx / (BN / 8), nc = idx % (BN / 8);
          float w[4][8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float A = rscale[4 * u + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float2 p = pair[(kreg[4 * u + i] >> (8 * j)) & 0xFF];
              w[i][2 * j] = p.x * A;
              w[i][2 * j + 1] = p.y * A;
            }
          }
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const u32x2 v = {pack_bf16x2(w[0][n], w[1][n]), pack_bf16x2(w[2][n], w[3][n])};
            *reinterpret_cast<u32x2 *>(&Rs[(8 * nc + n) * LDS_LD + 4 * kq]) = v;
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < KN_UNITS; ++u) {
        const int idx = tid + u * kThreads;
        if (idx < 16 * (BN / 8)) {
          const int kq = idx / (BN / 8), nc = idx % (BN / 8);
          const u32x4 *r = &preg[4 * u];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            // columns 2h, 2h+1 of the 8: low / high halves of word h of each row
            const uint32_t w0 = r[0][h], w1 = r[1][h], w2 = r[2][h], w3 = r[3][h];
            const u32x2 lo = {__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u)};
            const u32x2 hi = {__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u)};
            *reinterpret_cast<u32x2 *>(&Rs[(8 * nc + 2 * h) * LDS_LD + 4 * kq]) = lo;
            *reinterpret_cast<u32x2 *>(&Rs[(8 * nc + 2 * h + 1) * LDS_LD + 4 * kq]) = hi;
          }
        }
      }
    }
  };

  auto compute_step = [&]() {
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        av[i] = *reinterpret_cast<const bf16x8 *>(&Ls[(wm * WM + i * 32 + lr) * LDS_LD + kk * 16 + lh * 8]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = *reinterpret_cast<const bf16x8 *>(&Rs[(wn * WN + j * 32 + lr) * LDS_LD + kk * 16 + lh * 8]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  __syncthreads();  // pair table
  if (steps_main > 0) load_step(s_begin);
  for (int64_t s = 0; s < steps_main; ++s) {
    store_step();
    __syncthreads();
    if (s + 1 < steps_main) load_step(s_begin + s + 1);
    compute_step();
    __syncthreads();
  }

  // ---- adapter term: extra contraction steps over j < r2 (masked, zero-padded)
  for (int64_t s = 0; s < steps_epi; ++s) {
    const int64_t j0 = s * BK;
    for (int idx = tid; idx < BM * BK; idx += kThreads) {
      const int row = idx / BK, jj = idx % BK;
      const int64_t gm = m0 + row, gj = j0 + jj;
      uint16_t v = 0;
      if (gm < a.Mrows && gj < a.r2) v = a.L2[gm * a.ldl2 + gj];
      Ls[row * LDS_LD + jj] = v;
    }
    for (int idx = tid; idx < BN * BK; idx += kThreads) {
      int row, jj;
      if constexpr (EK == E_NK) { row = idx / BK; jj = idx % BK; }
      else { jj = idx / BN; row = idx % BN; }
      const int64_t gn = n0 + row, gj = j0 + jj;
      uint16_t v = 0;
      if (gj < a.r2 && gn < a.Nout) v = (EK == E_NK) ? a.R2[gn * a.ldr2 + gj] : a.R2[gj * a.ldr2 + gn];
      Rs[row * LDS_LD + jj] = v;
    }
    __syncthreads();
    compute_step();
    __syncthreads();
  }

  // ---- store: lane holds column (lane & 31) of each 32x32 tile, rows
  // 8*(e/4) + 4*(lane/32) + (e%4) for accumulator element e.
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t gn = n0 + wn * WN + j * 32 + lr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t gm = m0 + wm * WM + i * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (gm < a.Mrows && gn < a.Nout) {
          if constexpr (OUT_F32) a.out_f32[(int64_t)split * a.split_stride + gm * a.ldo + gn] = acc[i][j][e];
          else a.out_bf16[gm * a.ldo + gn] = f32_to_bf16(acc[i][j][e]);
        }
      }
    }
}

// ================================================================ skinny GEMM
// C_part[split][m][j] = sum_{k in split} L[m][k] * P[j][k], j < R (R <= 64).
// Each wave owns 32 rows of L and loads them straight from global memory in the
// MFMA operand layout; P's slice lives in LDS.  Within a 64-wide step, lane half
// h covers k in [32h, 32h+32) so that each lane reads 64 contiguous bytes; the
// same permutation is applied to P, so the contraction is unchanged.
struct SkinnyArgs {
  const uint16_t *L;
  int64_t ldl, M, Kc;
  const uint16_t *P;  // [R, Kc] row-major, leading dim ldp
  int64_t ldp, R;
  float *part;        // [splits][M][64]
  int64_t steps_per_split;
};

template <int RT>  // 32-column tiles: 1 (R <= 32) or 2 (R <= 64)
__global__ __launch_bounds__(kThreads) void skinny_kernel(SkinnyArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ps[RT * 32 * LDS_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t m = (int64_t)blockIdx.x * 128 + wave * 32 + lr;
  const int split = blockIdx.y;
  const int64_t steps_total = a.Kc / BK;
  const int64_t s0 = (int64_t)split * a.steps_per_split;
  const int64_t s1 = min(steps_total, s0 + a.steps_per_split);
  f32x16 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  for (int64_t s = s0; s < s1; ++s) {
    const int64_t k0 = s * BK;
    // P slice -> LDS (RT*32 rows x 64), 16-B chunks, rows >= R zero.
    for (int idx = tid; idx < RT * 32 * 8; idx += kThreads) {
      const int row = idx >> 3, col = (idx & 7) * 8;
      u32x4 v = {0, 0, 0, 0};
      if (row < a.R) v = *reinterpret_cast<const u32x4 *>(a.P + row * a.ldp + k0 + col);
      *reinterpret_cast<u32x4 *>(&Ps[row * LDS_LD + col]) = v;
    }
    u32x4 lv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (m < a.M) lv[c] = *reinterpret_cast<const u32x4 *>(a.L + m * a.ldl + k0 + lh * 32 + c * 8);
      else lv[c] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, lv[c]);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&Ps[(t * 32 + lr) * LDS_LD + lh * 32 + c * 8]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // Store the partial: element e of tile t is row 8*(e/4)+4*lh+(e%4) of this
  // wave's 32 rows, column t*32 + lr.
  const int64_t mbase = (int64_t)blockIdx.x * 128 + wave * 32;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t gm = mbase + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (gm < a.M) a.part[((int64_t)split * a.M + gm) * 64 + t * 32 + lr] = acc[t][e];
    }
}

// Sum skinny partials; write any of: fp32 [M][R] (ld R), bf16 [M][ldb] (zero
// beyond R), bf16 transposed [ldt rows][M] (rows >= R zero), each times `scale`
// (the fp32 output unscaled when scale_f32 is false).
// out_t has Mp >= M columns; its columns m >= M are written as zero.
__global__ __launch_bounds__(kThreads) void skinny_reduce_kernel(const float *__restrict__ part, int splits,
                                                                 int64_t M, int64_t Mp, int64_t R, float scale,
                                                                 float *out_f32, bool scale_f32,
                                                                 uint16_t *out_b, int64_t ldb,
                                                                 uint16_t *out_t, int64_t ldt_rows) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // over Mp * 64
  if (idx >= Mp * 64) return;
  const int64_t m = idx / 64;
  const int j = (int)(idx % 64);
  float v = 0.0f;
  if (j < R && m < M)
    for (int s = 0; s < splits; ++s) v += part[((int64_t)s * M + m) * 64 + j];
  const uint16_t b = (j < R && m < M) ? f32_to_bf16(v * scale) : (uint16_t)0;
  if (out_t && j < ldt_rows) out_t[(int64_t)j * Mp + m] = b;
  if (m >= M) return;
  if (out_f32 && j < R) out_f32[m * R + j] = scale_f32 ? v * scale : v;
  if (out_b && j < ldb) out_b[m * ldb + j] = b;
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

// Sum split-K partials [splits][Mrows][Ncols] and store bf16 either as is
// ([Mvalid][Ncols]) or transposed ([Ncols][Mvalid]).
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float *__restrict__ part, int splits,
                                                                 int64_t Mvalid, int64_t Ncols,
                                                                 int64_t split_stride, bool transpose,
                                                                 uint16_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= Mvalid * Ncols) return;
  const int64_t m = idx / Ncols, n = idx % Ncols;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += part[(int64_t)s * split_stride + m * Ncols + n];
  const uint16_t b = f32_to_bf16(v);
  if (transpose) out[n * Mvalid + m] = b;
  else out[m * Ncols + n] = b;
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

int skinny_splits(int64_t M, int64_t Kc) {
  const int64_t tiles = cdiv(M, 128);
  const int64_t steps = Kc / BK;
  int64_t sp = std::max<int64_t>(1, (2LL * num_cus()) / tiles);
  sp = std::min<int64_t>(sp, steps);
  sp = std::min<int64_t>(sp, 64);
  return (int)sp;
}

hipError_t run_skinny(const uint16_t *L, int64_t ldl, int64_t M, int64_t Kc, const uint16_t *P, int64_t ldp,
                      int64_t R, float *part, int splits, hipStream_t st) {
  SkinnyArgs sa{L, ldl, M, Kc, P, ldp, R, part, cdiv(Kc / BK, splits)};
  dim3 grid((unsigned)cdiv(M, 128), (unsigned)splits);
  if (R <= 32) hipLaunchKernelGGL(skinny_kernel<1>, grid, dim3(kThreads), 0, st, sa);
  else hipLaunchKernelGGL(skinny_kernel<2>, grid, dim3(kThreads), 0, st, sa);
  return hipGetLastError();
}

template <int BM, int BN, int WAVES_M, int RK, int EK, bool OUT_F32>
hipError_t launch_gemm(GemmArgs ga, int splits, hipStream_t st, int trace_kind) {
  ga.tiles_m = (int)cdiv(ga.Mrows, BM);
  ga.tiles_n = (int)cdiv(ga.Nout, BN);
  dim3 grid((unsigned)(ga.tiles_m * ga.tiles_n), (unsigned)splits);
  TraceScope tr(trace_kind, st);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WAVES_M, RK, EK, OUT_F32>), grid, dim3(kThreads), 0, st, ga, code16());
  return hipGetLastError();
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
namespace {
int gemm_splits(int64_t tiles, int64_t steps) {
  int64_t sp = std::max<int64_t>(1, (2LL * num_cus()) / std::max<int64_t>(tiles, 1));
  return (int)std::min<int64_t>(sp, std::min<int64_t>(steps, 32));
}
}  // namespace

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

  // B^T [rp, N] (rows >= r zero) so that dH = dY (B^T)^T runs on the skinny kernel.
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
