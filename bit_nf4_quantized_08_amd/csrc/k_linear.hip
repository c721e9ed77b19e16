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
//                         applied to partial sums.  Its waves also compute
//                         the adapter's H partials.
//   gemv_epilogue_kernel  adds the split partials and the adapter term.
//   bwd_prep_kernel       B^T for the backward's dH = dY B, and (s H)^T from a
//                         given H.

#include <map>
#include <mutex>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;        // contraction step: one NF4 block along K

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;          // raw buffer, 32-bit dwords
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;   // a per-lane offset that always reads zero
constexpr int kNontemporal = 2;                 // cache policy of data read once

// Buffer resource over [base, base + bytes): loads beyond `bytes` (by the
// per-lane offset) return zero.  Built from the first lane's values so that it
// stays in scalar registers even where the compiler takes the base for
// divergent (it depends on the wave index).
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0xFFFFFFF0LL;
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(uint32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcFlags);
}

__device__ __forceinline__ int64_t cdiv_d(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Backward preparation in one launch: Bt[j][n] = B[n][j] for j < r and zero for
// r <= j < rp (B is [N, r]); when H is given, also sHt[j][m] = bf16(s H[m][j])
// for j < r, m < M, zero elsewhere in [rp, Mp] (H is [M, r] fp32).  Thread idx
// writes element idx of Bt, then of sHt: the writes are coalesced, the reads of
// the two small factors strided.
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const uint16_t *__restrict__ B, int64_t N, int64_t r,
                                                            int64_t rp, uint16_t *__restrict__ Bt,
                                                            const float *__restrict__ H, int64_t M, int64_t Mp,
                                                            float s, uint16_t *__restrict__ sHt) {
  int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx < rp * N) {
    const int64_t j = idx / N, n = idx % N;
    Bt[idx] = j < r ? B[n * r + j] : (uint16_t)0;
    return;
  }
  idx -= rp * N;
  if (!H || idx >= rp * Mp) return;
  const int64_t j = idx / Mp, m = idx % Mp;
  sHt[idx] = (j < r && m < M) ? f32_to_bf16(H[m * r + j] * s) : (uint16_t)0;
}

// ================================================================ GEMV (decode)
// y_part[split][m][n] = sum over the split's K-segment of x[m][k] * W_hat[n][k],
// the block scale applied to each 32-weight partial sum.  A wave owns one
// K-segment of KW 2048-wide chunks and holds its activations in registers for
// the whole kernel; lane l owns 32 consecutive k of each chunk (16 bytes of
// codes).  The wave then walks rows n = v, v + row_waves, ...: each row is
// one contiguous read of KW KB of codes (rows of neighbouring waves are
// neighbours in memory), and the next row is requested before the current one
// is multiplied.
// After its weight rows a wave computes the adapter's H partials for its
// K-segment (one adapter row j at a time, against the activations it already
// holds): h_part[split][m][j] = sum over the segment of x[m][k] * A[j][k].
// There are no separate H workgroups, so every workgroup slot serves rows.
// 2048-wide chunks per wave segment (KW): the activations of a segment take
// 16 * KW * MM registers per lane, at most 64 (128 for MM = 8, KW = 1), and a
// segment is no longer than the row needs.  Two chunks at most, so that three
// rows' registers fit beside them at three or more waves per SIMD.
int gemv_kw(int mm, int64_t chunks) {
  const int cap = mm <= 2 ? 2 : 1;
  int kw = 1;
  while (kw < cap && kw < chunks) kw *= 2;
  return kw;
}

struct GemvArgs {
  const uint16_t *X;  // [M, K]
  int64_t M, N, K;
  const uint8_t *codes;
  ScaleSrc sc;
  const uint16_t *A;  // [r, K]
  int64_t r;
  float *y_part;      // [splits][M][N]
  float *h_part;      // [splits][M][64]
  int64_t k_per_split;   // KW * 2048: the K-segment of one wave
  int splits;            // K-segments
  int64_t row_waves;     // waves per K-segment; wave v takes rows v, v + row_waves, ...
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over each group of G consecutive lanes (G = 8, 16, 32 or 64), returned
// in every lane of the group, with no LDS traffic: DPP within a row of 16
// lanes (quad swaps, then half-row and row mirrors, which pair lanes holding
// equal partial sums), then the rows' sums read out with readlane.  (A
// butterfly of lane shuffles costs one LDS round trip per step, and the
// decode kernel pays it once per weight row.)
template <int G>
__device__ __forceinline__ float group_sum(float t, int lane) {
  static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group size");
  t += dpp_f32<0xB1>(t);    // quad: lanes i ^ 1
  t += dpp_f32<0x4E>(t);    // quad: lanes i ^ 2
  t += dpp_f32<0x141>(t);   // half-row mirror: quad sums of the two quads of 8
  if constexpr (G >= 16) t += dpp_f32<0x140>(t);   // row mirror: the two halves of 16
  if constexpr (G == 32) {
    const float a = lane_f32(t, 0) + lane_f32(t, 16), b = lane_f32(t, 32) + lane_f32(t, 48);
    t = lane < 32 ? a : b;
  }
  if constexpr (G == 64) t = (lane_f32(t, 0) + lane_f32(t, 16)) + (lane_f32(t, 32) + lane_f32(t, 48));
  return t;
}

__device__ __forceinline__ float wave_sum(float v, int lane) { return group_sum<64>(v, lane); }

// Wave sums of MM values at once (MM a power of two <= 8): each exchange step
// halves the values a lane carries (MM - 1 shuffles), and one group sum over
// the remaining 64 / MM lanes finishes.  Returns, in every lane, the full sum
// of value m = lane >> (6 - log2(MM)).
template <int MM>
__device__ __forceinline__ float wave_sum_multi(float (&v)[MM], int lane) {
  int off = 32;
#pragma unroll
  for (int cnt = MM; cnt > 1; cnt >>= 1, off >>= 1) {
    // The choice between the two halves is made on the values' bits: a select
    // between two array elements would be folded into a lane-dependent index
    // and push the array out of registers.
    const uint32_t up = (lane & off) != 0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < cnt / 2; ++i) {
      const uint32_t lo = as_u32(v[i]), hi = as_u32(v[i + cnt / 2]);
      const float keep = as_f32((hi & up) | (lo & ~up));
      const float send = as_f32((lo & up) | (hi & ~up));
      v[i] = keep + __shfl_xor(send, off, 64);
    }
  }
  return group_sum<64 / MM>(v[0], lane);
}

// Several decode problems in one launch: workgroups [start[g], start[g+1])
// run problem g (its H blocks first, then its row blocks).
struct GemvGroup {
  GemvArgs p[QN_MAX_GROUP];
  int start[QN_MAX_GROUP + 1];
  int n;
};

template <int MM, bool DQ, int KW>
__device__ __forceinline__ void gemv_body(const GemvArgs &a, int block, const uint32_t *pairs);

template <int MM, bool DQ, int KW>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvGroup g, Code16 cb) {
  __shared__ uint32_t pairs[256];  // byte -> bf16(row lo) | bf16(row hi) << 16
  {
    const uint32_t v = threadIdx.x;
    pairs[v] = pack_bf16x2(cb.v[v & 15], cb.v[v >> 4]);
  }
  __syncthreads();
  int gi = 0;
#pragma unroll
  for (int i = 1; i < QN_MAX_GROUP; ++i) gi += (i < g.n && (int)blockIdx.x >= g.start[i]) ? 1 : 0;
  gi = __builtin_amdgcn_readfirstlane(gi);
  const GemvArgs a = g.p[gi];
  gemv_body<MM, DQ, KW>(a, (int)blockIdx.x - g.start[gi], pairs);
}

template <int MM, bool DQ, int KW>
__device__ __forceinline__ void gemv_body(const GemvArgs &a, int block, const uint32_t *pairs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  static_assert(KW * MM <= 4 || KW == 1, "activation registers");
  const int64_t v = (int64_t)block * (kThreads / 64) + wave;
  const int split = (int)(v % a.splits);
  const int64_t n_first = v / a.splits;
  if (n_first >= a.row_waves) return;
  const int64_t kb = (int64_t)split * a.k_per_split;
  const int64_t ke = min(a.K, kb + a.k_per_split);
  const int64_t bpr = a.K / QN_BLOCK;  // blocks per row
  static_assert(QN_BLOCK == 64 && QN_GROUP == 256, "shifts below");

  // Activations of the segment, zero past its end (rows m >= M read row M - 1
  // and are never stored).
  uint32_t x[KW][MM][16];
#pragma unroll
  for (int c = 0; c < KW; ++c) {
    const int64_t k = kb + c * 2048 + lane * 32;
    const bool in = k < ke;
    const int64_t ks = in ? k : kb;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const u32x4 *p = reinterpret_cast<const u32x4 *>(a.X + min((int64_t)m, a.M - 1) * a.K + ks);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 w = p[q];
        x[c][m][4 * q] = in ? w.x : 0u; x[c][m][4 * q + 1] = in ? w.y : 0u;
        x[c][m][4 * q + 2] = in ? w.z : 0u; x[c][m][4 * q + 3] = in ? w.w : 0u;
      }
    }
  }
  const rsrc_t rs2 = make_rsrc(a.sc.scale2, DQ ? cdiv_d(a.N * bpr, QN_GROUP) * 4 : 0);

  // One row's codes and raw block scales: the aligned dword holding each 8-bit
  // scale code plus its group step, or the fp32 scale's bits.  Buffer
  // resources over the row alone; a row n >= N gets empty ones, so that its
  // loads (the prefetch after the last row) read zeros without touching
  // memory, and so do lanes past the segment.
  struct Row {
    u32x4 cw[KW];
    uint32_t sa[KW];
    float sb[KW];
  };
  auto load_row = [&](Row &R, int64_t n) {
    const bool nin = n < a.N;
    const int64_t nn = nin ? n : 0;
    const int64_t b0 = nn * bpr;  // first block of the row
    const rsrc_t rc = make_rsrc(a.codes + nn * (a.K / 2), nin ? a.K / 2 : 0);
    const rsrc_t rs = DQ ? make_rsrc(a.sc.absmax_q + (b0 & ~3LL), nin ? ((b0 & 3) + bpr + 3) & ~3LL : 0)
                         : make_rsrc(a.sc.absmax + b0, nin ? bpr * 4 : 0);
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      const int64_t k = kb + c * 2048 + lane * 32;
      const bool in = k < ke;
      R.cw[c] = __builtin_amdgcn_raw_buffer_load_b128(rc, in ? (uint32_t)(k >> 1) : kOutOfRange, 0, kNontemporal);
      if constexpr (DQ) {
        const uint32_t off = (uint32_t)(b0 & 3) + (uint32_t)(k >> 6);
        R.sa[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, in ? off & ~3u : kOutOfRange, 0, 0);
        R.sb[c] = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
            rs2, in ? (uint32_t)((uint64_t)(b0 + (k >> 6)) >> 8) * 4 : kOutOfRange, 0, 0));
      } else {
        R.sa[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, in ? (uint32_t)(k >> 6) * 4 : kOutOfRange, 0, 0);
        R.sb[c] = 1.0f;
      }
    }
  };

  // Multiply row n (its loads already issued into R) and store its sums.
  // The scheduling fences keep one chunk's table lookups live at a time.
  auto row_dot = [&](Row &R, int64_t n) {
    float acc[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[m] = 0.0f;
    const uint32_t b03 = (uint32_t)((n * bpr) & 3);
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" : "+v"(R.sa[c]), "+v"(R.sb[c]));  // the scale is formed here, not earlier
      const uint32_t w[4] = {R.cw[c].x, R.cw[c].y, R.cw[c].z, R.cw[c].w};
      const uint32_t sh = 8 * ((b03 + (uint32_t)((kb + c * 2048 + lane * 32) >> 6)) & 3u);
      const float A = DQ ? (float)((R.sa[c] >> sh) & 0xFFu) * R.sb[c] : as_f32(R.sa[c]);
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
                                                   __builtin_bit_cast(bf16x2, x[c][m][4 * q + b]), p[m], false);
        }
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        acc[m] = __builtin_fmaf(A, p[m], acc[m]);
        asm volatile("" : "+v"(acc[m]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kLog2MM = MM == 1 ? 0 : (MM == 2 ? 1 : (MM == 4 ? 2 : 3));
    const float t = wave_sum_multi<MM>(acc, lane);
    const int m = lane >> (6 - kLog2MM);
    if ((lane & ((64 >> kLog2MM) - 1)) == 0 && m < a.M) a.y_part[((int64_t)split * a.M + m) * a.N + n] = t;
  };

  // Rows in threes with three register sets (no copies between them): two
  // rows' loads stay in flight while the third is multiplied.
  const int64_t rows = cdiv_d(a.N - n_first, a.row_waves);
  const int64_t rw = a.row_waves;
  Row r0, r1, r2;
  load_row(r0, n_first);
  load_row(r1, n_first + rw);
  int64_t n = n_first;
  int64_t t = 0;
  for (; t + 3 <= rows; t += 3) {
    __builtin_amdgcn_sched_barrier(0);
    load_row(r2, n + 2 * rw);
    row_dot(r0, n);
    n += rw;
    __builtin_amdgcn_sched_barrier(0);
    load_row(r0, n + 2 * rw);
    row_dot(r1, n);
    n += rw;
    __builtin_amdgcn_sched_barrier(0);
    load_row(r1, n + 2 * rw);
    row_dot(r2, n);
    n += rw;
  }
  if (t < rows) row_dot(r0, n);
  if (t + 1 < rows) row_dot(r1, n + rw);

  // The adapter's H partials for this wave's K-segment, h_part[split][m][j] =
  // sum over the segment of x[m][k] A[j][k], with the activations already in
  // registers (zero past the segment's end).  Adapter row j goes to the wave
  // with n_first = (N mod W + j) mod W (W = row_waves), so the first adapter
  // rows go to the waves with one weight row fewer.  The loads of A's row
  // carry no condition: past the segment's end (or of A) they re-read the
  // segment's first chunk, and the zero activations cancel them.
  const int64_t W = a.row_waves;
  int64_t j = n_first - a.N % W;
  if (j < 0) j += W;
  for (; j < a.r; j += W) {
    float hm[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) hm[m] = 0.0f;
    u32x4 av[KW][4];
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      const int64_t k = kb + c * 2048 + lane * 32;
      const u32x4 *pa = reinterpret_cast<const u32x4 *>(a.A + j * a.K + (k < ke ? k : kb + lane * 32));
#pragma unroll
      for (int q = 0; q < 4; ++q) av[c][q] = pa[q];
    }
#pragma unroll
    for (int c = 0; c < KW; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t aw[4] = {av[c][q].x, av[c][q].y, av[c][q].z, av[c][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int m = 0; m < MM; ++m)
            hm[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[e]),
                                                    __builtin_bit_cast(bf16x2, x[c][m][4 * q + e]), hm[m], false);
      }
    constexpr int kLog2MM = MM == 1 ? 0 : (MM == 2 ? 1 : (MM == 4 ? 2 : 3));
    float hs[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) hs[m] = hm[m];
    const float t = wave_sum_multi<MM>(hs, lane);
    const int m = lane >> (6 - kLog2MM);
    if ((lane & ((64 >> kLog2MM) - 1)) == 0 && m < a.M) a.h_part[((int64_t)split * a.M + m) * 64 + j] = t;
  }
}

// y[m][n] = sum_s y_part[s][m][n] + s_lora * sum_j H[m][j] * B[n][j], H summed
// from its partials; rounded to bf16.  Optionally writes H (fp32, unscaled).
// A workgroup covers EPI_ROWS rows n.  For the adapter term eight lanes share
// a row of B, each reading 8 consecutive entries (one 16-byte load when r is a
// multiple of 8), so that a wave reads 8 whole rows of B per instruction; the
// eight partial sums are added with lane shuffles.
constexpr int EPI_ROWS = kThreads / 8;

struct EpiArgs {
  const float *y_part;
  int splits;
  const float *h_part;
  int hsplits;
  int64_t M, N, r;
  const uint16_t *B;
  float s_lora;
  uint16_t *Y;
  float *H_out;
};
struct EpiGroup {
  EpiArgs p[QN_MAX_GROUP];
  int start[QN_MAX_GROUP + 1];   // N / EPI_ROWS workgroups per problem
  int n;
};

__global__ __launch_bounds__(kThreads) void gemv_epilogue_kernel(EpiGroup g) {
  __shared__ float Hs[8 * 64];          // H[m][j], zero for j >= r
  __shared__ float Ls[8 * EPI_ROWS];    // sum_j H[m][j] B[n][j] for the workgroup's rows
  int gi = 0;
#pragma unroll
  for (int i = 1; i < QN_MAX_GROUP; ++i) gi += (i < g.n && (int)blockIdx.x >= g.start[i]) ? 1 : 0;
  gi = __builtin_amdgcn_readfirstlane(gi);
  const EpiArgs ea = g.p[gi];
  const float *__restrict__ y_part = ea.y_part;
  const int splits = ea.splits;
  const float *__restrict__ h_part = ea.h_part;
  const int hsplits = ea.hsplits;
  const int64_t M = ea.M, N = ea.N, r = ea.r;
  const uint16_t *__restrict__ B = ea.B;
  const float s_lora = ea.s_lora;
  uint16_t *__restrict__ Y = ea.Y;
  float *H_out = ea.H_out;
  const int eblock = (int)blockIdx.x - g.start[gi];
  const int64_t n0 = (int64_t)eblock * EPI_ROWS;
  const int t = threadIdx.x, row = t >> 3, j0 = 8 * (t & 7);
  const int64_t n = n0 + row;  // N % EPI_ROWS == 0
  // This thread's slice of B's row n first, so that its load overlaps those
  // of the partial sums below.  The load has no condition: a thread without
  // a 16-byte slice (r not a multiple of 8, or j0 >= r) reads B's first 16
  // bytes (B is 16-byte aligned and holds at least EPI_ROWS rows) and
  // discards them.
  const bool b16 = r % 8 == 0, bin = b16 && j0 < r;
  const u32x4 bw = *reinterpret_cast<const u32x4 *>(B + (bin ? n * r + j0 : 0));
  // Thread t sums output (t / EPI_ROWS, n0 + t % EPI_ROWS) over the K-segments
  // (8 EPI_ROWS == kThreads: at most one output each) and H entries t and
  // t + kThreads over the H ranges, in range order.  The loads of a batch of
  // ranges carry no condition (threads without an element read the first
  // element, slots past the last range re-read the last one; both are
  // discarded), so that each batch waits for memory once.
  static_assert(8 * EPI_ROWS == kThreads && 8 * 64 <= 2 * kThreads, "epilogue thread map");
  const bool yo = t < M * EPI_ROWS;
  const float *yp = y_part + (yo ? (int64_t)(t / EPI_ROWS) * N + n0 + t % EPI_ROWS : 0);
  const int64_t ys = M * N, hs = M * 64;
  bool ho[2];
  const float *hp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = t + u * kThreads;
    ho[u] = idx < M * 64 && idx % 64 < r;
    hp[u] = h_part + (ho[u] ? idx : 0);
  }
  float ysum = 0.0f, hsum[2] = {0.0f, 0.0f};
  constexpr int BATCH = 8;
  const int nr = max(splits, hsplits);
  for (int s0 = 0; s0 < nr; s0 += BATCH) {
    float yv[BATCH], hv[2][BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      yv[q] = yp[(int64_t)min(s0 + q, splits - 1) * ys];
#pragma unroll
      for (int u = 0; u < 2; ++u) hv[u][q] = hp[u][(int64_t)min(s0 + q, hsplits - 1) * hs];
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (s0 + q < splits) ysum += yv[q];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (s0 + q < hsplits) hsum[u] += hv[u][q];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = t + u * kThreads;
    if (idx < 8 * 64) {
      const float v = ho[u] ? hsum[u] : 0.0f;
      Hs[idx] = v;
      if (H_out && eblock == 0 && ho[u]) H_out[(idx / 64) * r + idx % 64] = v;
    }
  }
  float b[8];
  if (b16) {
    const uint32_t w[4] = {bin ? bw.x : 0u, bin ? bw.y : 0u, bin ? bw.z : 0u, bin ? bw.w : 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) { b[2 * q] = bf16_lo(w[q]); b[2 * q + 1] = bf16_hi(w[q]); }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) b[q] = j0 + q < r ? bf16_to_f32(B[n * r + j0 + q]) : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m >= M) break;
    float l = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) l = __builtin_fmaf(Hs[m * 64 + j0 + q], b[q], l);
    l += __shfl_xor(l, 1, 64);
    l += __shfl_xor(l, 2, 64);
    l += __shfl_xor(l, 4, 64);
    if (j0 == 0) Ls[m * EPI_ROWS + row] = l;
  }
  __syncthreads();
  if (yo) Y[(int64_t)(t / EPI_ROWS) * N + n0 + t % EPI_ROWS] = f32_to_bf16(__builtin_fmaf(s_lora, Ls[t], ysum));
}

// ================================================================ host side
int num_cus() { return device_cus(); }

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

struct GemvPlan {
  int splits;          // K-segments of gemv_kw(mm) chunks
  int64_t kps;         // K per segment
};

int gemv_mm(int64_t M) { return M == 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8)); }

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K) {
  GemvPlan p;
  const int64_t chunks = cdiv(K, 2048);
  const int64_t kw = gemv_kw(gemv_mm(M), chunks);
  p.kps = kw * 2048;
  p.splits = (int)cdiv(chunks, kw);
  return p;
}

// The decode kernel instance for M rows of activations and kw chunks per
// segment.
template <bool DQ>
const void *gemv_fn(int64_t M, int64_t kw) {
  switch (gemv_mm(M)) {
    case 1:
      return kw == 2 ? reinterpret_cast<const void *>(&gemv_kernel<1, DQ, 2>)
                     : reinterpret_cast<const void *>(&gemv_kernel<1, DQ, 1>);
    case 2:
      return kw == 2 ? reinterpret_cast<const void *>(&gemv_kernel<2, DQ, 2>)
                     : reinterpret_cast<const void *>(&gemv_kernel<2, DQ, 1>);
    case 4: return reinterpret_cast<const void *>(&gemv_kernel<4, DQ, 1>);
    default: return reinterpret_cast<const void *>(&gemv_kernel<8, DQ, 1>);
  }
}

// Workgroups of an instance that fit on one CU at once (cached per instance).
int gemv_resident(const void *fn) {
  static std::mutex mu;
  static std::map<const void *, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(fn);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, 0) != hipSuccess || nb < 1) nb = 1;
  cache[fn] = nb;
  return nb;
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
    const GemvPlan p = gemv_plan(M, N, K);
    c.take<float>((int64_t)p.splits * M * N);
    c.take<float>((int64_t)p.splits * M * 64);
  } else {
    c.take<uint16_t>(M * align_up(r, 8));
    c.take<char>((int64_t)lowrank_part_bytes(M, K, r));
  }
  return c.off;
}

// Arguments of the forward's MFMA path: the low-rank product H = X A^T
// (written unscaled to H_out, and as bf16(s H) to the workspace) and the tile
// GEMM that takes bf16(s H) B^T as its extra contraction step.
static void fwd_mfma_args(const FwdArgs &a, LowRankArgs &la, QGemmArgs &g) {
  Carve c(a.ws);
  const int64_t rp = align_up(a.r, 8);
  uint16_t *sH = c.take<uint16_t>(a.M * rp);
  float *part = reinterpret_cast<float *>(c.take<char>((int64_t)lowrank_part_bytes(a.M, a.K, a.r)));
  la = LowRankArgs{};
  la.L = a.X; la.ldl = a.K; la.M = a.M; la.Kc = a.K;
  la.P = a.A; la.ldp = a.K; la.R = a.r; la.scale = a.s;
  la.out_f32 = a.H_out; la.out_b = sH; la.ldb = rp; la.out_t = nullptr; la.Mp = a.M; la.part = part;
  g = QGemmArgs{};
  g.L = a.X; g.ldl = a.K; g.M = a.M; g.Nout = a.N; g.Kc = a.K;
  g.codes = a.codes; g.absmax = a.sc.absmax; g.absmax_q = a.sc.absmax_q; g.scale2 = a.sc.scale2;
  g.qtype = a.sc.qtype;
  g.L2 = sH; g.ldl2 = rp; g.R2 = a.B; g.ldr2 = a.r; g.r = a.r;
  g.out = a.Y; g.ldo = a.N;
}

// Launch arguments of one decode-path problem (its workspace carved from a.ws).
struct DecodePlan {
  const void *fn;      // kernel instance (rows of X, scale source, chunks per segment)
  GemvArgs ga;
  EpiArgs ea;
  int blocks;          // H blocks + row blocks
  int qtype;
};

static DecodePlan decode_plan(const FwdArgs &a) {
  Carve c(a.ws);
  DecodePlan d;
  GemvPlan p = gemv_plan(a.M, a.N, a.K);
  const int64_t kw = p.kps / 2048;
  d.fn = a.sc.absmax_q ? gemv_fn<true>(a.M, kw) : gemv_fn<false>(a.M, kw);
  float *y_part = c.take<float>((int64_t)p.splits * a.M * a.N);
  float *h_part = c.take<float>((int64_t)p.splits * a.M * 64);
  d.ga = GemvArgs{a.X, a.M, a.N, a.K, a.codes, a.sc, a.A, a.r, y_part, h_part, p.kps, p.splits, 0};
  d.ea = EpiArgs{y_part, p.splits, h_part, p.splits, a.M, a.N, a.r, a.B, a.s, a.Y, a.H_out};
  d.blocks = 0;   // set by share_row_waves
  d.qtype = a.sc.qtype;
  return d;
}

// Row waves of the problems of one decode launch.  Every wave walks its rows
// to the end, so the row workgroups are sized to what fits on the GPU at once
// (a workgroup that waits for a free slot finishes late by the whole wait),
// and those waves are shared among the problems in proportion to their
// weights' bytes, so that the problems run side by side and end together.
// Which wave computes a row does not change the row's arithmetic.
static void share_row_waves(DecodePlan *d, int n) {
  const int64_t slots = (int64_t)gemv_resident(d[0].fn) * num_cus();
  double bytes = 0.0;
  for (int i = 0; i < n; ++i) bytes += (double)d[i].ga.N * (double)d[i].ga.K;
  const int64_t waves = slots * (kThreads / 64);
  for (int i = 0; i < n; ++i) {
    GemvArgs &ga = d[i].ga;
    const int64_t share = (int64_t)((double)waves * ((double)ga.N * (double)ga.K / bytes));
    ga.row_waves = std::min<int64_t>(cdiv(ga.N, 2), std::max<int64_t>(1, share / ga.splits));
    d[i].blocks = (int)cdiv(ga.row_waves * ga.splits, kThreads / 64);
  }
}

// One streaming launch and one epilogue launch over n decode problems that
// share the kernel instance and the 4-bit type.
static hipError_t launch_decode(const DecodePlan *dp, int n, hipStream_t st) {
  DecodePlan d[QN_MAX_GROUP];
  for (int i = 0; i < n; ++i) d[i] = dp[i];
  share_row_waves(d, n);
  GemvGroup gg{};
  EpiGroup eg{};
  int64_t gb = 0, eb = 0;
  for (int i = 0; i < n; ++i) {
    gg.p[i] = d[i].ga;
    gg.start[i] = (int)gb;
    gb += d[i].blocks;
    eg.p[i] = d[i].ea;
    eg.start[i] = (int)eb;
    eb += d[i].ea.N / EPI_ROWS;
  }
  for (int k = n; k <= QN_MAX_GROUP; ++k) {
    gg.start[k] = (int)gb;
    eg.start[k] = (int)eb;
  }
  gg.n = eg.n = n;
  const Code16 cb = code16(d[0].qtype);
  {
    // The trace brackets the streaming kernel alone, not the epilogue.
    TraceScope tr(QN_TRACE_GEMV, st);
    void *args[] = {&gg, const_cast<Code16 *>(&cb)};
    QN_TRY(hipLaunchKernel(d[0].fn, dim3((unsigned)gb), dim3(kThreads), args, 0, st));
  }
  QN_TRY(hipGetLastError());
  hipLaunchKernelGGL(gemv_epilogue_kernel, dim3((unsigned)eb), dim3(kThreads), 0, st, eg);
  return hipGetLastError();
}

hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
  if (a.M <= GEMV_MAX_M) {
    const DecodePlan d = decode_plan(a);
    return launch_decode(&d, 1, st);
  }
  // MFMA path: H = X A^T (low-rank kernel) -> sH bf16 -> tile GEMM with the
  // adapter term as extra contraction steps.
  LowRankArgs la;
  QGemmArgs g;
  fwd_mfma_args(a, la, g);
  QN_TRY(launch_lowrank(la, st));
  return launch_qgemm_fwd(g, st);
}

hipError_t run_fwd_group(const FwdArgs *a, int n, hipStream_t st) {
  LowRankArgs la[QN_MAX_GROUP];
  QGemmArgs g[4][QN_MAX_GROUP];   // [2 * (4-bit type) + (double-quantised scales?)][problem]
  int nl = 0, ng[4] = {0, 0, 0, 0};
  // Decode-path problems: one launch pair per kernel instance and type.
  DecodePlan dp[QN_MAX_GROUP];
  bool done[QN_MAX_GROUP] = {};
  int nd = 0;
  for (int i = 0; i < n; ++i)
    if (a[i].M <= GEMV_MAX_M) dp[nd++] = decode_plan(a[i]);
  for (int i = 0; i < nd; ++i) {
    if (done[i]) continue;
    DecodePlan batch[QN_MAX_GROUP];
    int nb = 0;
    for (int k = i; k < nd; ++k)
      if (!done[k] && dp[k].fn == dp[i].fn && dp[k].qtype == dp[i].qtype) {
        batch[nb++] = dp[k];
        done[k] = true;
      }
    QN_TRY(launch_decode(batch, nb, st));
  }
  for (int i = 0; i < n; ++i) {
    if (a[i].M <= GEMV_MAX_M) continue;
    const int kind = 2 * (a[i].sc.qtype == QN_FP4) + (a[i].sc.absmax_q != nullptr);
    fwd_mfma_args(a[i], la[nl], g[kind][ng[kind]]);
    ++nl;
    ++ng[kind];
  }
  if (nl) QN_TRY(launch_lowrank_n(la, nl, st));
  for (int kind = 0; kind < 4; ++kind)
    if (ng[kind]) QN_TRY(launch_qgemm_fwd_group(g[kind], ng[kind], st));
  return hipSuccess;
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
  c.take<char>((int64_t)lowrank_part_bytes(M, N, r));  // dH partial products
  c.take<char>((int64_t)lowrank_part_bytes(M, K, r));  // H partial products (H not given)
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
  float *dhpart = reinterpret_cast<float *>(c.take<char>((int64_t)lowrank_part_bytes(a.M, a.N, a.r)));
  float *hpart = reinterpret_cast<float *>(c.take<char>((int64_t)lowrank_part_bytes(a.M, a.K, a.r)));

  // B^T [rp, N] (rows >= r zero) so that dH = dY (B^T)^T runs on the low-rank
  // kernel; with the forward's H given, (sH)^T from it in the same launch.
  {
    const int64_t elems = rp * a.N + (a.H ? rp * Mp : 0);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)cdiv(elems, kThreads)), dim3(kThreads), 0, st, a.B, a.N,
                       a.r, rp, Bt, a.H, a.M, Mp, a.s, sHt);
    QN_TRY(hipGetLastError());
  }
  // One launch: dH = s dY B -> dHb [M, rp], dHt [rp, Mp]; without a given H also
  // H = X A^T -> (sH)^T [rp, Mp].
  {
    LowRankArgs ld{}, lh{};
    ld.L = a.dY; ld.ldl = a.N; ld.M = a.M; ld.Kc = a.N;
    ld.P = Bt; ld.ldp = a.N; ld.R = a.r; ld.scale = a.s;
    ld.out_b = dHb; ld.ldb = rp; ld.out_t = dHt; ld.ldt_rows = rp; ld.Mp = Mp; ld.part = dhpart;
    lh.L = a.X; lh.ldl = a.K; lh.M = a.M; lh.Kc = a.K;
    lh.P = a.A; lh.ldp = a.K; lh.R = a.r; lh.scale = a.s;
    lh.out_t = sHt; lh.ldt_rows = rp; lh.Mp = Mp; lh.part = hpart;
    QN_TRY(launch_lowrank2(ld, a.H ? nullptr : &lh, st));
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
    g.qtype = a.sc.qtype;
    g.L2 = dHb; g.ldl2 = rp; g.R2 = a.A; g.ldr2 = a.K; g.r = a.r;
    g.out = a.dX; g.ldo = a.K;
    QN_TRY(launch_qgemm_dx(g, st));
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- no-allocation forward
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): the forward's workspace is this file-scope array,
// one copy per device, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per device
// with that device current, and is cached.  Nothing in the forward's workspace
// needs to start at zero (every piece is written before it is read), so the
// array is never cleared.  Calls on one device share it: two such calls that
// overlap in time on one device (different streams or host threads without
// ordering) race on it.
static __device__ __align__(256) uint8_t scratch[QN_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace qn
