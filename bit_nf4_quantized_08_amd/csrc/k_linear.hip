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
// y_part[split][m][n] = sum over the split's K-segment of x[m][k] * W_hat[n][k],
// the block scale applied to each 32-weight partial sum.  A wave owns one
// K-segment of KW 2048-wide chunks and holds its activations in registers for
// the whole kernel; lane l owns 32 consecutive k of each chunk (16 bytes of
// codes).  The wave then walks rows n = v, v + row_waves, ...: each row is
// one contiguous read of KW KB of codes (rows of neighbouring waves are
// neighbours in memory), and the next row is requested before the current one
// is multiplied.
// The first h_blocks blocks instead compute H partials,
// h_part[split][m][j] = sum over the split's K-range of x[m][k] * A[j][k]:
// block b takes K-range b % hsplits and adapter rows 4 (b / hsplits) .. +3,
// one per wave, so that every wave makes a single pass and H is spread over
// many short blocks that start first.
// 2048-wide chunks per wave segment (KW): the activations of a segment take
// 16 * KW * MM registers per lane, at most 64 (128 for MM = 8, KW = 1), and a
// segment is no longer than the row needs.
int gemv_kw(int mm, int64_t chunks) {
  const int cap = mm == 1 ? 4 : (mm == 2 ? 2 : 1);
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
  float *h_part;      // [hsplits][M][64]
  int64_t k_per_split;   // KW * 2048: the K-segment of one wave
  int splits;            // K-segments
  int64_t row_waves;     // waves per K-segment; wave v takes rows v, v + row_waves, ...
  int h_blocks;       // hsplits * ceil(r / 4)
  int hsplits;
  int64_t hk_per_split;  // H partial K-range per block (multiple of 2048 or K)
};

// 32 activations of each row m at column k (k must be in range).  Rows m >= M
// read row M - 1 instead, so that every load is unconditional; their results
// are never stored.
template <int MM>
__device__ __forceinline__ void load_x_chunk(const GemvArgs &a, int64_t k, uint32_t (&x)[MM][16]) {
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    const int64_t mr = min((int64_t)m, a.M - 1);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(a.X + mr * a.K + k);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = p[c];
      x[m][4 * c] = v.x; x[m][4 * c + 1] = v.y; x[m][4 * c + 2] = v.z; x[m][4 * c + 3] = v.w;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Wave sums of MM values at once (MM a power of two <= 8): each exchange step
// halves the values a lane carries, so MM sums cost MM - 1 + 6 - log2(MM)
// shuffles instead of 6 MM.  Returns, in every lane, the full sum of value
// m = lane >> (6 - log2(MM)).
template <int MM>
__device__ __forceinline__ float wave_sum_multi(float (&v)[MM], int lane) {
  int off = 32;
#pragma unroll
  for (int cnt = MM; cnt > 1; cnt >>= 1, off >>= 1) {
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < cnt / 2; ++i) {
      const float keep = upper ? v[i + cnt / 2] : v[i];
      const float send = upper ? v[i] : v[i + cnt / 2];
      v[i] = keep + __shfl_xor(send, off, 64);
    }
  }
  float t = v[0];
  for (; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
  return t;
}

template <int MM, bool DQ, int KW>
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
        load_x_chunk<MM>(a, k, x);
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

  static_assert(KW * MM <= 4 || KW == 1, "activation registers");
  const int64_t v = (int64_t)((int)blockIdx.x - a.h_blocks) * (kThreads / 64) + wave;
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

  // Rows in pairs with two register sets (no copies between them, so that
  // a set's loads stay in flight while the other set is multiplied), then
  // the odd row out.  (Two rows ahead costs occupancy and was slower.)
  const int64_t rows = cdiv_d(a.N - n_first, a.row_waves);
  Row r0, r1;
  load_row(r0, n_first);
  int64_t n = n_first;
  for (int64_t t = 0; t + 2 <= rows; t += 2) {
    __builtin_amdgcn_sched_barrier(0);
    load_row(r1, n + a.row_waves);
    row_dot(r0, n);
    n += a.row_waves;
    __builtin_amdgcn_sched_barrier(0);
    load_row(r0, n + a.row_waves);
    row_dot(r1, n);
    n += a.row_waves;
  }
  if (rows & 1) row_dot(r0, n);
}

// y[m][n] = sum_s y_part[s][m][n] + s_lora * sum_j H[m][j] * B[n][j], H summed
// from its partials; rounded to bf16.  Optionally writes H (fp32, unscaled).
// A workgroup covers EPI_ROWS rows n.  For the adapter term eight lanes share
// a row of B, each reading 8 consecutive entries (one 16-byte load when r is a
// multiple of 8), so that a wave reads 8 whole rows of B per instruction; the
// eight partial sums are added with lane shuffles.
constexpr int EPI_ROWS = kThreads / 8;

__global__ __launch_bounds__(kThreads) void gemv_epilogue_kernel(const float *__restrict__ y_part, int splits,
                                                                 const float *__restrict__ h_part, int hsplits,
                                                                 int64_t M, int64_t N, int64_t r,
                                                                 const uint16_t *__restrict__ B, float s_lora,
                                                                 uint16_t *__restrict__ Y, float *H_out) {
  __shared__ float Hs[8 * 64];          // H[m][j], zero for j >= r
  __shared__ float Ls[8 * EPI_ROWS];    // sum_j H[m][j] B[n][j] for the workgroup's rows
  const int64_t n0 = (int64_t)blockIdx.x * EPI_ROWS;
  // The split sums of this thread's outputs first, so that their loads
  // overlap those of H and B.
  float ysum[(8 * EPI_ROWS + kThreads - 1) / kThreads];
#pragma unroll
  for (int u = 0; u < (8 * EPI_ROWS + kThreads - 1) / kThreads; ++u) {
    const int idx = threadIdx.x + u * kThreads;
    ysum[u] = 0.0f;
    if (idx < M * EPI_ROWS) {
      const int64_t m = idx / EPI_ROWS, i = idx % EPI_ROWS;
      for (int s = 0; s < splits; ++s) ysum[u] += y_part[((int64_t)s * M + m) * N + n0 + i];
    }
  }
  for (int idx = threadIdx.x; idx < M * 64; idx += kThreads) {
    const int m = idx / 64, j = idx % 64;
    float v = 0.0f;
    if (j < r) {
#pragma unroll 8
      for (int s = 0; s < hsplits; ++s) v += h_part[((int64_t)s * M + m) * 64 + j];
    }
    Hs[idx] = v;
    if (H_out && blockIdx.x == 0 && j < r) H_out[m * r + j] = v;
  }
  const int t = threadIdx.x, row = t >> 3, j0 = 8 * (t & 7);
  const int64_t n = n0 + row;  // N % EPI_ROWS == 0
  float b[8];
  if (r % 8 == 0) {
    const u32x4 v = j0 < r ? *reinterpret_cast<const u32x4 *>(B + n * r + j0) : u32x4{0, 0, 0, 0};
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
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
#pragma unroll
  for (int u = 0; u < (8 * EPI_ROWS + kThreads - 1) / kThreads; ++u) {
    const int idx = t + u * kThreads;
    if (idx < M * EPI_ROWS) {
      const int64_t m = idx / EPI_ROWS, i = idx % EPI_ROWS;
      Y[m * N + n0 + i] = f32_to_bf16(__builtin_fmaf(s_lora, Ls[idx], ysum[u]));
    }
  }
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

struct GemvPlan {
  int splits;          // K-segments of gemv_kw(mm) chunks
  int64_t kps;         // K per segment
  int64_t row_waves;   // waves per segment
  int row_wgs;         // workgroups for the rows
  int hsplits;         // K-ranges of the H partials
  int64_t hkps;
};

int gemv_mm(int64_t M) { return M == 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8)); }

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K) {
  GemvPlan p;
  const int64_t chunks = cdiv(K, 2048);
  const int64_t kw = gemv_kw(gemv_mm(M), chunks);
  p.kps = kw * 2048;
  p.splits = (int)cdiv(chunks, kw);
  p.row_waves = 0;
  p.row_wgs = 0;
  p.hkps = 2048 * cdiv(chunks, std::min<int64_t>(chunks, 64));
  p.hsplits = (int)cdiv(K, p.hkps);
  return p;
}

// The decode kernel instance for M rows of activations and kw chunks per
// segment.
template <bool DQ>
const void *gemv_fn(int64_t M, int64_t kw) {
  switch (gemv_mm(M)) {
    case 1:
      return kw == 4 ? reinterpret_cast<const void *>(&gemv_kernel<1, DQ, 4>)
           : kw == 2 ? reinterpret_cast<const void *>(&gemv_kernel<1, DQ, 2>)
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

// Rows are dealt to as many waves as fit on the GPU at once (each wave then
// walks its rows to the end with no second round of workgroups), but to no
// more than half the rows, so that every wave has a next row to prefetch.
void gemv_rows(GemvPlan &p, int64_t N, const void *fn) {
  const int64_t waves = (int64_t)gemv_resident(fn) * num_cus() * (kThreads / 64);
  p.row_waves = std::min<int64_t>(cdiv(N, 2), std::max<int64_t>(1, waves / p.splits));
  p.row_wgs = (int)cdiv(p.row_waves * p.splits, kThreads / 64);
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
    c.take<float>((int64_t)p.hsplits * M * 64);
  } else {
    c.take<uint16_t>(M * align_up(r, 8));
  }
  return c.off;
}

hipError_t run_fwd(const FwdArgs &a, hipStream_t st) {
  Carve c(a.ws);
  if (a.M <= GEMV_MAX_M) {
    GemvPlan p = gemv_plan(a.M, a.N, a.K);
    const int64_t kw = p.kps / 2048;
    const void *fn = a.sc.absmax_q ? gemv_fn<true>(a.M, kw) : gemv_fn<false>(a.M, kw);
    gemv_rows(p, a.N, fn);
    float *y_part = c.take<float>((int64_t)p.splits * a.M * a.N);
    float *h_part = c.take<float>((int64_t)p.hsplits * a.M * 64);
    const int h_blocks = p.hsplits * (int)cdiv(a.r, 4);
    GemvArgs ga{a.X, a.M, a.N, a.K, a.codes, a.sc, a.A, a.r, y_part, h_part, p.kps, p.splits, p.row_waves,
                h_blocks, p.hsplits, p.hkps};
    dim3 grid((unsigned)(h_blocks + p.row_wgs));
    const Code16 cb = code16();
    TraceScope tr(QN_TRACE_GEMV, st);
    void *args[] = {&ga, const_cast<Code16 *>(&cb)};
    QN_TRY(hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, st));
    QN_TRY(hipGetLastError());
    hipLaunchKernelGGL(gemv_epilogue_kernel, dim3((unsigned)(a.N / EPI_ROWS)), dim3(kThreads), 0, st,
                       y_part, p.splits, h_part, p.hsplits, a.M, a.N, a.r, a.B, a.s, a.Y, a.H_out);
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
