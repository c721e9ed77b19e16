// Dequant-GEMM for the QLoRA linear on gfx950: the large contractions of the
// forward (Y = X W_hat^T + s H B^T) and of the backward (dX = dY W_hat + dH A).
//
// "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", "Why the
// expansion cannot be skipped": for every multiply the kernel reads the 4-bit
// codes of a block of weights, looks each up in the sixteen-row table,
// multiplies by the block's scale, writes the bf16 result to on-chip memory,
// and only then feeds the matrix unit.  Here every code becomes
// bf16(fl32(c[q] * A)) (round to nearest even) in an LDS tile that feeds
// v_mfma_f32_32x32x16_bf16: row-major weights through byte permutes in
// registers, transposed weights through a byte-pair table in LDS.
//
// Tiling.  A workgroup computes a 256 x 128 output tile with 8 waves in two
// roles.
//   * Four MMA waves (one per SIMD), each owning 64 rows x 128 columns (2 x 4
//     MFMA tiles of 32 x 32).  A wave issues no global loads: it reads the
//     operand fragments from LDS two k-slices ahead of the MFMAs that use
//     them and issues the MFMAs.
//   * Four producer waves, one per MMA wave, move that wave's activation rows
//     into LDS with direct-to-LDS loads (three stages, one step ahead of the
//     stage being read, waited for with explicit vmcnt before the barrier),
//     load the weight codes and block scales two steps ahead into registers,
//     dequantise them and write the next weight stage.  Sharing each SIMD with
//     an MMA wave, their VALU work overlaps the matrix-core work.
// The contraction runs in steps of 64 (one NF4 block along K), the weight
// stage double-buffered in LDS, one barrier per step.  Within a step, lane
// half h of an MMA wave covers contraction indices [32h, 32h+32); slice c of
// the four MFMA k-slices uses [32h+8c, 32h+8c+8) for both operands, which
// leaves the contraction unchanged.
// The adapter term is one more step after the last weight step: its left
// operand (H or dH, zero beyond ldl2) comes through the activation stages and
// its right operand (B or A, zero beyond r) through the weight stage, into
// the same accumulators before the bf16 store.
//
// Weight layouts:
//   NK (forward): output column n reads weight row n, contraction along K; a
//      producer lane dequantises 32 consecutive codes of one row (16 bytes).
//   KN (dX): the contraction runs over the weight's rows; a producer lane
//      loads 32 codes of one row (16 bytes, one block), the four lanes of a
//      quad transpose their words with DPP so that each lane holds a 4 x 8
//      patch (4 rows, 8 columns), and the patch is written transposed.
// Both stage layouts are XOR-swizzled in 16-byte chunks so that the fragment
// reads and the weight-stage writes are free of bank conflicts (see kswz and
// the activation-stage comment below).

#include <algorithm>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 512;            // 4 MMA waves + 4 producer waves
constexpr int kProducers = 256;
constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LD = BK + 8;               // bf16 per LDS row of the weight tile (16 B pad)
constexpr int WM = 64;                   // rows per MMA wave
constexpr int TM = WM / 32, TN = BN / 32;
constexpr int R_TILE = BN * LD;          // bf16 elements per weight stage
constexpr int kPairCopies = 8;
constexpr int XW = WM * BK;             // bf16 per wave per activation stage (8 KB)
constexpr int XSTAGE = 4 * XW;           // bf16 per activation stage (4 MMA waves)

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit dwords
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // a per-lane offset that always reads zero

// Buffer resource over [base, base + bytes); loads beyond `bytes` (by the
// per-lane offset) return zero, which masks ragged tile edges.
// Every resource of this kernel is wave-uniform; building it from values read
// out of the first lane keeps it in scalar registers (a resource the compiler
// takes for divergent turns each access into a loop, and then it can no
// longer count outstanding loads and waits for all of them).
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0xFFFFFFF0LL;
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(uint32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcFlags);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

__device__ __forceinline__ void tile_coords(int h, int tiles_m, int tiles_n, int gm_rows, int &tm, int &tn) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of logical tiles, ordered in groups of `gm_rows` row-tiles,
  // so that the workgroups an XCD runs together share activation row-panels
  // and weight column-panels in its L2.
  const int T = tiles_m * tiles_n;
  int L = h;
  if ((T & 7) == 0) L = (h & 7) * (T >> 3) + (h >> 3);
  const int GM = gm_rows;
  const int group = GM * tiles_n;
  const int g = L / group;
  const int first_m = g * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in = L - g * group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// LDS weight stage: output column `col` (a row of the stage, LD bf16 long)
// holds contraction positions 0..63.  Position k is stored at k ^ kswz(col):
// the XOR moves whole 8-element chunks, so every 16-byte fragment stays
// contiguous.  On gfx950 a 16-byte LDS read serves 16 lanes per cycle, taken
// as 8-lane blocks 0+3, 1+2, 4+7 and 5+6 of the wave (measured over 256 bank
// patterns: all agree with this pairing and with no other).  With the row
// pitch of 36 banks, columns c .. c+7 and c+24 .. c+31 (c = 32j) fall into
// complementary bank sets, as do c+8 .. c+15 and c+16 .. c+23, so the MMA
// reads (lane lr reads column 32j + lr) are conflict-free as long as the
// half-row XOR (32) is the same within each pair: it is keyed on bit 3 XOR
// bit 4 of the column.  That XOR also separates columns c and c + 16, which
// the transposed-weight producers write in the same cycle (8-byte writes),
// and the 8j term staggers the producer waves.
__device__ __forceinline__ int kswz(int col) { return 32 * (((col >> 3) ^ (col >> 4)) & 1) + 8 * ((col >> 5) & 3); }

template <int CTRL>
__device__ __forceinline__ uint32_t qperm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// ------------------------------------------------------------ producer waves
// NK: producer thread t owns output column row_nk = 16*(t>>5) + (t&15) and the
// contraction half (t>>4)&1 of each step: 32 codes = 16 contiguous bytes.
// KN: the weight's rows are the contraction.  Thread t = 4q + j loads the 32
// codes of contraction row 4*(q&15) + j, columns 32*(q>>4) .. +31 (16 bytes,
// one block), then the four lanes of a quad transpose their 4-byte words so
// that lane j holds columns 32*(q>>4) + 8j .. +7 of all four rows: each column
// then has 4 consecutive contraction positions, written as one 8-byte store.
template <bool KN, bool DQ>
struct Producer {
  struct Set {
    uint32_t code[4];
    uint32_t q;
    float st;
  };
  rsrc_t rc, rq, rs;
  uint32_t cvoff, qvoff;
  int64_t blk_base, blk_step;
  int soff_c;                     // code byte advance per step
  int wr_col, wr_k;               // LDS position written by this thread
  int64_t Nout;

  __device__ void init(const QGemmArgs &a, int tid, int64_t n0) {
    Nout = a.Nout;
    if constexpr (!KN) {
      const int row = ((tid >> 5) << 4) | (tid & 15), half = (tid >> 4) & 1;
      rc = make_rsrc(a.codes + n0 * (a.Kc / 2), (a.Nout - n0) * (a.Kc / 2));
      cvoff = (uint32_t)(row * (a.Kc / 2) + half * 16);
      soff_c = BK / 2;
      blk_base = (n0 + row) * (a.Kc / 64);
      blk_step = 1;
      if constexpr (DQ) {
        rq = make_rsrc(a.absmax_q + n0 * (a.Kc / 64), (a.Nout - n0) * (a.Kc / 64));
        qvoff = (uint32_t)(row * (a.Kc / 64));
      } else {
        rq = make_rsrc(a.absmax + n0 * (a.Kc / 64), (a.Nout - n0) * (a.Kc / 64) * 4);
        qvoff = (uint32_t)(row * (a.Kc / 64) * 4);
      }
      if (n0 + row >= a.Nout) cvoff = qvoff = kOutOfRange;
      wr_col = row;
      wr_k = half * 32;
    } else {
      const int q = tid >> 2, j = tid & 3, rr = 4 * (q & 15) + j, cb = 32 * (q >> 4);
      const bool in = n0 + cb < a.Nout;
      const int64_t e0 = (int64_t)rr * a.Nout + n0 + cb;   // element at step 0
      rc = make_rsrc(a.codes, a.Kc * a.Nout / 2);
      cvoff = in ? (uint32_t)(e0 / 2) : kOutOfRange;
      soff_c = (int)(BK / 2 * a.Nout);
      blk_base = e0 >> 6;                                   // 32 codes lie in one block
      blk_step = a.Nout;                                    // BK rows of Nout / 64 blocks
      qvoff = in ? 0u : kOutOfRange;
      if constexpr (DQ) rq = make_rsrc(a.absmax_q, a.Kc * a.Nout / 64);
      else rq = make_rsrc(a.absmax, a.Kc * a.Nout / 64 * 4);
      wr_col = cb + 8 * j;
      wr_k = 4 * (q & 15);
    }
    if constexpr (DQ) rs = make_rsrc(a.scale2, (a.Nout * a.Kc / 64 + 255) / 256 * 4);
  }

  // s is wave-uniform (it becomes the loads' scalar offset).
  __device__ __forceinline__ void issue(Set &t, int s) {
    const u32x4 c4 = __builtin_amdgcn_raw_buffer_load_b128(rc, cvoff, s * soff_c, 0);
    t.code[0] = c4.x; t.code[1] = c4.y; t.code[2] = c4.z; t.code[3] = c4.w;
    const int64_t b = blk_base + (int64_t)s * blk_step;
    if constexpr (!KN) {
      if constexpr (DQ) {
        t.q = __builtin_amdgcn_raw_buffer_load_b8(rq, qvoff, s, 0);
        t.st = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
            rs, qvoff == kOutOfRange ? kOutOfRange : (uint32_t)((b >> 8) * 4), 0, 0));
      } else {
        t.q = __builtin_amdgcn_raw_buffer_load_b32(rq, qvoff, s * 4, 0);
      }
    } else {
      if constexpr (DQ) {
        t.q = __builtin_amdgcn_raw_buffer_load_b8(rq, qvoff == kOutOfRange ? kOutOfRange : (uint32_t)b, 0, 0);
        t.st = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
            rs, qvoff == kOutOfRange ? kOutOfRange : (uint32_t)((b >> 8) * 4), 0, 0));
      } else {
        t.q = __builtin_amdgcn_raw_buffer_load_b32(rq, qvoff == kOutOfRange ? kOutOfRange : (uint32_t)(b * 4), 0, 0);
      }
    }
  }

  __device__ __forceinline__ float scale(const Set &t) const {
    if constexpr (DQ) return (float)t.q * t.st;
    else return as_f32(t.q);
  }

  // hook(i), i = 0..3, is called at four evenly spaced points of the work
  // (the caller issues its own memory operations there; each call is fenced
  // off from the scheduler so that it stays where it is).
  template <typename Hook>
  __device__ __forceinline__ void store(const Set &t, uint16_t *Rs, const float2 *pair, const float *cv,
                                        int lane, Hook &&hook) const {
    const int copy = lane & (kPairCopies - 1);
    const float A = scale(t);
    if constexpr (!KN) {
      // All 32 codes share one block scale: build the block's sixteen bf16
      // products bf16(fl32(c[q] * A)) once, split into a low-byte and a
      // high-byte plane (4 words each, entries 4m..4m+3 in word m), and look the
      // codes up four at a time with byte permutes (no LDS traffic).
      uint32_t P[8], LO[4], HI[4];
#pragma unroll
      for (int k = 0; k < 8; ++k) P[k] = pack_bf16x2(cv[2 * k] * A, cv[2 * k + 1] * A);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        LO[m] = __builtin_amdgcn_perm(P[2 * m + 1], P[2 * m], 0x06040200u);
        HI[m] = __builtin_amdgcn_perm(P[2 * m + 1], P[2 * m], 0x07050301u);
      }
      // x: four codes in element order, one per byte (bits 0-3) -> low and high
      // bytes of their products.  Bit 3 picks the table half; its byte mask
      // comes from a packed 16-bit multiply (full rate, unlike a 32-bit one).
      auto look = [&](uint32_t x, uint32_t &lo, uint32_t &hi) {
        const uint32_t s7 = x & 0x07070707u;
        const u16x2 bit3 = __builtin_bit_cast(u16x2, (x >> 3) & 0x01010101u);
        const uint32_t upper = __builtin_bit_cast(uint32_t, bit3 * (u16x2){0xFF, 0xFF});
        const uint32_t l0 = __builtin_amdgcn_perm(LO[1], LO[0], s7), l1 = __builtin_amdgcn_perm(LO[3], LO[2], s7);
        const uint32_t h0 = __builtin_amdgcn_perm(HI[1], HI[0], s7), h1 = __builtin_amdgcn_perm(HI[3], HI[2], s7);
        lo = (upper & l1) | (~upper & l0);
        hi = (upper & h1) | (~upper & h0);
      };
      uint32_t o[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        hook(i);
        __builtin_amdgcn_sched_barrier(0);
        // Byte b of the word holds element 2b (low nibble) and 2b + 1 (high
        // nibble).  Interleave the word with itself shifted by a nibble so that
        // each byte's low nibble is one element, in element order.
        const uint32_t w = t.code[i], w4 = w >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t lo, hi;
          look(__builtin_amdgcn_perm(w4, w, h ? 0x07030602u : 0x05010400u), lo, hi);
          o[4 * i + 2 * h + 0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
          o[4 * i + 2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
        // Pin this chunk's results here (the compiler would otherwise sink
        // the arithmetic to the stores below, past every hook).
        asm volatile("" : "+v"(o[4 * i]), "+v"(o[4 * i + 1]), "+v"(o[4 * i + 2]), "+v"(o[4 * i + 3]));
      }
      uint16_t *row = Rs + wr_col * LD;
      const int sw = kswz(wr_col);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4 *>(&row[(wr_k + 8 * i) ^ sw]) = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    } else {
      // 4 x 4 transpose of words within the quad: w[i] of lane j <- word j of lane i.
      uint32_t w0 = t.code[0], w1 = t.code[1], w2 = t.code[2], w3 = t.code[3];
      const bool odd = lane & 1, hi = lane & 2;
      {
        uint32_t x = odd ? w0 : w1, y = odd ? w2 : w3;
        x = qperm<0xB1>(x);
        y = qperm<0xB1>(y);
        if (odd) { w0 = x; w2 = y; } else { w1 = x; w3 = y; }
      }
      {
        uint32_t x = hi ? w0 : w2, y = hi ? w1 : w3;
        x = qperm<0x4E>(x);
        y = qperm<0x4E>(y);
        if (hi) { w0 = x; w1 = y; } else { w2 = x; w3 = y; }
      }
      const uint32_t au = as_u32(A);
      const float S[4] = {as_f32(qperm<0x00>(au)), as_f32(qperm<0x55>(au)), as_f32(qperm<0xAA>(au)),
                          as_f32(qperm<0xFF>(au))};
      const uint32_t wv[4] = {w0, w1, w2, w3};
      float v[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        hook(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float2 p = pair[((wv[i] >> (8 * m)) & 0xFF) * kPairCopies + copy];
          v[i][2 * m] = p.x * S[i];
          v[i][2 * m + 1] = p.y * S[i];
        }
      }
      const int k = wr_k ^ kswz(wr_col);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x2 *>(&Rs[(wr_col + c) * LD + k]) =
            u32x2{pack_bf16x2(v[0][c], v[1][c]), pack_bf16x2(v[2][c], v[3][c])};
    }
  }
};

// Adapter term as one more contraction step (r <= 64 = BK): its right operand,
// positions j < r of the tile's 128 columns (zero beyond r and beyond Nout),
// is fetched by the producers into registers when the kernel starts and
// written to the weight stage after the last weight step.  Producer thread t
// owns column t & 127, positions 32 (t >> 7) .. +31: 32 independent 2-byte
// loads (R2 need not be 16-byte aligned), one latency in all.
template <bool EPI_NK>
__device__ __forceinline__ void load_adapter_right(const QGemmArgs &a, int64_t n0, int t, uint32_t (&h)[32]) {
  const int row = t & (BN - 1), j0 = 32 * (t >> 7);
  const int64_t gn = n0 + row;
  const rsrc_t rr = make_rsrc(a.R2, EPI_NK ? a.Nout * a.ldr2 * 2 : a.r * a.ldr2 * 2);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t j = j0 + i;
    const bool in = j < a.r && gn < a.Nout;
    const uint32_t off = in ? (uint32_t)((EPI_NK ? gn * a.ldr2 + j : j * a.ldr2 + gn) * 2) : kOutOfRange;
    h[i] = __builtin_amdgcn_raw_buffer_load_b16(rr, off, 0, 0);
  }
}
// The 2-byte values are packed only here, at the use, so that the wait for
// the loads falls at the end of the main loop.
__device__ __forceinline__ void store_adapter_right(const uint32_t (&h)[32], uint16_t *Rs, int t) {
  const int row = t & (BN - 1), j0 = 32 * (t >> 7);
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (h[2 * i] & 0xFFFFu) | (h[2 * i + 1] << 16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x4 *>(&Rs[row * LD + ((j0 + 8 * q) ^ kswz(row))]) = u32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// Workgroup barrier that orders the waves' own LDS reads and writes only:
// global loads issued before it stay in flight, including the producers'
// direct-to-LDS activation loads for later stages, which they wait for with
// explicit counts before the barrier that publishes each stage (a
// compiler-generated LDS fence would wait for all of them here).
// The LDS wait is the builtin, not asm, so that the compiler's own wait
// tracking knows every LDS read issued before the barrier has completed;
// otherwise it re-waits for them after the barrier, and since the counter is
// in order that also waits for the fragment reads issued since.  The empty
// asm and the asm barrier (both memory clobbers) keep LDS accesses on their
// side of the wait.
// s_waitcnt with vmcnt(n), the other counters unconstrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not constrained
  asm volatile("s_barrier" ::: "memory");
}

// Exactly one workgroup (2 waves per SIMD) fits a CU, so tell the compiler
// that higher occupancy is not reachable: it may then keep a whole step's
// operands in registers instead of re-reading them one by one.
template <bool KN, bool DQ, bool EPI_NK>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qgemm_kernel(QGemmArgs a, Code16 cb) {
  // Separate arrays per stage: the compiler then tracks the direct-to-LDS
  // loads into each activation stage on their own and waits only for the
  // stage a fragment read touches.
  __shared__ __attribute__((aligned(16))) uint16_t xs0[XSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[XSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[XSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t ws0[R_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ws1[R_TILE];
  // Byte -> (row lo, row hi) table for the transposed-weight producers.
  __shared__ __attribute__((aligned(16))) float2 pair[KN ? 256 * kPairCopies : 1];
  for (int i = threadIdx.x; KN && i < 256 * kPairCopies; i += kThreads) {
    const int e = i / kPairCopies;
    pair[i] = make_float2(cb.v[e & 15], cb.v[e >> 4]);
  }

  int tm, tn;
  tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool producer = wave >= 4;
  const int64_t steps = __builtin_amdgcn_readfirstlane((int)(a.Kc / BK));
  // Contraction steps of 64: Kc / 64 weight steps, then one adapter step
  // (left operand L2, zero beyond ldl2; right operand R2 restricted to j < r).
  const int64_t total = steps + 1;
  lds_barrier();  // pair table

  if (producer) {
    const int tid = threadIdx.x - kProducers;
    Producer<KN, DQ> P;
    P.init(a, tid, n0);
    typename Producer<KN, DQ>::Set s0, s1;
    const int nsteps = __builtin_amdgcn_readfirstlane((int)steps), last = nsteps - 1;   // nsteps >= 1
    const int ntotal = nsteps + 1;   // contraction steps including the adapter step

    // Activation stages.  Producer wave p moves the 64 rows of MMA wave p from
    // global memory into LDS with direct-to-LDS loads (the compiler sees them,
    // so its waits for the code sets stay exact).  Chunk k (16 bytes) of stage
    // row r sits at slot k ^ ((r >> 1) & 7), so the fragment reads of 16
    // consecutive rows hit 16 distinct bank groups.  Load g fills rows 8g ..
    // 8g + 7 (1 KB in lane order): lane l writes slot l & 7 of row 8g + l / 8,
    // every 8 lanes reading one 128-byte line; the swizzle (row >> 1) & 7 is
    // (lane >> 4) ^ 4 (g & 1), so the offsets are two per-lane bases plus 8g
    // rows.  Step `nsteps` (the adapter step) takes columns 0..63 of L2 (zero
    // at or beyond ldl2) the same way.
    const int pw = wave - 4;
    const int64_t wrow0 = m0 + (int64_t)pw * WM;
    const rsrc_t xr = make_rsrc(a.L + wrow0 * a.ldl, (a.M - wrow0) * a.ldl * 2);
    const rsrc_t l2r = make_rsrc(a.L2 + wrow0 * a.ldl2, (a.M - wrow0) * a.ldl2 * 2);
    const uint32_t c0 = (uint32_t)((lane & 7) ^ (lane >> 4));   // chunk for even g; odd g: c0 ^ 4
    const uint32_t xbase0 = (uint32_t)((lane >> 3) * a.ldl * 2 + c0 * 16);
    const uint32_t xbase1 = (uint32_t)((lane >> 3) * a.ldl * 2 + (c0 ^ 4u) * 16);
    const uint32_t xrow8 = (uint32_t)(8 * a.ldl * 2);
    // The adapter step reads L2 the same way (row pitch ldl2, columns at or
    // beyond ldl2 zero); loads at t >= ntotal read zero (every offset out of
    // range) into a slot that no one reads again, which keeps the number of
    // loads per half-step fixed.  One branch-free issue path for all three:
    // the resource and the scalar offset are chosen uniformly, the per-lane
    // offset from precomputed bases.
    const uint32_t l2base0 = (uint32_t)((lane >> 3) * a.ldl2 * 2 + c0 * 16);
    const uint32_t l2base1 = (uint32_t)((lane >> 3) * a.ldl2 * 2 + (c0 ^ 4u) * 16);
    const bool l2ok0 = 8 * (int64_t)c0 < a.ldl2, l2ok1 = 8 * (int64_t)(c0 ^ 4u) < a.ldl2;
    const uint32_t l2row8 = (uint32_t)(8 * a.ldl2 * 2);
    // Loads 2q and 2q + 1 of activation stage t (q = 0..3).
    auto issue_x = [&](int t, int q) {
      const int i = t % 3;
      const uint32_t base =
          (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr((i == 0 ? xs0 : (i == 1 ? xs1 : xs2)) + pw * XW));
      const bool main_step = t < nsteps, live = t < ntotal;
      const rsrc_t r = main_step ? xr : l2r;
      const int soff = main_step ? t * BK * 2 : 0;
#pragma unroll
      for (int g = 2 * q; g < 2 * q + 2; ++g) {
        const bool odd = g & 1;
        const uint32_t l2off =
            live && (odd ? l2ok1 : l2ok0) ? (odd ? l2base1 : l2base0) + (uint32_t)g * l2row8 : kOutOfRange;
        const uint32_t off = main_step ? (odd ? xbase1 : xbase0) + (uint32_t)g * xrow8 : l2off;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(size_t)(base + g * 1024),
                                                 16, off, soff, 0, 0);
      }
    };

    // Half-step t (t = 0 .. nsteps) ends with barrier t.  It issues activation
    // stage t + 1 (its slot was last read before barrier t - 1), writes weight
    // step t (t = nsteps: the adapter's right operand) to stage t & 1 from
    // register set t & 1, reloads that set for step t + 2, and before the
    // barrier waits for activation stage t, issued in the previous half-step:
    // the loads issued after it are that half-step's reload (kReload), stage
    // t + 1 (8) and this half-step's reload.  Every half-step issues the same
    // loads (code loads past the end re-read the last step, activation loads
    // past the end read zero), and the prologue issues code set 0, stage 0 and
    // code set 1 in that order, so the loop is entered with the loads in the
    // order of its back edge and the compiler's own waits for the code sets
    // stay exact.
    uint32_t adapter[32];
    load_adapter_right<EPI_NK>(a, n0, tid, adapter);
    __builtin_amdgcn_sched_barrier(0);
    P.issue(s0, 0);
    __builtin_amdgcn_sched_barrier(0);
    {
      // Stage 0 is always a weight step (nsteps >= 1): the same eight loads as
      // issue_x(0) without its selects, which the compiler would otherwise
      // turn into branches with different load counts on each side (and then
      // wait conservatively inside the loop).
      const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(xs0 + pw * XW));
#pragma unroll
      for (int g = 0; g < 8; ++g)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void *)(size_t)(base + g * 1024), 16,
                                                 ((g & 1) ? xbase1 : xbase0) + (uint32_t)g * xrow8, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    P.issue(s1, __builtin_amdgcn_readfirstlane(min(1, last)));
    __builtin_amdgcn_sched_barrier(0);
    // The eight activation loads are spread over the dequantisation: issued
    // back to back, the four producer waves' loads fill the CU's vector memory
    // path for several hundred cycles, and each wave would sit at its next
    // load instead of dequantising.
    // A half-step's reload is the code set plus its block scale: the
    // quantised scale and the group step, or one fp32 scale.
    constexpr int kReload = DQ ? 3 : 2;
    auto half = [&](int t, typename Producer<KN, DQ>::Set &set, uint16_t *wdst) {   // t < nsteps
      P.store(set, wdst, pair, cb.v, lane, [&](int q) { issue_x(t + 1, q); });
      __builtin_amdgcn_sched_barrier(0);
      P.issue(set, min(t + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_only(kReload + 8 + kReload));
      lds_barrier();
    };
    // Weight half-steps in pairs, then the odd one out.  Neither an exit from
    // the middle of the loop body nor a branch between two arms that both
    // load: the compiler gives such control flow a path that skips the loads
    // (or leaves the loop body early), and its wait counts then assume that
    // path and wait for loads that are still a half-step early.
    int t = 0;
    for (; t + 2 <= nsteps; t += 2) {
      half(t, s0, ws0);
      half(t + 1, s1, ws1);
    }
    if (t < nsteps) {
      half(t, s0, ws0);
      ++t;
    }
    // Half-step nsteps: the adapter's right operand; its left operand is
    // activation stage nsteps, issued in the last weight half-step.
    store_adapter_right(adapter, (t & 1) ? ws1 : ws0, tid);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    lds_barrier();
    lds_barrier();   // the MMA waves' barrier after the adapter step: nothing is in flight
    return;
  }

  // ---------------------------------------------------------- MMA waves
  const int lr = lane & 31, lh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Activation stages are filled by the producer waves (see there); this
  // wave only reads them, after the barrier that follows their loads.
  // Fragment offsets: A (activations) tile i, slice c: row 32i + lr, chunk 4lh + c;
  // B (weights) column 32j + lr, positions 32lh + 8c .. +7, stored at 32(lh ^ g) + 8(c ^ j),
  // g = bit 3 ^ bit 4 of lr.
  uint32_t aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = (uint32_t)(wave_u * XW + lr * BK + (((4 * lh + c) ^ ((lr >> 1) & 7)) * 8));
  const int rb = lr * LD + 32 * (lh ^ (((lr >> 3) ^ (lr >> 4)) & 1));
  struct Frag {
    bf16x8 a[TM];
    bf16x8 b[TN];
  };
  auto read_b = [&](bf16x8 *b, const uint16_t *wc, int c) {
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(&wc[rb + j * 32 * LD + 8 * (c ^ j)]);
  };
  auto read_f = [&](Frag &f, const uint16_t *xc, const uint16_t *wc, int c) {
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const bf16x8 *>(&xc[aoff[c] + i * 32 * BK]);
    read_b(f.b, wc, c);
  };
  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // Fragment reads run two slices ahead of the MFMAs that use them (three
  // fragment buffers rotate).  One step: stages (xc, wc) now, (xn, wn) next,
  // x2 is refilled for step s + 2 (it was last read in step s - 1).  On entry
  // F0 and F1 hold slices 0 and 1 of step s; on exit F1 and F2 hold slices 0
  // and 1 of step s + 1, so the next step takes (F1, F2, F0).
  auto step = [&](int64_t s, const uint16_t *xc, const uint16_t *wc, const uint16_t *xn, const uint16_t *wn,
                  uint16_t *x2, Frag &F0, Frag &F1, Frag &F2) {
    (void)x2;
    read_f(F2, xc, wc, 2);
    __builtin_amdgcn_sched_barrier(0);
    mma(F0);
    read_f(F0, xc, wc, 3);
    __builtin_amdgcn_sched_barrier(0);
    mma(F1);
    lds_barrier();
    if (s + 1 < steps) read_f(F1, xn, wn, 0);
    __builtin_amdgcn_sched_barrier(0);
    mma(F2);
    if (s + 1 < steps) read_f(F2, xn, wn, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(F0);
  };
  Frag fa, fb, fc;
  lds_barrier();
  read_f(fa, xs0, ws0, 0);
  read_f(fb, xs0, ws0, 1);
  // Step s uses activation stage s % 3 and weight stage s % 2.
  for (int64_t s = 0; s < steps; s += 6) {
    step(s, xs0, ws0, xs1, ws1, xs2, fa, fb, fc);
    if (s + 1 >= steps) break;
    step(s + 1, xs1, ws1, xs2, ws0, xs0, fb, fc, fa);
    if (s + 2 >= steps) break;
    step(s + 2, xs2, ws0, xs0, ws1, xs1, fc, fa, fb);
    if (s + 3 >= steps) break;
    step(s + 3, xs0, ws1, xs1, ws0, xs2, fa, fb, fc);
    if (s + 4 >= steps) break;
    step(s + 4, xs1, ws0, xs2, ws1, xs0, fb, fc, fa);
    if (s + 5 >= steps) break;
    step(s + 5, xs2, ws1, xs0, ws0, xs1, fc, fa, fb);
  }

  // ---- adapter step: its left operand (direct-to-LDS, issued two steps
  // ago) sits in activation stage steps % 3, its right operand in weight stage
  // steps & 1 (written by the producers before the main loop's last barrier).
  // The trip count is written in terms of r (it is 1 for every 1 <= r <= 64):
  // with a constant count the code after the main loop becomes straight-line
  // and the register allocator then spills the accumulators inside the loop.
  const int64_t epi_steps = (a.r + BK - 1) / BK;
  for (int64_t e = 0; e < epi_steps; ++e) {
    const int xi = (int)(steps % 3);
    const uint16_t *xa = xi == 0 ? xs0 : (xi == 1 ? xs1 : xs2);
    const uint16_t *wa = (steps & 1) ? ws1 : ws0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Frag f;
      read_f(f, xa, wa, c);
      mma(f);
    }
    lds_barrier();   // pairs with the producers' last barrier
  }

  // ---- store bf16 through LDS.  Element e of a 32 x 32 accumulator tile is
  // row 8*(e/4) + 4*lh + (e%4), column lr: stored straight to global memory
  // that is 2 bytes per lane and 128 stores per lane.  Instead each wave
  // writes its two 32 x 128 blocks into the activation stages (all LDS reads
  // ended at the barrier above; only this wave touches its blocks) with a row
  // pitch of kOutPitch (rows r and r + 4 land 16 banks apart), then reads back
  // 16-byte row chunks and stores them whole: 16 row-contiguous stores per
  // wave.  Rows at or beyond M fall outside the buffer and are dropped;
  // columns beyond Nout (or an output not 16-byte aligned) take element stores.
  constexpr int kOutPitch = BN + 8;
  static_assert(3 * 32 * kOutPitch <= XSTAGE, "three output blocks per activation stage");
  const rsrc_t rout = make_rsrc(a.out + m0 * a.ldo, (a.M - m0) * a.ldo * 2);
  const bool vec_ok = (a.ldo & 7) == 0 && ((uint64_t)a.out & 15) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int k = 2 * wave_u + i;   // output block 0..7: three per activation stage
    uint16_t *blk = (k < 3 ? xs0 : (k < 6 ? xs1 : xs2)) + (k % 3) * 32 * kOutPitch;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        blk[(8 * (e >> 2) + 4 * lh + (e & 3)) * kOutPitch + j * 32 + lr] = f32_to_bf16(acc[i][j][e]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 4 * q + (lane >> 4), c8 = 8 * (lane & 15);
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&blk[row * kOutPitch + c8]);
      const int64_t lrow = (int64_t)wave_u * WM + i * 32 + row, gn = n0 + c8;
      if (vec_ok && gn + 8 <= a.Nout) {
        __builtin_amdgcn_raw_buffer_store_b128(v, rout, (uint32_t)((lrow * a.ldo + gn) * 2), 0, 0);
      } else if (m0 + lrow < a.M) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (gn + t < a.Nout) a.out[(m0 + lrow) * a.ldo + gn + t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
      }
    }
  }
}

int64_t cdiv(int64_t x, int64_t y) { return (x + y - 1) / y; }

template <bool KN, bool EPI_NK>
hipError_t launch(const QGemmArgs &a0, hipStream_t st, int trace_kind) {
  QGemmArgs a = a0;
  // The adapter term is exactly one extra contraction step, and the producer
  // and MMA waves count their barriers on that: reject any other rank here.
  if (a.r < 1 || a.r > BK || a.Kc < BK || a.Kc % BK != 0) return hipErrorInvalidValue;
  a.tiles_m = (int)cdiv(a.M, BM);
  a.tiles_n = (int)cdiv(a.Nout, BN);
  // Row-tile group size: each XCD runs T/8 tiles; choose the group so that an
  // XCD's share covers about as many activation bytes (rows x Kc x 2) as weight
  // bytes (columns x Kc / 2).
  {
    const int T8 = std::max(1, a.tiles_m * a.tiles_n / 8);
    int best = 1;
    double best_cost = 1e300;
    for (int g = 1; g <= a.tiles_m; ++g) {
      const int cols = std::max(1, std::min(a.tiles_n, T8 / g));
      const double cost = (double)g * BM * 2 + (double)cols * BN / 2;
      if (cost < best_cost) { best_cost = cost; best = g; }
    }
    a.group_m = best;
  }
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
  TraceScope tr(trace_kind, st);
  if (a.absmax_q)
    hipLaunchKernelGGL((qgemm_kernel<KN, true, EPI_NK>), grid, dim3(kThreads), 0, st, a, code16());
  else
    hipLaunchKernelGGL((qgemm_kernel<KN, false, EPI_NK>), grid, dim3(kThreads), 0, st, a, code16());
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm_fwd(const QGemmArgs &a, hipStream_t st) {
  return launch<false, true>(a, st, QN_TRACE_GEMM_FWD);
}

hipError_t launch_qgemm_dx(const QGemmArgs &a, hipStream_t st) {
  return launch<true, false>(a, st, QN_TRACE_GEMM_DX);
}

}  // namespace qn
