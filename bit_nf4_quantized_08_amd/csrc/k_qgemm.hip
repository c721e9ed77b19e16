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
// The activation stages are XOR-swizzled in 16-byte chunks and the forward
// weight stage has a padded row pitch, so that fragment reads and stage writes
// are free of bank conflicts; the dX weight stage permutes its output columns
// over stage rows and XORs positions per group of 16 rows, so that its
// transposed 8-byte writes spread over the banks while the fragment reads stay
// conflict-free (see wswz, kswz, kn_row and the activation-stage comment
// below).

#include <algorithm>
#include <atomic>
#include <type_traits>

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
// holds contraction positions 0..63, 16-byte chunks of 8.  Bank behaviour of
// gfx950 LDS, measured with a probe of 30 access patterns (timing and the
// SQ_LDS_BANK_CONFLICT counter): a 16-byte read serves 16 consecutive lanes
// per cycle over 64 banks of 4 bytes; a 16-byte write serves 8 consecutive
// lanes per cycle over 32 banks.  With the row pitch of 36 banks, sixteen
// consecutive columns read at one 16-byte position fall on 16 distinct 4-bank
// groups, and eight consecutive columns written at one position on 8 distinct
// groups of the 32: the forward (row-major weight) stages store position k at
// k, with no XOR (wswz<false>).  The transposed producer of dX writes 8-byte
// column patches, the four lanes of a quad to output columns 8 apart at the
// same positions, and 8-byte writes are served 16 lanes per cycle over 32
// banks: with the pitch alone those four columns fall on the same banks.  So
// dX stores output column n in stage row kn_row(n), which puts the four
// columns of a write cycle into four different aligned groups of 16 rows, and
// keeps position k of stage row s at k ^ kswz(s), kswz = 16 * (group of 16 rows
// mod 4): the writes of a cycle fall on four disjoint spans of 8 banks, while
// the MMA reads (16 consecutive stage rows at one position) see one XOR per
// read and stay conflict-free.  kn_row keeps 8-column chunks whole, so the
// output is still stored in 16-byte row chunks (output column kn_col(s)).
__device__ __forceinline__ int kswz(int row) { return 16 * ((row >> 4) & 3); }
__device__ __forceinline__ int kn_row(int n) {
  return 64 * (n >> 6) + 16 * ((n >> 3) & 3) + 8 * ((n >> 5) & 1) + (n & 7);
}
__device__ __forceinline__ int kn_col(int row) {
  return 64 * (row >> 6) + 32 * ((row >> 3) & 1) + 8 * ((row >> 4) & 3) + (row & 7);
}
template <bool KN>
__device__ __forceinline__ int wswz(int col) { return KN ? kswz(col) : 0; }

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
template <bool KN, bool DQ, bool Q4 = false>
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
      wr_col = kn_row(cb + 8 * j);   // stage row of output column cb + 8j (+c for c < 8)
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
      if constexpr (Q4) {
        (void)b;   // the scales come from Scale4
      } else if constexpr (DQ) {
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
    store_scaled(t, scale(t), Rs, pair, cv, lane, hook);
  }
  // The same with the block scale A given.
  template <typename Hook>
  __device__ __forceinline__ void store_scaled(const Set &t, float A, uint16_t *Rs, const float2 *pair,
                                               const float *cv, int lane, Hook &&hook) const {
    const int copy = lane & (kPairCopies - 1);
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
      const int sw = wswz<KN>(wr_col);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4 *>(&row[(wr_k + 8 * i) ^ sw]) = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    } else {
      uint32_t wv[4];
      float S[4];
      patch_prep(t, A, lane, wv, S);
      float v[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        hook(i);
        __builtin_amdgcn_sched_barrier(0);
        patch_row(wv, S, i, pair, copy, v[i]);
      }
      write_patch(Rs, v[0], v[1], v[2], v[3]);
    }
  }

  // Transposed weights, in parts that a caller can spread over its own work:
  // patch_prep transposes the quad's 4 x 4 code words (w[i] of lane j <- word
  // j of lane i) and broadcasts the four rows' block scales within the quad;
  // patch_row expands row i of the lane's 4 x 8 patch through the byte-pair
  // table; write_patch stores the patch transposed (8-byte column pieces).
  __device__ __forceinline__ void patch_prep(const Set &t, float A, int lane, uint32_t (&wv)[4], float (&S)[4]) const {
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
    S[0] = as_f32(qperm<0x00>(au));
    S[1] = as_f32(qperm<0x55>(au));
    S[2] = as_f32(qperm<0xAA>(au));
    S[3] = as_f32(qperm<0xFF>(au));
    wv[0] = w0; wv[1] = w1; wv[2] = w2; wv[3] = w3;
  }
  __device__ __forceinline__ static void patch_row(const uint32_t (&wv)[4], const float (&S)[4], int i,
                                                   const float2 *pair, int copy, float (&v)[8]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float2 p = pair[((wv[i] >> (8 * m)) & 0xFF) * kPairCopies + copy];
      v[2 * m] = p.x * S[i];
      v[2 * m + 1] = p.y * S[i];
    }
  }
  // Rows 0 and 1 may come packed already (pk01[c] = bf16 pair of rows 0, 1).
  __device__ __forceinline__ void write_patch(uint16_t *Rs, const uint32_t (&pk01)[8], const float (&v2)[8],
                                              const float (&v3)[8]) const {
    const int k = wr_k ^ kswz(wr_col);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<u32x2 *>(&Rs[(wr_col + c) * LD + k]) = u32x2{pk01[c], pack_bf16x2(v2[c], v3[c])};
  }
  __device__ __forceinline__ void write_patch(uint16_t *Rs, const float (&v0)[8], const float (&v1)[8],
                                              const float (&v2)[8], const float (&v3)[8]) const {
    uint32_t pk01[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) pk01[c] = pack_bf16x2(v0[c], v1[c]);
    write_patch(Rs, pk01, v2, v3);
  }
};

// Double-quantised block scales of row-major weights four steps at a time,
// for rows of a multiple of four blocks (K % 256 == 0): blocks 4k .. 4k + 3 of
// a row are then one aligned dword of absmax_q and fall in one group of 256
// (a row starts at a multiple of four blocks, a group at a multiple of 256),
// so a thread loads one dword and one group scale per four steps instead of a
// byte and a scale per step (each of those loads touches a cache line per row
// of the tile).  Row mapping as the row-major producer's.  `nxt` holds dword
// k + 1 while `cur` holds dword k.
struct Scale4 {
  rsrc_t rq, rs;
  uint32_t qoff;
  int64_t b0;   // first block of the thread's row
  uint32_t cur, nxt;
  float cur_s, nxt_s;

  __device__ void init(const QGemmArgs &a, int tid, int64_t n0) {
    const int row = ((tid >> 5) << 4) | (tid & 15);
    const int64_t nbr = a.Kc / 64;
    rq = make_rsrc(a.absmax_q + n0 * nbr, (a.Nout - n0) * nbr);
    rs = make_rsrc(a.scale2, (a.Nout * nbr + 255) / 256 * 4);
    qoff = n0 + row < a.Nout ? (uint32_t)(row * nbr) : kOutOfRange;
    b0 = (n0 + row) * nbr;
  }
  // Loads dword k (wave-uniform) into nxt.
  __device__ __forceinline__ void issue(int k) {
    nxt = __builtin_amdgcn_raw_buffer_load_b32(rq, qoff, 4 * k, 0);
    nxt_s = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
        rs, qoff == kOutOfRange ? kOutOfRange : (uint32_t)(((b0 + 4 * k) >> 8) * 4), 0, 0));
  }
  __device__ __forceinline__ static float scale(uint32_t w, float st, int byte) {
    return (float)((w >> (8 * byte)) & 0xFFu) * st;
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
template <bool KN>
__device__ __forceinline__ void store_adapter_right(const uint32_t (&h)[32], uint16_t *Rs, int t) {
  const int row = KN ? kn_row(t & (BN - 1)) : (t & (BN - 1)), j0 = 32 * (t >> 7);
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (h[2 * i] & 0xFFFFu) | (h[2 * i + 1] << 16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x4 *>(&Rs[row * LD + ((j0 + 8 * q) ^ wswz<KN>(row))]) = u32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
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
template <bool KN, bool DQ, bool EPI_NK, bool Q4>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qgemm_kernel(QGemmGroup grp, Code16 cb) {
  // The problem this workgroup belongs to (a grouped launch runs several
  // independent products; see QGemmGroup) and its tile index within it.
  int gi = 0;
#pragma unroll
  for (int i = 1; i < QN_MAX_GROUP; ++i) gi += (i < grp.n && (int)blockIdx.x >= grp.start[i]) ? 1 : 0;
  gi = __builtin_amdgcn_readfirstlane(gi);
  const QGemmArgs a = grp.p[gi];
  const int tile = (int)blockIdx.x - grp.start[gi];
  if (tile >= a.tiles_m * a.tiles_n) return;   // padding of the problem's range to a multiple of 8
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
  tile_coords(tile, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
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
    Producer<KN, DQ, Q4> P;
    P.init(a, tid, n0);
    typename Producer<KN, DQ, Q4>::Set s0, s1;
    Scale4 q4;
    if constexpr (Q4) q4.init(a, tid, n0);
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
    if constexpr (Q4) q4.issue(0);   // Scale4 dword 0, in nxt
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
    // With Scale4 (a code set reload is then the code load alone) the loop
    // runs four half-steps per iteration (nsteps is a multiple of 4): half-step
    // 4k + p takes byte p of dword k, and half-step 4k first moves dword k from
    // nxt to cur and loads dword k + 1 (two more loads before its stage t + 1,
    // counted in its wait).
    constexpr int kReload = Q4 ? 1 : (DQ ? 3 : 2);
    const int last4 = last >> 2;
    // The last half-step of an odd count (tail) reloads a set that nothing
    // reads again, and the compiler drops that load; its wait then counts only
    // the loads that remain after stage t (the previous reload and stage t + 1),
    // which is right whether or not the dead load survives.
    auto half = [&](auto phase, int t, typename Producer<KN, DQ, Q4>::Set &set, uint16_t *wdst,
                    bool tail = false) {   // t < nsteps
      constexpr int ph = decltype(phase)::value;
      constexpr int kScale = Q4 && ph == 0 ? 2 : 0;
      if constexpr (kScale) {
        q4.cur = q4.nxt;
        q4.cur_s = q4.nxt_s;
        q4.issue(__builtin_amdgcn_readfirstlane(min((t >> 2) + 1, last4)));
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (Q4)
        P.store_scaled(set, Scale4::scale(q4.cur, q4.cur_s, ph), wdst, pair, cb.v, lane,
                       [&](int q) { issue_x(t + 1, q); });
      else
        P.store(set, wdst, pair, cb.v, lane, [&](int q) { issue_x(t + 1, q); });
      __builtin_amdgcn_sched_barrier(0);
      P.issue(set, min(t + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      if (tail) __builtin_amdgcn_s_waitcnt(vmcnt_only(kReload + 8 + kScale));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(kReload + 8 + kScale + kReload));
      lds_barrier();
    };
    // Weight half-steps in pairs, then the odd one out.  Neither an exit from
    // the middle of the loop body nor a branch between two arms that both
    // load: the compiler gives such control flow a path that skips the loads
    // (or leaves the loop body early), and its wait counts then assume that
    // path and wait for loads that are still a half-step early.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int t = 0;
    if constexpr (Q4) {
      using P2 = std::integral_constant<int, 2>;
      using P3 = std::integral_constant<int, 3>;
      for (; t + 4 <= nsteps; t += 4) {
        half(P0{}, t, s0, ws0);
        half(P1{}, t + 1, s1, ws1);
        half(P2{}, t + 2, s0, ws0);
        half(P3{}, t + 3, s1, ws1);
      }
    } else {
      for (; t + 2 <= nsteps; t += 2) {
        half(P0{}, t, s0, ws0);
        half(P1{}, t + 1, s1, ws1);
      }
      if (t < nsteps) {
        half(P0{}, t, s0, ws0, true);
        ++t;
      }
    }
    // Half-step nsteps: the adapter's right operand; its left operand is
    // activation stage nsteps, issued in the last weight half-step.
    store_adapter_right<KN>(adapter, (t & 1) ? ws1 : ws0, tid);
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
  // B (weights) stage row 32j + lr, positions 32lh + 8c .. +7, stored there (forward) or
  // at (32lh + 8c) ^ kswz(32j + lr) (dX).
  uint32_t aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = (uint32_t)(wave_u * XW + lr * BK + (((4 * lh + c) ^ ((lr >> 1) & 7)) * 8));
  const int rb = lr * LD + (KN ? 0 : 32 * lh);
  int bpos[TN];   // dX: position base of tile j, before the slice's 8c
#pragma unroll
  for (int j = 0; j < TN; ++j) bpos[j] = KN ? ((32 * lh) ^ kswz(32 * j + lr)) : 0;
  struct Frag {
    bf16x8 a[TM];
    bf16x8 b[TN];
  };
  auto read_b = [&](bf16x8 *b, const uint16_t *wc, int c) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const bf16x8 *>(&wc[rb + j * 32 * LD + (KN ? (bpos[j] ^ (8 * c)) : 8 * c)]);
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
      const int64_t lrow = (int64_t)wave_u * WM + i * 32 + row, gn = n0 + (KN ? kn_col(c8) : c8);
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

// ============================================================ 256 x 256 tiles
// Second tiling of the forward product (row-major weights): a workgroup
// computes a 256 x 256 output tile with 8 waves, two per SIMD, and every wave
// both multiplies and dequantises.  Wave w owns rows 64 (w & 3) .. +63 and
// columns 128 (w >> 2) .. +127 of the tile (2 x 4 MFMA tiles of 32 x 32, as an
// MMA wave above), and the 512 threads together dequantise the 256 x 64
// weight stage of the next step (thread t: the producer row and half of the
// tiling above, over 256 rows) while the MFMAs of the current step run on the
// matrix cores.  Against the 256 x 128 tile, the activation rows staged per
// step serve twice the columns (half the activation traffic per FLOP), and the
// dequantisation sits in the same instruction streams as the MFMAs of two
// waves per SIMD instead of in one producer wave per SIMD, so the matrix cores
// and the vector units overlap without a producer wave setting the pace.
//
// LDS: two activation stages (256 rows x 64, XOR-swizzled as above, 32 KB
// each) and two weight stages (256 columns x LD, 36 KB each): one step ahead.
// Step s reads activation stage s & 1 and weight stage s & 1; during it the
// waves issue the direct-to-LDS loads of activation step s + 1, write weight
// step s + 1 from the register set loaded two steps earlier and reload that set
// for step s + 3; one barrier per step.  The adapter term is one more step
// whose left operand (H or sH, zero beyond ldl2) comes through the activation
// stage and whose right operand (B, zero beyond r) is loaded after the main
// loop and written as the weight stage.
constexpr int kThreads2 = 512;
constexpr int BM2 = 256, BN2 = 256;
constexpr int R_TILE2 = BN2 * LD;
constexpr int XSTAGE2 = BM2 * BK;

template <bool DQ, bool Q4, bool KN>
__global__ __launch_bounds__(kThreads2, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qgemm2_kernel(QGemmGroup grp, Code16 cb) {
  static_assert(!(KN && Q4), "four-step scales are for row-major weights");
  int gi = 0;
#pragma unroll
  for (int i = 1; i < QN_MAX_GROUP; ++i) gi += (i < grp.n && (int)blockIdx.x >= grp.start[i]) ? 1 : 0;
  gi = __builtin_amdgcn_readfirstlane(gi);
  const QGemmArgs a = grp.p[gi];
  const int tile = (int)blockIdx.x - grp.start[gi];
  if (tile >= a.tiles_m * a.tiles_n) return;

  __shared__ __attribute__((aligned(16))) uint16_t xs0[XSTAGE2];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[XSTAGE2];
  __shared__ __attribute__((aligned(16))) uint16_t ws0[R_TILE2];
  __shared__ __attribute__((aligned(16))) uint16_t ws1[R_TILE2];
  // Byte -> (row lo, row hi) table of the transposed-weight expansion (dX).
  __shared__ __attribute__((aligned(16))) float2 pair[KN ? 256 * kPairCopies : 1];
  if constexpr (KN) {
    for (int i = threadIdx.x; i < 256 * kPairCopies; i += kThreads2) {
      const int e = i / kPairCopies;
      pair[i] = make_float2(cb.v[e & 15], cb.v[e >> 4]);
    }
    lds_barrier();
  }

  int tm, tn;
  tile_coords(tile, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * BM2, n0 = (int64_t)tn * BN2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3, cg = wave >> 2;
  const int nsteps = __builtin_amdgcn_readfirstlane((int)(a.Kc / BK));   // >= 1
  const int last = nsteps - 1, ntotal = nsteps + 1;

  // ---- activation stages: wave w loads rows 32 cg .. +31 of row group rg
  // (loads g = 4 cg .. 4 cg + 3 of that group's eight 8-row loads; chunk
  // swizzle and lane layout as in the tiling above).
  const int64_t grow0 = m0 + (int64_t)rg * WM;
  const rsrc_t xr = make_rsrc(a.L + grow0 * a.ldl, (a.M - grow0) * a.ldl * 2);
  const rsrc_t l2r = make_rsrc(a.L2 + grow0 * a.ldl2, (a.M - grow0) * a.ldl2 * 2);
  const uint32_t c0 = (uint32_t)((lane & 7) ^ (lane >> 4));
  const uint32_t xbase0 = (uint32_t)((lane >> 3) * a.ldl * 2 + c0 * 16);
  const uint32_t xbase1 = (uint32_t)((lane >> 3) * a.ldl * 2 + (c0 ^ 4u) * 16);
  const uint32_t xrow8 = (uint32_t)(8 * a.ldl * 2);
  const uint32_t l2base0 = (uint32_t)((lane >> 3) * a.ldl2 * 2 + c0 * 16);
  const uint32_t l2base1 = (uint32_t)((lane >> 3) * a.ldl2 * 2 + (c0 ^ 4u) * 16);
  const bool l2ok0 = 8 * (int64_t)c0 < a.ldl2, l2ok1 = 8 * (int64_t)(c0 ^ 4u) < a.ldl2;
  const uint32_t l2row8 = (uint32_t)(8 * a.ldl2 * 2);
  auto issue_x = [&](uint16_t *stage, int t) {
    const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(stage + rg * XW));
    const bool main_step = t < nsteps, live = t < ntotal;
    const rsrc_t r = main_step ? xr : l2r;
    const int soff = main_step ? t * BK * 2 : 0;
#pragma unroll
    for (int g = 4 * cg; g < 4 * cg + 4; ++g) {
      const bool odd = g & 1;
      const uint32_t l2off =
          live && (odd ? l2ok1 : l2ok0) ? (odd ? l2base1 : l2base0) + (uint32_t)g * l2row8 : kOutOfRange;
      const uint32_t off = main_step ? (odd ? xbase1 : xbase0) + (uint32_t)g * xrow8 : l2off;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(size_t)(base + g * 1024),
                                               16, off, soff, 0, 0);
    }
  };

  // ---- weight stages: the producer of the tiling above, over 256 rows.
  Producer<KN, DQ, Q4> P;
  P.init(a, tid, n0);
  typename Producer<KN, DQ, Q4>::Set s0, s1;
  Scale4 q4;
  if constexpr (Q4) q4.init(a, tid, n0);

  // ---- fragments
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = (uint32_t)(rg * XW + lr * BK + (((4 * lh + c) ^ ((lr >> 1) & 7)) * 8));
  // Weights: stage row 128 cg + 32 j + lr, positions 32 lh + 8 c .. +7, stored
  // there (row-major) or at (32 lh + 8 c) ^ kswz(32 j + lr) (dX: kswz depends
  // on bits 4 and 5 of the stage row only).
  const int rb = (128 * cg + lr) * LD + (KN ? 0 : 32 * lh);
  int bpos[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bpos[j] = KN ? ((32 * lh) ^ kswz(32 * j + lr)) : 0;
  struct Frag {
    bf16x8 a[TM];
    bf16x8 b[TN];
  };
  auto read_f = [&](Frag &f, const uint16_t *xc, const uint16_t *wc, int c) {
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const bf16x8 *>(&xc[aoff[c] + i * 32 * BK]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8 *>(&wc[rb + j * 32 * LD + (KN ? (bpos[j] ^ (8 * c)) : 8 * c)]);
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // ---- prologue: code sets of steps 0 and 1, activation stage 0, weight stage 0
  // (with Scale4: its dword 0 first, in nxt).
  // The scheduling fences keep the loads in this order, which the wait before
  // the barrier counts on: only the two code-set reloads issued after stage 0
  // may still be in flight there (unfenced, the compiler had moved the second
  // reload between stage 0's loads, and the barrier could pass before that
  // stage had landed).
  constexpr int kReload = Q4 ? 1 : (DQ ? 3 : 2);   // loads per code-set reload
  if constexpr (Q4) q4.issue(0);
  P.issue(s0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_x(xs0, 0);
  __builtin_amdgcn_sched_barrier(0);
  P.issue(s1, __builtin_amdgcn_readfirstlane(min(1, last)));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (Q4) P.store_scaled(s0, Scale4::scale(q4.nxt, q4.nxt_s, 0), ws0, nullptr, cb.v, lane, [&](int) {});
  else P.store(s0, ws0, KN ? pair : nullptr, cb.v, lane, [&](int) {});
  P.issue(s0, __builtin_amdgcn_readfirstlane(min(2, last)));
  __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kReload));
  lds_barrier();

  // Step s: multiply stage s while staging step s + 1 (its activations by
  // direct-to-LDS loads, its weights from register set `set`), then reload the
  // set for step s + 3 (clamped: past the end it re-reads the last step, whose
  // stage the adapter operand later replaces).  The dequantisation runs one
  // k-slice behind the MFMAs in the same instruction stream: the MFMAs of
  // slice 0 go with building the block's sixteen products, those of slice c
  // (c = 1..3) with expanding code word c - 1, and the scheduling groups below
  // alternate one MFMA with a few vector instructions, so that each wave keeps
  // the matrix core busy while it dequantises (the two waves of a SIMD start
  // every step together, so they cannot cover for each other).
  const uint16_t *wrow = nullptr;
  (void)wrow;
  // With Scale4 the loop runs four steps per iteration (nsteps is then a
  // multiple of 4): step 4k + p writes the stage of block 4k + p + 1, whose
  // scale is byte p + 1 of dword k (cur) for p < 3 and byte 0 of dword k + 1
  // (nxt, loaded at step 4k) for p = 3.
  const int wcol = P.wr_col, wk = P.wr_k;
  const int wsw = wswz<false>(wcol);
  const int last4 = last >> 2;
  auto step = [&](auto phase, int s, const uint16_t *xc, const uint16_t *wc, uint16_t *xn, uint16_t *wn,
                  typename Producer<KN, DQ, Q4>::Set &set) {
    constexpr int ph = decltype(phase)::value;
    issue_x(xn, s + 1);
    if constexpr (Q4 && ph == 0) {
      q4.cur = q4.nxt;
      q4.cur_s = q4.nxt_s;
      q4.issue(__builtin_amdgcn_readfirstlane(min((s >> 2) + 1, last4)));
    }
    if constexpr (KN) {
      // Transposed weights (dX): the producer of the 256 x 128 tiling, its
      // work spread over the four k-slices.  Slice 0 goes with the quad
      // transpose of the code words and the four rows' scales, slices 1 to 3
      // with the table lookups of the patch's rows, and the patch is written
      // transposed after the last slice.
      Frag f0, f1;
      read_f(f0, xc, wc, 0);
      read_f(f1, xc, wc, 1);
      uint32_t wv[4];
      float S[4];
      P.patch_prep(set, P.scale(set), lane, wv, S);
      mma(f0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      read_f(f0, xc, wc, 2);
      __builtin_amdgcn_sched_barrier(0);
      const int copy = lane & (kPairCopies - 1);
      float v[4][8];
      auto lookrow = [&](int i) { P.patch_row(wv, S, i, pair, copy, v[i]); };
      // slice 1 + rows 0 and 1
      mma(f1);
      lookrow(0);
      lookrow(1);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      read_f(f1, xc, wc, 3);
      __builtin_amdgcn_sched_barrier(0);
      // slice 2 + rows 0 and 1 packed, row 2
      mma(f0);
      uint32_t pk01[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) pk01[c] = pack_bf16x2(v[0][c], v[1][c]);
      lookrow(2);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 3 + row 3
      mma(f1);
      lookrow(3);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      P.write_patch(wn, pk01, v[2], v[3]);
      __builtin_amdgcn_sched_barrier(0);
      P.issue(set, __builtin_amdgcn_readfirstlane(min(s + 3, last)));
      __builtin_amdgcn_s_waitcnt(vmcnt_only(kReload));
      lds_barrier();
      return;
    }
    Frag f0, f1;
    read_f(f0, xc, wc, 0);
    read_f(f1, xc, wc, 1);
    uint32_t LO[4], HI[4];
    // slice 0 + the block's products
    {
      float A;
      if constexpr (Q4) A = ph == 3 ? Scale4::scale(q4.nxt, q4.nxt_s, 0) : Scale4::scale(q4.cur, q4.cur_s, ph + 1);
      else A = P.scale(set);
      uint32_t Pp[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) Pp[k] = pack_bf16x2(cb.v[2 * k] * A, cb.v[2 * k + 1] * A);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        LO[m] = __builtin_amdgcn_perm(Pp[2 * m + 1], Pp[2 * m], 0x06040200u);
        HI[m] = __builtin_amdgcn_perm(Pp[2 * m + 1], Pp[2 * m], 0x07050301u);
      }
      mma(f0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    read_f(f0, xc, wc, 2);
    __builtin_amdgcn_sched_barrier(0);
    auto look = [&](uint32_t x, uint32_t &lo, uint32_t &hi) {
      const uint32_t s7 = x & 0x07070707u;
      const u16x2 bit3 = __builtin_bit_cast(u16x2, (x >> 3) & 0x01010101u);
      const uint32_t upper = __builtin_bit_cast(uint32_t, bit3 * (u16x2){0xFF, 0xFF});
      const uint32_t l0 = __builtin_amdgcn_perm(LO[1], LO[0], s7), l1 = __builtin_amdgcn_perm(LO[3], LO[2], s7);
      const uint32_t h0 = __builtin_amdgcn_perm(HI[1], HI[0], s7), h1 = __builtin_amdgcn_perm(HI[3], HI[2], s7);
      lo = (upper & l1) | (~upper & l0);
      hi = (upper & h1) | (~upper & h0);
    };
    auto word = [&](int i) {
      const uint32_t w = set.code[i], w4 = w >> 4;
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t lo, hi;
        look(__builtin_amdgcn_perm(w4, w, h ? 0x07030602u : 0x05010400u), lo, hi);
        o[2 * h + 0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
        o[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
      }
      *reinterpret_cast<u32x4 *>(&wn[wcol * LD + ((wk + 8 * i) ^ wsw)]) = u32x4{o[0], o[1], o[2], o[3]};
    };
    // slice 1 + word 0
    mma(f1);
    word(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    read_f(f1, xc, wc, 3);
    __builtin_amdgcn_sched_barrier(0);
    // slice 2 + word 1
    mma(f0);
    word(1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    // slice 3 + word 2
    mma(f1);
    word(2);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    word(3);
    __builtin_amdgcn_sched_barrier(0);
    P.issue(set, __builtin_amdgcn_readfirstlane(min(s + 3, last)));
    __builtin_amdgcn_s_waitcnt(vmcnt_only(kReload));
    lds_barrier();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int s = 0;
  if constexpr (Q4) {
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    for (; s + 4 <= nsteps; s += 4) {
      step(P0{}, s, xs0, ws0, xs1, ws1, s1);
      step(P1{}, s + 1, xs1, ws1, xs0, ws0, s0);
      step(P2{}, s + 2, xs0, ws0, xs1, ws1, s1);
      step(P3{}, s + 3, xs1, ws1, xs0, ws0, s0);
    }
  } else {
    for (; s + 2 <= nsteps; s += 2) {
      step(P0{}, s, xs0, ws0, xs1, ws1, s1);
      step(P1{}, s + 1, xs1, ws1, xs0, ws0, s0);
    }
    if (s < nsteps) {
      step(P0{}, s, xs0, ws0, xs1, ws1, s1);
      ++s;
    }
  }
  // ---- adapter step: left operand in activation stage nsteps & 1 (loaded by
  // the last step); right operand B (zero beyond r) into weight stage nsteps & 1.
  uint16_t *xa = (nsteps & 1) ? xs1 : xs0;
  uint16_t *wa = (nsteps & 1) ? ws1 : ws0;
  {
    const int col = tid & (BN2 - 1), j0 = 32 * (tid >> 8);
    const int64_t gn = n0 + col;
    // B is [Nout, r]; for dX the operand is A, [r, Nout], into stage row kn_row(col).
    const rsrc_t rr = make_rsrc(a.R2, KN ? a.r * a.ldr2 * 2 : a.Nout * a.ldr2 * 2);
    uint32_t h[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int64_t j = j0 + i;
      const bool in = j < a.r && gn < a.Nout;
      const int64_t e = KN ? j * a.ldr2 + gn : gn * a.ldr2 + j;
      h[i] = __builtin_amdgcn_raw_buffer_load_b16(rr, in ? (uint32_t)(e * 2) : kOutOfRange, 0, 0);
    }
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (h[2 * i] & 0xFFFFu) | (h[2 * i + 1] << 16);
    const int srow = KN ? kn_row(col) : col;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4 *>(&wa[srow * LD + ((j0 + 8 * q) ^ wswz<KN>(srow))]) = u32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  lds_barrier();
  {
    Frag f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      read_f(f, xa, wa, c);
      mma(f);
    }
  }
  lds_barrier();

  // ---- store bf16 through LDS, one 32 x 128 block per wave at a time (the
  // layout and the 16-byte row stores of the tiling above); a wave reuses its
  // own block region, so the two passes need no barrier between them.
  constexpr int kOutPitch = BN + 8;
  const rsrc_t rout = make_rsrc(a.out + m0 * a.ldo, (a.M - m0) * a.ldo * 2);
  const bool vec_ok = (a.ldo & 7) == 0 && ((uint64_t)a.out & 15) == 0;
  uint16_t *blk = (wave < 3 ? xs0 : (wave < 6 ? xs1 : ws0)) + (wave < 6 ? wave % 3 : wave - 6) * 32 * kOutPitch;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        blk[(8 * (e >> 2) + 4 * lh + (e & 3)) * kOutPitch + j * 32 + lr] = f32_to_bf16(acc[i][j][e]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 4 * q + (lane >> 4), c8 = 8 * (lane & 15);
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&blk[row * kOutPitch + c8]);
      const int64_t lrow = (int64_t)rg * WM + i * 32 + row, gn = n0 + (KN ? kn_col(128 * cg + c8) : 128 * cg + c8);
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

// ============================================================ 256 x 256, 4 waves
// Third tiling of the forward product: the same 256 x 256 output tile with
// four waves, one per SIMD, each owning 128 x 128 (4 x 4 MFMA tiles of 32 x 32,
// the accumulators in the accumulation registers).  A wave's fragment reads
// per step are (128 + 128) x 64 values for 128 x 128 x 64 multiply-adds, a
// third less LDS read traffic per FLOP than 64 x 128 per wave, and each k-slice
// gives a wave sixteen MFMAs (512 matrix-core cycles) behind which it issues
// the next slice's fragment reads and its share of the dequantisation.
// Thread t dequantises weight row t of the tile: the 64 codes of a step are one
// NF4 block (one scale, one table of products), 32 bytes read as two 16-byte
// loads; they are written as eight 16-byte chunks of the swizzled weight stage.
constexpr int kThreads3 = 256;
constexpr int TM3 = 4, TN3 = 4;

template <bool DQ>
struct RowProducer {
  struct Set {
    u32x4 c0, c1;   // 64 codes of one row, one step
    uint32_t q;
    float st;
  };
  rsrc_t rc, rq, rs;
  uint32_t cvoff, qvoff;
  int64_t blk_base;
  int row;
  __device__ void init(const QGemmArgs &a, int tid, int64_t n0) {
    row = tid;
    rc = make_rsrc(a.codes + n0 * (a.Kc / 2), (a.Nout - n0) * (a.Kc / 2));
    cvoff = (uint32_t)(row * (a.Kc / 2));
    blk_base = (n0 + row) * (a.Kc / 64);
    if constexpr (DQ) {
      rq = make_rsrc(a.absmax_q + n0 * (a.Kc / 64), (a.Nout - n0) * (a.Kc / 64));
      qvoff = (uint32_t)(row * (a.Kc / 64));
      rs = make_rsrc(a.scale2, (a.Nout * a.Kc / 64 + 255) / 256 * 4);
    } else {
      rq = make_rsrc(a.absmax + n0 * (a.Kc / 64), (a.Nout - n0) * (a.Kc / 64) * 4);
      qvoff = (uint32_t)(row * (a.Kc / 64) * 4);
    }
    if (n0 + row >= a.Nout) cvoff = qvoff = kOutOfRange;
  }
  __device__ __forceinline__ void issue(Set &t, int s) {
    t.c0 = __builtin_amdgcn_raw_buffer_load_b128(rc, cvoff, s * (BK / 2), 0);
    t.c1 = __builtin_amdgcn_raw_buffer_load_b128(rc, cvoff == kOutOfRange ? kOutOfRange : cvoff + 16, s * (BK / 2), 0);
    if constexpr (DQ) {
      t.q = __builtin_amdgcn_raw_buffer_load_b8(rq, qvoff, s, 0);
      const int64_t b = blk_base + s;
      t.st = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
          rs, qvoff == kOutOfRange ? kOutOfRange : (uint32_t)((b >> 8) * 4), 0, 0));
    } else {
      t.q = __builtin_amdgcn_raw_buffer_load_b32(rq, qvoff, s * 4, 0);
    }
  }
  __device__ __forceinline__ float scale(const Set &t) const {
    if constexpr (DQ) return (float)t.q * t.st;
    else return as_f32(t.q);
  }
};

template <bool DQ>
__global__ __launch_bounds__(kThreads3, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void qgemm3_kernel(QGemmGroup grp, Code16 cb) {
  int gi = 0;
#pragma unroll
  for (int i = 1; i < QN_MAX_GROUP; ++i) gi += (i < grp.n && (int)blockIdx.x >= grp.start[i]) ? 1 : 0;
  gi = __builtin_amdgcn_readfirstlane(gi);
  const QGemmArgs a = grp.p[gi];
  const int tile = (int)blockIdx.x - grp.start[gi];
  if (tile >= a.tiles_m * a.tiles_n) return;

  __shared__ __attribute__((aligned(16))) uint16_t xs0[XSTAGE2];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[XSTAGE2];
  __shared__ __attribute__((aligned(16))) uint16_t ws0[R_TILE2];
  __shared__ __attribute__((aligned(16))) uint16_t ws1[R_TILE2];

  int tm, tn;
  tile_coords(tile, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * BM2, n0 = (int64_t)tn * BN2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave & 1, ch = wave >> 1;       // rows 128 rh .., columns 128 ch ..
  const int nsteps = __builtin_amdgcn_readfirstlane((int)(a.Kc / BK));   // >= 1
  const int last = nsteps - 1, ntotal = nsteps + 1;

  // ---- activation stages: wave w loads the 64 rows of row block w (eight
  // 8-row loads, chunk swizzle and lane layout of the first tiling).
  const int64_t grow0 = m0 + (int64_t)wave * WM;
  const rsrc_t xr = make_rsrc(a.L + grow0 * a.ldl, (a.M - grow0) * a.ldl * 2);
  const rsrc_t l2r = make_rsrc(a.L2 + grow0 * a.ldl2, (a.M - grow0) * a.ldl2 * 2);
  const uint32_t c0 = (uint32_t)((lane & 7) ^ (lane >> 4));
  const uint32_t xbase0 = (uint32_t)((lane >> 3) * a.ldl * 2 + c0 * 16);
  const uint32_t xbase1 = (uint32_t)((lane >> 3) * a.ldl * 2 + (c0 ^ 4u) * 16);
  const uint32_t xrow8 = (uint32_t)(8 * a.ldl * 2);
  const uint32_t l2base0 = (uint32_t)((lane >> 3) * a.ldl2 * 2 + c0 * 16);
  const uint32_t l2base1 = (uint32_t)((lane >> 3) * a.ldl2 * 2 + (c0 ^ 4u) * 16);
  const bool l2ok0 = 8 * (int64_t)c0 < a.ldl2, l2ok1 = 8 * (int64_t)(c0 ^ 4u) < a.ldl2;
  const uint32_t l2row8 = (uint32_t)(8 * a.ldl2 * 2);
  auto issue_x = [&](uint16_t *stage, int t) {
    const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(stage + wave * XW));
    const bool main_step = t < nsteps, live = t < ntotal;
    const rsrc_t r = main_step ? xr : l2r;
    const int soff = main_step ? t * BK * 2 : 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const bool odd = g & 1;
      const uint32_t l2off =
          live && (odd ? l2ok1 : l2ok0) ? (odd ? l2base1 : l2base0) + (uint32_t)g * l2row8 : kOutOfRange;
      const uint32_t off = main_step ? (odd ? xbase1 : xbase0) + (uint32_t)g * xrow8 : l2off;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(size_t)(base + g * 1024),
                                               16, off, soff, 0, 0);
    }
  };

  RowProducer<DQ> P;
  P.init(a, tid, n0);
  typename RowProducer<DQ>::Set s0, s1;
  const int wsw = wswz<false>(tid);

  // ---- fragments: A row tile i of the wave is rows 128 rh + 32 i + lr (row
  // block 2 rh + i / 2); B column tile j is column 128 ch + 32 j + lr.
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = (uint32_t)(2 * rh * XW + lr * BK + (((4 * lh + c) ^ ((lr >> 1) & 7)) * 8));
  const int rb = (128 * ch + lr) * LD + 32 * lh;
  struct Frag {
    bf16x8 a[TM3];
    bf16x8 b[TN3];
  };
  auto read_f = [&](Frag &f, const uint16_t *xc, const uint16_t *wc, int c) {
#pragma unroll
    for (int i = 0; i < TM3; ++i) f.a[i] = *reinterpret_cast<const bf16x8 *>(&xc[aoff[c] + i * 32 * BK]);
#pragma unroll
    for (int j = 0; j < TN3; ++j) f.b[j] = *reinterpret_cast<const bf16x8 *>(&wc[rb + j * 32 * LD + 8 * c]);
  };
  f32x16 acc[TM3][TN3];
#pragma unroll
  for (int i = 0; i < TM3; ++i)
#pragma unroll
    for (int j = 0; j < TN3; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mma = [&](const Frag &f) {
#pragma unroll
    for (int i = 0; i < TM3; ++i)
#pragma unroll
      for (int j = 0; j < TN3; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // Dequantise one row-step: the block's sixteen bf16 products, split into
  // low-byte and high-byte planes, looked up four codes at a time with byte
  // permutes (as the first tiling's producer), written as 16-byte chunks.
  uint32_t LO[4], HI[4];
  auto prep = [&](const typename RowProducer<DQ>::Set &t) {
    const float A = P.scale(t);
    uint32_t Pp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) Pp[k] = pack_bf16x2(cb.v[2 * k] * A, cb.v[2 * k + 1] * A);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      LO[m] = __builtin_amdgcn_perm(Pp[2 * m + 1], Pp[2 * m], 0x06040200u);
      HI[m] = __builtin_amdgcn_perm(Pp[2 * m + 1], Pp[2 * m], 0x07050301u);
    }
  };
  auto look = [&](uint32_t x, uint32_t &lo, uint32_t &hi) {
    const uint32_t s7 = x & 0x07070707u;
    const u16x2 bit3 = __builtin_bit_cast(u16x2, (x >> 3) & 0x01010101u);
    const uint32_t upper = __builtin_bit_cast(uint32_t, bit3 * (u16x2){0xFF, 0xFF});
    const uint32_t l0 = __builtin_amdgcn_perm(LO[1], LO[0], s7), l1 = __builtin_amdgcn_perm(LO[3], LO[2], s7);
    const uint32_t h0 = __builtin_amdgcn_perm(HI[1], HI[0], s7), h1 = __builtin_amdgcn_perm(HI[3], HI[2], s7);
    lo = (upper & l1) | (~upper & l0);
    hi = (upper & h1) | (~upper & h0);
  };
  // code word i (0..7) of the row-step: positions 8 i .. 8 i + 7
  auto word = [&](const typename RowProducer<DQ>::Set &t, int i, uint16_t *wn) {
    const uint32_t cw[8] = {t.c0.x, t.c0.y, t.c0.z, t.c0.w, t.c1.x, t.c1.y, t.c1.z, t.c1.w};
    const uint32_t w = cw[i], w4 = w >> 4;
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t lo, hi;
      look(__builtin_amdgcn_perm(w4, w, h ? 0x07030602u : 0x05010400u), lo, hi);
      o[2 * h + 0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
      o[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
    *reinterpret_cast<u32x4 *>(&wn[tid * LD + ((8 * i) ^ wsw)]) = u32x4{o[0], o[1], o[2], o[3]};
  };

  // ---- prologue
  // Fenced so that the wait before the barrier covers stage 0 (see the
  // 8-wave tiling's prologue).
  constexpr int kReload3 = DQ ? 4 : 3;
  P.issue(s0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_x(xs0, 0);
  __builtin_amdgcn_sched_barrier(0);
  P.issue(s1, __builtin_amdgcn_readfirstlane(min(1, last)));
  __builtin_amdgcn_sched_barrier(0);
  prep(s0);
#pragma unroll
  for (int i = 0; i < 8; ++i) word(s0, i, ws0);
  P.issue(s0, __builtin_amdgcn_readfirstlane(min(2, last)));
  __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kReload3));
  lds_barrier();

  // Step s: four k-slices of sixteen MFMAs; slice c goes with two code words
  // of step s + 1 (slice 0 also with building the products) and the fragment
  // reads of slice c + 1.
  auto step = [&](int s, const uint16_t *xc, const uint16_t *wc, uint16_t *xn, uint16_t *wn,
                  typename RowProducer<DQ>::Set &set) {
    issue_x(xn, s + 1);
    Frag f0, f1;
    read_f(f0, xc, wc, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Frag &cur = (c & 1) ? f1 : f0;
      Frag &nxt = (c & 1) ? f0 : f1;
      if (c < 3) read_f(nxt, xc, wc, c + 1);
      mma(cur);
      if (c == 0) prep(set);
      word(set, 2 * c, wn);
      word(set, 2 * c + 1, wn);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    P.issue(set, __builtin_amdgcn_readfirstlane(min(s + 3, last)));
    __builtin_amdgcn_s_waitcnt(vmcnt_only(kReload3));
    lds_barrier();
  };
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    step(s, xs0, ws0, xs1, ws1, s1);
    step(s + 1, xs1, ws1, xs0, ws0, s0);
  }
  if (s < nsteps) {
    step(s, xs0, ws0, xs1, ws1, s1);
    ++s;
  }
  // ---- adapter step: left operand in activation stage nsteps & 1; right
  // operand row t of B (positions j < r, zero beyond) into weight stage
  // nsteps & 1, eight 16-byte chunks per thread.
  uint16_t *xa = (nsteps & 1) ? xs1 : xs0;
  uint16_t *wa = (nsteps & 1) ? ws1 : ws0;
  {
    const int64_t gn = n0 + tid;
    const rsrc_t rr = make_rsrc(a.R2, a.Nout * a.ldr2 * 2);
    const bool vec = (a.r % 8) == 0 && (a.ldr2 % 8) == 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t v[16];
      if (vec) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t j = 32 * half + 8 * q;
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
              rr, (j < a.r && gn < a.Nout) ? (uint32_t)((gn * a.ldr2 + j) * 2) : kOutOfRange, 0, 0);
          v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
        }
      } else {
        uint32_t h[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int64_t j = 32 * half + i;
          h[i] = __builtin_amdgcn_raw_buffer_load_b16(
              rr, (j < a.r && gn < a.Nout) ? (uint32_t)((gn * a.ldr2 + j) * 2) : kOutOfRange, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = (h[2 * i] & 0xFFFFu) | (h[2 * i + 1] << 16);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4 *>(&wa[tid * LD + ((32 * half + 8 * q) ^ wsw)]) =
            u32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  lds_barrier();
  {
    Frag f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      read_f(f, xa, wa, c);
      mma(f);
    }
  }
  lds_barrier();

  // ---- store bf16 through LDS, one 32 x 128 block per wave at a time.
  constexpr int kOutPitch = BN + 8;
  const rsrc_t rout = make_rsrc(a.out + m0 * a.ldo, (a.M - m0) * a.ldo * 2);
  const bool vec_ok = (a.ldo & 7) == 0 && ((uint64_t)a.out & 15) == 0;
  uint16_t *blk = xs0 + wave * 32 * kOutPitch;
#pragma unroll
  for (int i = 0; i < TM3; ++i) {
#pragma unroll
    for (int j = 0; j < TN3; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        blk[(8 * (e >> 2) + 4 * lh + (e & 3)) * kOutPitch + j * 32 + lr] = f32_to_bf16(acc[i][j][e]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 4 * q + (lane >> 4), c8 = 8 * (lane & 15);
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&blk[row * kOutPitch + c8]);
      const int64_t lrow = (int64_t)rh * 128 + i * 32 + row, gn = n0 + 128 * ch + c8;
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

// Tiles, and the row-tile group size of the XCD-aware order.  Each XCD runs a
// contiguous run of T/8 logical tiles, and about CUs/8 of them at once (one
// workgroup per CU); the tiles running together walk the contraction at about
// the same pace, so the XCD's L2 serves each activation row-panel and weight
// column-panel they share.  The group size g (row tiles per group) is chosen
// for that concurrent set: g row panels (bm x 2 bytes per contraction index)
// plus R/g column panels (bn / 2 bytes) for R = CUs/8 tiles, as few bytes as
// possible.
bool plan(QGemmArgs &a, int bm = BM, int bn = BN) {
  // The adapter term is exactly one extra contraction step, and the producer
  // and MMA waves count their barriers on that: reject any other rank here.
  if (a.r < 1 || a.r > BK || a.Kc < BK || a.Kc % BK != 0) return false;
  a.tiles_m = (int)cdiv(a.M, bm);
  a.tiles_n = (int)cdiv(a.Nout, bn);
  const int R = std::max(1, std::min(a.tiles_m * a.tiles_n / 8, device_cus() / 8));
  int best = 1;
  double best_cost = 1e300;
  for (int g = 1; g <= a.tiles_m; ++g) {
    const int cols = std::max(1, std::min(a.tiles_n, (R + g - 1) / g));
    const double cost = (double)std::min(g, R) * bm * 2 + (double)cols * bn / 2;
    if (cost < best_cost * (1.0 - 1e-9)) { best_cost = cost; best = g; }
  }
  a.group_m = best;
  return true;
}

// One launch over n problems.  Problems with the longest contraction (the
// most work per tile) are dispatched first, so that short tiles fill in at
// the end; each problem's workgroup range is rounded up to a multiple of 8 so
// that the XCD-aware order within it holds (workgroups are dealt to the XCDs
// round-robin by their global index).
std::atomic<int> g_variant{0};   // 0 automatic, 1 256 x 128, 2 256 x 256 (8 waves), 3 256 x 256 (4 waves)

// One launch of one tiling over n problems (wide: 256 x 256; dX has only the 8-wave one).
template <bool KN, bool EPI_NK>
hipError_t launch_tiling(const QGemmArgs *in, int n, bool wide, int wide_kind, hipStream_t st) {
  const int bm = wide ? BM2 : BM, bn = wide ? BN2 : BN;
  QGemmGroup grp{};
  int order[QN_MAX_GROUP];
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order, order + n, [&](int x, int y) { return in[x].Kc > in[y].Kc; });
  const bool dq = in[0].absmax_q != nullptr;
  int64_t total = 0;
  for (int k = 0; k < n; ++k) {
    QGemmArgs a = in[order[k]];
    if ((a.absmax_q != nullptr) != dq || a.qtype != in[0].qtype || !plan(a, bm, bn)) return hipErrorInvalidValue;
    grp.p[k] = a;
    grp.start[k] = (int)total;
    total += (int64_t)((a.tiles_m * a.tiles_n + 7) / 8) * 8;
  }
  if (total > INT32_MAX) return hipErrorInvalidValue;
  for (int k = n; k <= QN_MAX_GROUP; ++k) grp.start[k] = (int)total;
  grp.n = n;
  const dim3 grid((unsigned)total);
  if constexpr (KN) {
    if (wide) {   // dX: the 8-wave 256 x 256 tiling
      if (dq) hipLaunchKernelGGL((qgemm2_kernel<true, false, true>), grid, dim3(kThreads2), 0, st, grp, code16(in[0].qtype));
      else hipLaunchKernelGGL((qgemm2_kernel<false, false, true>), grid, dim3(kThreads2), 0, st, grp, code16(in[0].qtype));
      return hipGetLastError();
    }
  } else {
    if (wide && wide_kind == 3) {
      if (dq) hipLaunchKernelGGL((qgemm3_kernel<true>), grid, dim3(kThreads3), 0, st, grp, code16(in[0].qtype));
      else hipLaunchKernelGGL((qgemm3_kernel<false>), grid, dim3(kThreads3), 0, st, grp, code16(in[0].qtype));
      return hipGetLastError();
    }
    if (wide) {
      bool q4 = dq;   // Scale4 needs rows of a multiple of four blocks
      for (int k = 0; k < n; ++k) q4 = q4 && in[k].Kc % 256 == 0;
      if (q4) hipLaunchKernelGGL((qgemm2_kernel<true, true, false>), grid, dim3(kThreads2), 0, st, grp, code16(in[0].qtype));
      else if (dq) hipLaunchKernelGGL((qgemm2_kernel<true, false, false>), grid, dim3(kThreads2), 0, st, grp, code16(in[0].qtype));
      else hipLaunchKernelGGL((qgemm2_kernel<false, false, false>), grid, dim3(kThreads2), 0, st, grp, code16(in[0].qtype));
      return hipGetLastError();
    }
  }
  bool q4 = !KN && dq;   // Scale4 needs row-major weights with rows of a multiple of four blocks
  for (int k = 0; k < n; ++k) q4 = q4 && in[k].Kc % 256 == 0;
  if (q4)
    hipLaunchKernelGGL((qgemm_kernel<KN, true, EPI_NK, !KN>), grid, dim3(kThreads), 0, st, grp, code16(in[0].qtype));
  else if (dq)
    hipLaunchKernelGGL((qgemm_kernel<KN, true, EPI_NK, false>), grid, dim3(kThreads), 0, st, grp, code16(in[0].qtype));
  else
    hipLaunchKernelGGL((qgemm_kernel<KN, false, EPI_NK, false>), grid, dim3(kThreads), 0, st, grp, code16(in[0].qtype));
  return hipGetLastError();
}

// One call over n problems.  Forward tiling, automatic: each tiling's time is
// its rounds of tiles over the compute units (one workgroup per CU) times the
// time of one tile; a 256 x 256 tile measures about 1.74 times a 256 x 128 one
// on the configured shapes (the same work per tile costs about 13 % less).
// The problems may also be split into a wide launch and a narrow one (say a
// layer's q projection on 256 x 256 tiles and its short k and v on 256 x 128)
// when the two launches' rounds cost less than either tiling alone, counting
// a tenth of a round for the second launch.  The kernel trace brackets the
// call's launches together.  dX takes the same choice between its two tilings
// (the 8-wave 256 x 256 one and 256 x 128; a forced variant 3 means the
// 8-wave one there): its wide tile measures about 1.8 times a narrow one.
template <bool KN, bool EPI_NK>
hipError_t launch(const QGemmArgs *in, int n, hipStream_t st, int trace_kind) {
  if (n < 1 || n > QN_MAX_GROUP) return hipErrorInvalidValue;
  TraceScope tr(trace_kind, st);
  const int v = g_variant.load(std::memory_order_relaxed);
  const int wide_kind = v == 3 ? 3 : 2;
  if (v != 0) return launch_tiling<KN, EPI_NK>(in, n, v >= 2, wide_kind, st);
  const int64_t cus = device_cus();
  int64_t tw[QN_MAX_GROUP], tn[QN_MAX_GROUP];
  for (int i = 0; i < n; ++i) {
    tw[i] = cdiv(in[i].M, BM2) * cdiv(in[i].Nout, BN2);
    tn[i] = cdiv(in[i].M, BM) * cdiv(in[i].Nout, BN);
  }
  // subset = problems on the wide tiling
  unsigned best = 0;
  double best_cost = 1e300;
  for (unsigned sub = 0; sub < (1u << n); ++sub) {
    int64_t w = 0, nn = 0;
    for (int i = 0; i < n; ++i) (sub >> i & 1u ? w : nn) += sub >> i & 1u ? tw[i] : tn[i];
    const double cost = 1.74 * (double)cdiv(w, cus) + (double)cdiv(nn, cus) + (w && nn ? 0.1 : 0.0);
    if (cost < best_cost - 1e-9) { best_cost = cost; best = sub; }
  }
  if (best == 0 || best == (1u << n) - 1)
    return launch_tiling<KN, EPI_NK>(in, n, best != 0, wide_kind, st);
  QGemmArgs wa[QN_MAX_GROUP], na[QN_MAX_GROUP];
  int nw = 0, nnw = 0;
  for (int i = 0; i < n; ++i) {
    if (best >> i & 1u) wa[nw++] = in[i];
    else na[nnw++] = in[i];
  }
  const hipError_t e = launch_tiling<KN, EPI_NK>(wa, nw, true, wide_kind, st);
  if (e != hipSuccess) return e;
  return launch_tiling<KN, EPI_NK>(na, nnw, false, wide_kind, st);
}

}  // namespace

hipError_t launch_qgemm_fwd(const QGemmArgs &a, hipStream_t st) {
  return launch<false, true>(&a, 1, st, QN_TRACE_GEMM_FWD);
}

hipError_t launch_qgemm_fwd_group(const QGemmArgs *a, int n, hipStream_t st) {
  return launch<false, true>(a, n, st, QN_TRACE_GEMM_FWD);
}

hipError_t launch_qgemm_dx(const QGemmArgs &a, hipStream_t st) {
  return launch<true, false>(&a, 1, st, QN_TRACE_GEMM_DX);
}

void set_gemm_variant(int v) { g_variant.store(v, std::memory_order_relaxed); }

}  // namespace qn
