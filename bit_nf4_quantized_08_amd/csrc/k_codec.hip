// Codec kernels for gfx950: blockwise NF4 quantisation, double quantisation of
// the block scales, dequantisation.
//
// "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs":
//   - "The table, and the number that stretches it": scale = largest magnitude
//     of the group, divide, round to the closest row, store its index; read back
//     by looking the row up and multiplying by the scale.
//   - "Why the groups are small": groups of 64, each with its own scale.
//   - "Shrink the scale factors too, and total up the real bill": the scales in
//     8 bits, 256 per group with one 32-bit constant.
//
// All three are HBM-streaming kernels: 128-bit coalesced loads and stores,
// grid-stride loops over a grid sized to a few waves per CU.  No floating-point
// contraction: every rounding step is the one the format defines.

#pragma clang fp contract(off)

#include <algorithm>
#include <map>
#include <mutex>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;

// Code of one normalised value n: bucket lookup plus one compare.  t5 is the
// fp32 value of n + 5 rounded once (in [4, 8) for n in [-1, 1 + 2^-23]):
// its mantissa's top six bits are the bucket floor(16 n + 16), 0 .. 32.
// lut[b] holds the bucket's threshold and, for NF4, the level below it (whose
// code is the level itself), for FP4 the two candidate codes (low byte below
// the threshold, second byte at or above it).
template <int QT>
__device__ __forceinline__ uint32_t nearest_row(float nrm, float t5, const float2 *lut) {
  const float2 e = lut[(as_u32(t5) >> 17) & 63u];
  if constexpr (QT == QN_NF4) return as_u32(e.y) + (nrm >= e.x ? 1u : 0u);
  else return (as_u32(e.y) >> (nrm >= e.x ? 8 : 0)) & 0xFu;
}

__device__ __forceinline__ void load_lut(float2 *lut, const CodecTables &tab, int qt) {
  if (threadIdx.x < kBuckets)
    lut[threadIdx.x] = make_float2(tab.thr[threadIdx.x],
                                   __builtin_bit_cast(float, qt == QN_NF4 ? tab.base[threadIdx.x] : tab.lohi[threadIdx.x]));
}

// ---------------------------------------------------------------- quantise
// A wave takes spans of 1024 consecutive elements (16 blocks), two per
// iteration of the plain quantiser, with every load of both issued first.  Its
// load instructions are fully coalesced (lane l reads the l-th 16 bytes of a 1
// KB span), so a block is spread over consecutive lanes: 16 lanes for fp32
// input (4 elements each), 8 lanes for bf16 input (8 elements each).  The block
// absmax is reduced across those lanes with DPP (quad permutes, then a row
// rotation or half-row mirror); one correctly rounded reciprocal per block;
// codes are stored from registers as 2 or 4 bytes per lane.  The last partial
// span (fewer than 1024 elements) is done by one wave, 16 elements per lane,
// with bounds checks.
constexpr int kQChunk = 1024;
constexpr int kQGroupElems = QN_GROUP * QN_BLOCK;   // 16384 weights: one double-quant group

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Codes of `cnt` normalised values x[i] * rho (or x[i] / a when 1/a overflows),
// packed low nibble first.
template <int CNT, int QT>
__device__ __forceinline__ uint32_t encode(const float *x, float am, const float2 *lut) {
  // Correctly rounded reciprocal, once per block (infinite when 1/a overflows).
  const float rho = am > 0.0f ? 1.0f / am : 0.0f;
  uint32_t w = 0;
  if (!__builtin_isinf(rho)) {
#pragma unroll
    for (int i = 0; i < CNT; ++i)
      w |= nearest_row<QT>(x[i] * rho, __builtin_fmaf(x[i], rho, 5.0f), lut) << (4 * i);
  } else {
    // 1/a overflows fp32 (a < 2^-128): divide each weight by a instead.
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const float nrm = x[i] / am;
      w |= nearest_row<QT>(nrm, nrm + 5.0f, lut) << (4 * i);
    }
  }
  return w;
}

// The last partial span: 16 elements per lane from element `start`, bounds
// checked.  Block absmaxes go to absmax (and, when am_lds is given, to
// am_lds[(block - blk0)]).
template <bool BF16, int QT>
__device__ void quantize_tail(const void *__restrict__ W, int64_t n, int64_t start, uint8_t *__restrict__ codes,
                              float *__restrict__ absmax, const float2 *lut, int lane, float *am_lds = nullptr,
                              int64_t blk0 = 0) {
  const int64_t e0 = start + 16 * lane;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t e = e0 + i;
    float x = 0.0f;
    if (e < n) {
      if constexpr (BF16) x = bf16_to_f32(static_cast<const uint16_t *>(W)[e]);
      else x = static_cast<const float *>(W)[e];
    }
    v[i] = x;
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
  am = fmaxf(am, dpp_f32<0xB1>(am));
  am = fmaxf(am, dpp_f32<0x4E>(am));
  if ((lane & 3) == 0 && e0 < n) {
    absmax[e0 / QN_BLOCK] = am;
    if (am_lds) am_lds[e0 / QN_BLOCK - blk0] = am;
  }
  const uint32_t lo = encode<8, QT>(v, am, lut), hi = encode<8, QT>(v + 8, am, lut);
  if (e0 < n) {
    // Elements past n were zeros whose code is the zero code (0 for FP4, 7 for
    // NF4); clear those nibbles so the padding nibble of an odd count is 0.
    const int64_t valid = n - e0;
    uint64_t word = ((uint64_t)hi << 32) | lo;
    if (valid < 16) word &= (1ull << (4 * valid)) - 1ull;
    const int64_t nbytes = (n + 1) / 2, b0 = e0 / 2;
    for (int i = 0; i < 8 && b0 + i < nbytes; ++i) codes[b0 + i] = (uint8_t)(word >> (8 * i));
  }
}

// One full 1024-element span starting at `base`, in three parts so that a
// caller can have several spans' loads in flight and encode them in one
// straight-line stretch of code: span_load issues the wave's coalesced loads
// (fp32: 4 x 16 bytes per lane, bf16: 2 x 16 bytes), span_codes reduces the
// block absmaxes and encodes every element with the block's reciprocal,
// span_store writes codes and absmaxes (and, when am_lds is given, the
// absmaxes to am_lds[block - blk0]).  A block whose reciprocal overflows is
// re-encoded by span_codes_div, behind one wave-uniform test per span, so
// the common path has no branch and its table lookups can overlap.
template <bool BF16>
struct SpanRaw {
  u32x4 v[BF16 ? 2 : 4];
};

// Per load instruction i of a span: the lane's packed codes, its block's
// absmax and reciprocal.
template <bool BF16>
struct SpanEnc {
  static constexpr int kI = BF16 ? 2 : 4;
  uint32_t w[kI];
  float am[kI];
  float rho[kI];
};

template <bool BF16>
__device__ __forceinline__ void span_load(const void *__restrict__ W, int64_t base, int lane, SpanRaw<BF16> &raw) {
  if constexpr (!BF16) {
    // instruction i: elements base + 4 (64 i + lane) .. +4, block 4 i + lane / 16
    const float *p = static_cast<const float *>(W) + base;
#pragma unroll
    for (int i = 0; i < 4; ++i) raw.v[i] = ld_stream(p + 4 * (64 * i + lane));
  } else {
    // instruction i: elements base + 8 (64 i + lane) .. +8, block 8 i + lane / 8
    const uint16_t *p = static_cast<const uint16_t *>(W) + base;
#pragma unroll
    for (int i = 0; i < 2; ++i) raw.v[i] = ld_stream(p + 8 * (64 * i + lane));
  }
}

// The lane's elements of load instruction i as fp32.
template <bool BF16>
__device__ __forceinline__ void span_values(const SpanRaw<BF16> &raw, int i, float (&v)[BF16 ? 8 : 4]) {
  // Copy components to scalars before reinterpreting them: a bit_cast
  // applied directly to a vector component reads the wrong element.
  const uint32_t u[4] = {raw.v[i].x, raw.v[i].y, raw.v[i].z, raw.v[i].w};
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(u[j]);
      v[2 * j + 1] = bf16_hi(u[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = as_f32(u[j]);
  }
}

// Block absmaxes (every lane of a block ends with its block's value: DPP quad
// permutes, then a half-row mirror for the 8 lanes of a bf16 block or two row
// rotations for the 16 lanes of an fp32 block), correctly rounded reciprocals,
// codes by multiplying with the reciprocal.  Returns true in a lane whose
// reciprocal overflowed (its codes are then redone by span_codes_div).
template <bool BF16, int QT>
__device__ __forceinline__ bool span_codes(const SpanRaw<BF16> &raw, const float2 *lut, SpanEnc<BF16> &e) {
  constexpr int C = BF16 ? 8 : 4;
  bool slow = false;
#pragma unroll
  for (int i = 0; i < SpanEnc<BF16>::kI; ++i) {
    float v[C];
    span_values<BF16>(raw, i, v);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < C; ++j) am = fmaxf(am, fabsf(v[j]));
    // Across the block's lanes the maxima of magnitudes are taken on their
    // bit patterns (for non-negative fp32 the integer order is the value
    // order), which lets each DPP exchange fold into an integer max.
    uint32_t ab = as_u32(am);
    ab = max(ab, dpp_u32<0xB1>(ab));    // quad xor 1
    ab = max(ab, dpp_u32<0x4E>(ab));    // quad xor 2
    if constexpr (BF16) {
      ab = max(ab, dpp_u32<0x141>(ab));   // half-row mirror: the other quad of 8
    } else {
      ab = max(ab, dpp_u32<0x124>(ab));   // row rotate by 4
      ab = max(ab, dpp_u32<0x128>(ab));   // row rotate by 8
    }
    e.am[i] = as_f32(ab);
  }
  // Correctly rounded reciprocals of the lane's kI block maxima (infinite when
  // 1/a overflows) with one division: lane l divides for instruction l mod kI
  // (the kI lanes of an aligned group share their blocks) and takes the
  // others' results by DPP.
  constexpr int kI = SpanEnc<BF16>::kI;
  const int lane = threadIdx.x & 63;
  float mine = e.am[0];
#pragma unroll
  for (int i = 1; i < kI; ++i) mine = (lane & (kI - 1)) == i ? e.am[i] : mine;
  const float r = mine > 0.0f ? 1.0f / mine : 0.0f;
  if constexpr (kI == 2) {
    const float o = dpp_f32<0xB1>(r);   // lane ^ 1
    e.rho[0] = (lane & 1) ? o : r;
    e.rho[1] = (lane & 1) ? r : o;
  } else {
    e.rho[0] = dpp_f32<0x00>(r);   // quad broadcast of lane 0
    e.rho[1] = dpp_f32<0x55>(r);   // lane 1
    e.rho[2] = dpp_f32<0xAA>(r);   // lane 2
    e.rho[3] = dpp_f32<0xFF>(r);   // lane 3
  }
#pragma unroll
  for (int i = 0; i < kI; ++i) {
    float v[C];
    span_values<BF16>(raw, i, v);
    const float rho = e.rho[i];
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) w |= nearest_row<QT>(v[j] * rho, __builtin_fmaf(v[j], rho, 5.0f), lut) << (4 * j);
    e.w[i] = w;
    slow |= __builtin_isinf(rho);
  }
  return slow;
}

// 1/a overflows fp32 (a < 2^-128): divide each weight of such a block by a.
// Run for the whole wave (behind a wave-uniform test) and selected per lane,
// so that none of it is folded into the common path.
template <bool BF16, int QT>
__device__ void span_codes_div(const SpanRaw<BF16> &raw, const float2 *lut, SpanEnc<BF16> &e) {
  constexpr int C = BF16 ? 8 : 4;
#pragma unroll
  for (int i = 0; i < SpanEnc<BF16>::kI; ++i) {
    float v[C];
    span_values<BF16>(raw, i, v);
    // The divisor passes through an empty asm statement (a side effect the
    // compiler cannot move), so that the divisions stay behind the test
    // instead of being speculated into the common path.
    float a = e.am[i];
    asm volatile("" : "+v"(a));
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float nrm = v[j] / a;
      w |= nearest_row<QT>(nrm, nrm + 5.0f, lut) << (4 * j);
    }
    e.w[i] = __builtin_isinf(e.rho[i]) ? w : e.w[i];
  }
}

// Codes from registers (2 or 4 bytes per lane per instruction, contiguous over
// the wave); each block's absmax is stored by all lanes of the block, same
// value to the same address, so no lane needs a branch.
template <bool BF16>
__device__ __forceinline__ void span_store(const SpanEnc<BF16> &e, int64_t base, uint8_t *__restrict__ codes,
                                           float *__restrict__ absmax, int lane, float *am_lds, int64_t blk0) {
#pragma unroll
  for (int i = 0; i < SpanEnc<BF16>::kI; ++i) {
    const int64_t b = BF16 ? base / QN_BLOCK + 8 * i + (lane >> 3) : base / QN_BLOCK + 4 * i + (lane >> 4);
    absmax[b] = e.am[i];
    if (am_lds) am_lds[b - blk0] = e.am[i];
    if constexpr (BF16) *reinterpret_cast<uint32_t *>(codes + base / 2 + 4 * (64 * i + lane)) = e.w[i];
    else *reinterpret_cast<uint16_t *>(codes + base / 2 + 2 * (64 * i + lane)) = (uint16_t)e.w[i];
  }
}

// U consecutive full spans from span index ch0: all loads first, then each
// span's codes (one straight-line stretch, the rare division path behind a
// wave-uniform test) and stores.
template <bool BF16, int QT, int U>
__device__ __forceinline__ void quantize_spans(const void *__restrict__ W, int64_t ch0, uint8_t *__restrict__ codes,
                                               float *__restrict__ absmax, const float2 *lut, int lane,
                                               float *am_lds, int64_t blk0) {
  SpanRaw<BF16> raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) span_load<BF16>(W, (ch0 + u) * kQChunk, lane, raw[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    SpanEnc<BF16> e;
    if (__builtin_amdgcn_ballot_w64(span_codes<BF16, QT>(raw[u], lut, e)) != 0)
      span_codes_div<BF16, QT>(raw[u], lut, e);
    span_store<BF16>(e, (ch0 + u) * kQChunk, codes, absmax, lane, am_lds, blk0);
  }
}

// Spans per wave iteration of the plain quantiser.
constexpr int kQSpans = 2;

template <bool BF16, int QT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void quantize_kernel(const void *__restrict__ W, int64_t n,
                                                            uint8_t *__restrict__ codes,
                                                            float *__restrict__ absmax,
                                                            CodecTables tab) {
  __shared__ float2 lut[kBuckets];
  load_lut(lut, tab, QT);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t full = n / kQChunk;
  const int64_t groups = full / kQSpans;
  for (int64_t g = wave_id; g < groups; g += nwaves)
    quantize_spans<BF16, QT, kQSpans>(W, g * kQSpans, codes, absmax, lut, lane, nullptr, 0);
  // Full spans left over after the groups, one per wave.
  const int64_t left = full - groups * kQSpans;
  if (wave_id < left) quantize_spans<BF16, QT, 1>(W, groups * kQSpans + wave_id, codes, absmax, lut, lane, nullptr, 0);
  if (full * kQChunk < n && wave_id == nwaves - 1)
    quantize_tail<BF16, QT>(W, n, full * kQChunk, codes, absmax, lut, lane);
}

// Double quantisation of one group's scales held by the workgroup's 256
// threads (thread t: block g*256 + t, value a, 0 past nb): c = group max,
// step = fl32(c / 255), k = clamp(ceil(fl32(a / step) - 1/2), 0, 255), ties
// down; a zero group has step 0 and all k = 0.
__device__ __forceinline__ uint32_t dq_code(float a, float step) {
  if (!(step > 0.0f)) return 0u;
  const float t = a / step;
  // t - 1/2 is exact in fp32 for t >= 1/2; below that the ceiling is 0 anyway.
  const float kf = ceilf(t - 0.5f);
  return (uint32_t)fminf(fmaxf(kf, 0.0f), 255.0f);
}

// Maximum over the wave, in every lane, without LDS traffic: DPP within each
// row of 16 lanes (quad swaps, half-row and row mirrors), then the four rows'
// maxima read out with readlane.
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, dpp_f32<0xB1>(m));    // quad: lanes i ^ 1
  m = fmaxf(m, dpp_f32<0x4E>(m));    // quad: lanes i ^ 2
  m = fmaxf(m, dpp_f32<0x141>(m));   // half-row mirror: the two quads of 8
  m = fmaxf(m, dpp_f32<0x140>(m));   // row mirror: the two halves of 16
  const auto rd = [](float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  };
  return fmaxf(fmaxf(rd(m, 0), rd(m, 16)), fmaxf(rd(m, 32), rd(m, 48)));
}

// Quantise and double-quantise in one pass: a workgroup of 8 waves owns whole
// groups of 16384 weights (256 blocks); each wave quantises two 1024-element
// spans of the group, the block absmaxes also go to LDS, and after one barrier
// each of the first 256 threads double-quantises one block of the group.
constexpr int kDqThreads = 512;
constexpr int kDqSpans = kQGroupElems / kQChunk / (kDqThreads / 64);   // spans per wave: 2

template <bool BF16, int QT>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(BF16 ? 8 : 4, 8))) void quantize_dq_kernel(const void *__restrict__ W, int64_t n,
                                                                 uint8_t *__restrict__ codes,
                                                                 float *__restrict__ absmax,
                                                                 uint8_t *__restrict__ absmax_q,
                                                                 float *__restrict__ scale2, CodecTables tab) {
  static_assert(kDqThreads >= QN_GROUP && kDqSpans * (kDqThreads / 64) * kQChunk == kQGroupElems, "group split");
  __shared__ float2 lut[kBuckets];
  __shared__ float am_s[QN_GROUP];
  __shared__ float wmax[QN_GROUP / 64];
  load_lut(lut, tab, QT);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nb = (n + QN_BLOCK - 1) / QN_BLOCK;
  const int64_t ngroups = (nb + QN_GROUP - 1) / QN_GROUP;
  const int64_t full = n / kQChunk;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    if (tid < QN_GROUP) am_s[tid] = 0.0f;
    __syncthreads();   // lut ready, am_s cleared (and the previous group's reads done)
    const int64_t blk0 = g * QN_GROUP;
    const int64_t ch0 = g * (kQGroupElems / kQChunk) + kDqSpans * wave;   // the wave's spans
    if (ch0 + kDqSpans <= full) {
      // Both spans' loads in flight before the first is encoded.
      quantize_spans<BF16, QT, kDqSpans>(W, ch0, codes, absmax, lut, lane, am_s, blk0);
    } else {
      for (int i = 0; i < kDqSpans; ++i) {
        const int64_t ch = ch0 + i;
        if (ch < full) {
          quantize_spans<BF16, QT, 1>(W, ch, codes, absmax, lut, lane, am_s, blk0);
        } else if (ch == full && full * kQChunk < n) {
          quantize_tail<BF16, QT>(W, n, full * kQChunk, codes, absmax, lut, lane, am_s, blk0);
        }
      }
    }
    __syncthreads();
    float a = 0.0f;
    if (tid < QN_GROUP) {
      a = am_s[tid];
      const float m = wave_max(a);
      if (lane == 0) wmax[wave] = m;
    }
    __syncthreads();
    if (tid < QN_GROUP) {
      const float c = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
      const float step = c / 255.0f;
      if (tid == 0) scale2[g] = step;
      if (blk0 + tid < nb) absmax_q[blk0 + tid] = (uint8_t)dq_code(a, step);
    }
  }
}

// ------------------------------------------------------------ double quant
// One wave per group of 256 block scales: lane l takes scales 4l .. 4l+3 (one
// 16-byte load), the group max comes from a wave reduction, and the lane writes
// its four 8-bit codes as one word.  Four groups per workgroup.
__global__ __launch_bounds__(kThreads) void double_quant_kernel(const float *__restrict__ absmax, int64_t nb,
                                                                uint8_t *__restrict__ absmax_q,
                                                                float *__restrict__ scale2) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t ngroups = (nb + QN_GROUP - 1) / QN_GROUP;
  if (g >= ngroups) return;
  const int64_t b0 = g * QN_GROUP + 4 * lane;
  float a[4];
  if (b0 + 4 <= nb && ((reinterpret_cast<uintptr_t>(absmax + b0) & 15) == 0)) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(absmax + b0);
    a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = b0 + i < nb ? absmax[b0 + i] : 0.0f;
  }
  const float m = wave_max(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])));
  const float step = m / 255.0f;
  if (lane == 0) scale2[g] = step;
  uint32_t k[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k[i] = dq_code(a[i], step);
  if (b0 + 4 <= nb && ((reinterpret_cast<uintptr_t>(absmax_q + b0) & 3) == 0)) {
    *reinterpret_cast<uint32_t *>(absmax_q + b0) = k[0] | (k[1] << 8) | (k[2] << 16) | (k[3] << 24);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (b0 + i < nb) absmax_q[b0 + i] = (uint8_t)k[i];
  }
}

// ---------------------------------------------------------------- dequant
// A wave expands 2048 consecutive elements per iteration (1 KB of codes).  Its
// 32 block scales are computed by lanes 0..31 and handed out with a lane
// shuffle.  Each store instruction of the wave writes one contiguous 1 KB span:
// bf16 output, 8 elements (one 32-bit word of codes) per lane per instruction;
// fp32 output, 4 elements (16 bits of codes) per lane per instruction.  The
// byte -> (row lo, row hi) table lives in LDS, one copy per lane of an 8-lane
// group so that the lookups of a group hit distinct banks.
__device__ __forceinline__ float block_scale(const ScaleSrc &sc, int64_t b) {
  if (sc.absmax_q) return (float)sc.absmax_q[b] * sc.scale2[b / QN_GROUP];
  return sc.absmax[b];
}

constexpr int kDqChunk = 2048;   // elements per wave iteration
constexpr int kDqCopies = 8;

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t *__restrict__ codes, ScaleSrc sc,
                                                           int64_t n, void *__restrict__ out,
                                                           CodecTables tab) {
  __shared__ float2 pair[256 * kDqCopies];
  for (int i = threadIdx.x; i < 256 * kDqCopies; i += kThreads) {
    const int v = i / kDqCopies;
    pair[i] = make_float2(tab.code[v & 15], tab.code[v >> 4]);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int copy = lane & (kDqCopies - 1);
  const int64_t wave_id = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t full = n / kDqChunk;
  for (int64_t ch = wave_id; ch < full; ch += nwaves) {
    const int64_t base = ch * kDqChunk;
    const float my_scale = lane < 32 ? block_scale(sc, base / QN_BLOCK + lane) : 0.0f;
    if constexpr (OUT_BF16) {
      uint32_t cw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + base / 2) + i * 64 + lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // elements base + (i*64 + lane)*8 .. +8: block (i*64 + lane)/8 of the chunk
        const float A = __shfl(my_scale, i * 8 + (lane >> 3), 64);
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 c = pair[((cw[i] >> (8 * j)) & 0xFF) * kDqCopies + copy];
          o[j] = pack_bf16x2(c.x * A, c.y * A);
        }
        st_stream(static_cast<uint16_t *>(out) + base + (int64_t)(i * 64 + lane) * 8, u32x4{o[0], o[1], o[2], o[3]});
      }
    } else {
      uint32_t cw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        cw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(codes + base / 2) + i * 64 + lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // elements base + (i*64 + lane)*4 .. +4: block (i*64 + lane)/16 of the chunk
        const float A = __shfl(my_scale, i * 4 + (lane >> 4), 64);
        const float2 c0 = pair[(cw[i] & 0xFF) * kDqCopies + copy];
        const float2 c1 = pair[((cw[i] >> 8) & 0xFF) * kDqCopies + copy];
        st_stream_f4(static_cast<float *>(out) + base + (int64_t)(i * 64 + lane) * 4,
                     f32x4{c0.x * A, c0.y * A, c1.x * A, c1.y * A});
      }
    }
  }
  // Tail (fewer than 2048 elements): one element per lane of the first wave.
  if (wave_id == 0) {
    for (int64_t e = full * kDqChunk + lane; e < n; e += 64) {
      const uint8_t byte = codes[e >> 1];
      const uint32_t q = (e & 1) ? (byte >> 4) : (byte & 15);
      const float w = pair[q * kDqCopies].x * block_scale(sc, e / QN_BLOCK);
      if constexpr (OUT_BF16) static_cast<uint16_t *>(out)[e] = f32_to_bf16(w);
      else static_cast<float *>(out)[e] = w;
    }
  }
}

// Workgroups of kernel `fn` (`threads` threads) that fit on one CU at once
// (occupancy query, cached per kernel).
int resident_per_cu(const void *fn, int threads = kThreads) {
  static std::mutex mu;
  static std::map<const void *, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(fn);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, 0) != hipSuccess || nb < 1) nb = 1;
  cache[fn] = nb;
  return nb;
}

int grid_for(int64_t work_items, int per_cu_waves = 8) {
  // At most a few workgroups per CU for a grid-stride loop; at least one item each.
  int64_t wgs = (work_items + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cus() * per_cu_waves;
  if (wgs > cap) wgs = cap;
  if (wgs < 1) wgs = 1;
  return (int)wgs;
}

}  // namespace

template <int QT>
void launch_quantize_t(const void *W, int w_is_bf16, int64_t n, uint8_t *codes, float *absmax, uint8_t *absmax_q,
                       float *scale2, hipStream_t s) {
  const CodecTables &tab = codec_tables(QT);
  if (absmax_q) {
    // One 8-wave workgroup per group of 16384 weights, as many as are resident.
    const int64_t groups = (n + kQGroupElems - 1) / kQGroupElems;
    const void *fn = w_is_bf16 ? reinterpret_cast<const void *>(&quantize_dq_kernel<true, QT>)
                               : reinterpret_cast<const void *>(&quantize_dq_kernel<false, QT>);
    const int grid = (int)std::min<int64_t>(groups, (int64_t)device_cus() * resident_per_cu(fn, kDqThreads));
    if (w_is_bf16)
      hipLaunchKernelGGL((quantize_dq_kernel<true, QT>), dim3(grid), dim3(kDqThreads), 0, s, W, n, codes, absmax,
                         absmax_q, scale2, tab);
    else
      hipLaunchKernelGGL((quantize_dq_kernel<false, QT>), dim3(grid), dim3(kDqThreads), 0, s, W, n, codes, absmax,
                         absmax_q, scale2, tab);
    return;
  }
  // One wave per kQSpans spans, as many workgroups as are resident at once.
  const void *fn = w_is_bf16 ? reinterpret_cast<const void *>(&quantize_kernel<true, QT>)
                             : reinterpret_cast<const void *>(&quantize_kernel<false, QT>);
  const int64_t wave_iters = std::max<int64_t>(1, (n + kQSpans * kQChunk - 1) / (kQSpans * kQChunk));
  const int grid = (int)std::max<int64_t>(
      1, std::min<int64_t>((wave_iters + kThreads / 64 - 1) / (kThreads / 64),
                           (int64_t)device_cus() * resident_per_cu(fn)));
  if (w_is_bf16)
    hipLaunchKernelGGL((quantize_kernel<true, QT>), dim3(grid), dim3(kThreads), 0, s, W, n, codes, absmax, tab);
  else
    hipLaunchKernelGGL((quantize_kernel<false, QT>), dim3(grid), dim3(kThreads), 0, s, W, n, codes, absmax, tab);
}

hipError_t launch_quantize(const void *W, int w_is_bf16, int64_t n, int qtype, uint8_t *codes, float *absmax,
                           uint8_t *absmax_q, float *scale2, hipStream_t s) {
  TraceScope tr(QN_TRACE_QUANTIZE, s);
  if (qtype == QN_FP4) launch_quantize_t<QN_FP4>(W, w_is_bf16, n, codes, absmax, absmax_q, scale2, s);
  else launch_quantize_t<QN_NF4>(W, w_is_bf16, n, codes, absmax, absmax_q, scale2, s);
  return hipGetLastError();
}

hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *absmax_q, float *scale2,
                               hipStream_t s) {
  const int64_t ng = (nb + QN_GROUP - 1) / QN_GROUP;
  TraceScope tr(QN_TRACE_DOUBLE_QUANT, s);
  hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)((ng + 3) / 4)), dim3(kThreads), 0, s, absmax, nb,
                     absmax_q, scale2);
  return hipGetLastError();
}

hipError_t launch_dequant(const qn_nf4_weight &W, void *out, int out_bf16, hipStream_t s) {
  const CodecTables &tab = codec_tables(W.quant_type);
  const int64_t n = W.N * W.K;
  ScaleSrc sc{W.absmax, W.absmax_q, W.scale2, W.quant_type};
  const int grid = grid_for((n + 7) / 8, 4);   // a few resident workgroups per CU, each building its table once
  TraceScope tr(QN_TRACE_DEQUANT, s);
  if (out_bf16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid), dim3(kThreads), 0, s, W.codes, sc, n, out, tab);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid), dim3(kThreads), 0, s, W.codes, sc, n, out, tab);
  return hipGetLastError();
}

}  // namespace qn
