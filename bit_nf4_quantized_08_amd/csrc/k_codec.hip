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

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;

// Code of one normalised value: bucket lookup plus one compare.  lut[b] holds
// the bucket's threshold and, for NF4, the level below it (whose code is the
// level itself), for FP4 the two candidate codes (low byte below the
// threshold, second byte at or above it).
template <int QT>
__device__ __forceinline__ uint32_t nearest_row(float nrm, const float2 *lut) {
  int b = (int)__builtin_fmaf(nrm, 16.0f, 16.0f);
  b = min(max(b, 0), 31);
  const float2 e = lut[b];
  if constexpr (QT == QN_NF4) return as_u32(e.y) + (nrm >= e.x ? 1u : 0u);
  else return (as_u32(e.y) >> (nrm >= e.x ? 8 : 0)) & 0xFu;
}

__device__ __forceinline__ void load_lut(float2 *lut, const CodecTables &tab, int qt) {
  if (threadIdx.x < 32)
    lut[threadIdx.x] = make_float2(tab.thr[threadIdx.x],
                                   __builtin_bit_cast(float, qt == QN_NF4 ? tab.base[threadIdx.x] : tab.lohi[threadIdx.x]));
}

// ---------------------------------------------------------------- quantise
// A wave takes 1024 consecutive elements (16 blocks) per iteration.  Its load
// instructions are fully coalesced (lane l reads the l-th 16 bytes of a 1 KB
// span), so a block is spread over consecutive lanes: 16 lanes for fp32 input
// (4 elements each), 8 lanes for bf16 input (8 elements each).  The block
// absmax is reduced across those lanes with DPP (quad permutes, then a row
// rotation or half-row mirror); one correctly rounded reciprocal per block;
// codes are stored from registers as 2 or 4 bytes per lane.  The last partial
// wave span (fewer than 1024 elements) is done by one wave, 16 elements per
// lane, with bounds checks.
constexpr int kQChunk = 1024;
constexpr int kQGroupElems = QN_GROUP * QN_BLOCK;   // 16384 weights: one double-quant group

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
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
    for (int i = 0; i < CNT; ++i) w |= nearest_row<QT>(x[i] * rho, lut) << (4 * i);
  } else {
    // 1/a overflows fp32 (a < 2^-128): divide each weight by a instead.
#pragma unroll
    for (int i = 0; i < CNT; ++i) w |= nearest_row<QT>(x[i] / am, lut) << (4 * i);
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

// One full 1024-element span starting at `base`, in two halves so that a
// caller can have several spans' loads in flight before it encodes the first:
// span_load issues the wave's coalesced loads (fp32: 4 x 16 bytes per lane,
// bf16: 2 x 16 bytes), span_encode reduces the block absmaxes (written to
// absmax and, when am_lds is given, to am_lds[block - blk0]) and stores the codes.
template <bool BF16>
struct SpanRaw {
  u32x4 v[BF16 ? 2 : 4];
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

template <bool BF16, int QT>
__device__ __forceinline__ void span_encode(const SpanRaw<BF16> &raw, int64_t base, uint8_t *__restrict__ codes,
                                            float *__restrict__ absmax, const float2 *lut, int lane, float *am_lds,
                                            int64_t blk0) {
  if constexpr (!BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Copy components to scalars before reinterpreting them: a bit_cast
      // applied directly to a vector component reads the wrong element.
      const uint32_t u[4] = {raw.v[i].x, raw.v[i].y, raw.v[i].z, raw.v[i].w};
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = as_f32(u[j]);
      float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
      am = fmaxf(am, dpp_f32<0xB1>(am));    // quad xor 1
      am = fmaxf(am, dpp_f32<0x4E>(am));    // quad xor 2
      am = fmaxf(am, dpp_f32<0x124>(am));   // row rotate by 4
      am = fmaxf(am, dpp_f32<0x128>(am));   // row rotate by 8
      if ((lane & 15) == 0) {
        const int64_t b = base / QN_BLOCK + 4 * i + (lane >> 4);
        absmax[b] = am;
        if (am_lds) am_lds[b - blk0] = am;
      }
      const uint32_t w = encode<4, QT>(v, am, lut);
      *reinterpret_cast<uint16_t *>(codes + base / 2 + 2 * (64 * i + lane)) = (uint16_t)w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t u[4] = {raw.v[i].x, raw.v[i].y, raw.v[i].z, raw.v[i].w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_lo(u[j]);
        v[2 * j + 1] = bf16_hi(u[j]);
      }
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
      am = fmaxf(am, dpp_f32<0xB1>(am));    // quad xor 1
      am = fmaxf(am, dpp_f32<0x4E>(am));    // quad xor 2
      am = fmaxf(am, dpp_f32<0x141>(am));   // half-row mirror: the other quad of 8
      if ((lane & 7) == 0) {
        const int64_t b = base / QN_BLOCK + 8 * i + (lane >> 3);
        absmax[b] = am;
        if (am_lds) am_lds[b - blk0] = am;
      }
      const uint32_t w = encode<8, QT>(v, am, lut);
      *reinterpret_cast<uint32_t *>(codes + base / 2 + 4 * (64 * i + lane)) = w;
    }
  }
}

template <bool BF16, int QT>
__device__ __forceinline__ void quantize_span(const void *__restrict__ W, int64_t base, uint8_t *__restrict__ codes,
                                              float *__restrict__ absmax, const float2 *lut, int lane) {
  SpanRaw<BF16> raw;
  span_load<BF16>(W, base, lane, raw);
  span_encode<BF16, QT>(raw, base, codes, absmax, lut, lane, nullptr, 0);
}

template <bool BF16, int QT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void *__restrict__ W, int64_t n,
                                                            uint8_t *__restrict__ codes,
                                                            float *__restrict__ absmax,
                                                            CodecTables tab) {
  __shared__ float2 lut[32];
  load_lut(lut, tab, QT);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t full = n / kQChunk;
  for (int64_t ch = wave_id; ch < full; ch += nwaves) quantize_span<BF16, QT>(W, ch * kQChunk, codes, absmax, lut, lane);
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

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  return m;
}

// Quantise and double-quantise in one pass: a workgroup owns whole groups of
// 16384 weights (256 blocks); each wave quantises four 1024-element spans of
// the group, the block absmaxes also go to LDS, and after one barrier each
// thread double-quantises one block of the group.
template <bool BF16, int QT>
__global__ __launch_bounds__(kThreads) void quantize_dq_kernel(const void *__restrict__ W, int64_t n,
                                                               uint8_t *__restrict__ codes,
                                                               float *__restrict__ absmax,
                                                               uint8_t *__restrict__ absmax_q,
                                                               float *__restrict__ scale2, CodecTables tab) {
  static_assert(kThreads == QN_GROUP, "one thread per block of the group");
  __shared__ float2 lut[32];
  __shared__ float am_s[QN_GROUP];
  __shared__ float wmax[kThreads / 64];
  load_lut(lut, tab, QT);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nb = (n + QN_BLOCK - 1) / QN_BLOCK;
  const int64_t ngroups = (nb + QN_GROUP - 1) / QN_GROUP;
  const int64_t full = n / kQChunk;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    am_s[tid] = 0.0f;
    __syncthreads();   // lut ready, am_s cleared (and the previous group's reads done)
    const int64_t blk0 = g * QN_GROUP;
    const int64_t ch0 = g * (kQGroupElems / kQChunk) + 4 * wave;   // the wave's four spans
    if (ch0 + 4 <= full) {
      // All four spans' loads in flight before the first is encoded.
      SpanRaw<BF16> raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) span_load<BF16>(W, (ch0 + i) * kQChunk, lane, raw[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) span_encode<BF16, QT>(raw[i], (ch0 + i) * kQChunk, codes, absmax, lut, lane, am_s, blk0);
    } else {
      for (int i = 0; i < 4; ++i) {
        const int64_t ch = ch0 + i;
        if (ch < full) {
          SpanRaw<BF16> raw;
          span_load<BF16>(W, ch * kQChunk, lane, raw);
          span_encode<BF16, QT>(raw, ch * kQChunk, codes, absmax, lut, lane, am_s, blk0);
        } else if (ch == full && full * kQChunk < n) {
          quantize_tail<BF16, QT>(W, n, full * kQChunk, codes, absmax, lut, lane, am_s, blk0);
        }
      }
    }
    __syncthreads();
    const float a = am_s[tid];
    const float m = wave_max(a);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    const float c = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float step = c / 255.0f;
    if (tid == 0) scale2[g] = step;
    if (blk0 + tid < nb) absmax_q[blk0 + tid] = (uint8_t)dq_code(a, step);
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
    // One workgroup per group of 16384 weights, a few resident per CU.
    const int64_t groups = (n + kQGroupElems - 1) / kQGroupElems;
    const int grid = (int)std::min<int64_t>(groups, (int64_t)device_cus() * 8);
    if (w_is_bf16)
      hipLaunchKernelGGL((quantize_dq_kernel<true, QT>), dim3(grid), dim3(kThreads), 0, s, W, n, codes, absmax,
                         absmax_q, scale2, tab);
    else
      hipLaunchKernelGGL((quantize_dq_kernel<false, QT>), dim3(grid), dim3(kThreads), 0, s, W, n, codes, absmax,
                         absmax_q, scale2, tab);
    return;
  }
  const int grid = grid_for((n + kQChunk - 1) / kQChunk * 64);
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
