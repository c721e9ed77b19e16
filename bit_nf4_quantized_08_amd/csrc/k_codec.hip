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

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;

// Row index of one normalised value: bucket lookup plus one compare.
__device__ __forceinline__ uint32_t nearest_row(float nrm, const float2 *lut) {
  int b = (int)__builtin_fmaf(nrm, 16.0f, 16.0f);
  b = min(max(b, 0), 31);
  const float2 e = lut[b];
  const float thr = e.x, base = e.y;
  return as_u32(base) + (nrm >= thr ? 1u : 0u);
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

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Codes of `cnt` normalised values x[i] * rho (or x[i] / a when 1/a overflows),
// packed low nibble first.
template <int CNT>
__device__ __forceinline__ uint32_t encode(const float *x, float am, const float2 *lut) {
  // Correctly rounded reciprocal, once per block (infinite when 1/a overflows).
  const float rho = am > 0.0f ? 1.0f / am : 0.0f;
  uint32_t w = 0;
  if (!__builtin_isinf(rho)) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) w |= nearest_row(x[i] * rho, lut) << (4 * i);
  } else {
    // 1/a overflows fp32 (a < 2^-128): divide each weight by a instead.
#pragma unroll
    for (int i = 0; i < CNT; ++i) w |= nearest_row(x[i] / am, lut) << (4 * i);
  }
  return w;
}

template <bool BF16>
__device__ void quantize_tail(const void *__restrict__ W, int64_t n, int64_t start, uint8_t *__restrict__ codes,
                              float *__restrict__ absmax, const float2 *lut, int lane) {
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
  if ((lane & 3) == 0 && e0 < n) absmax[e0 / QN_BLOCK] = am;
  const uint32_t lo = encode<8>(v, am, lut), hi = encode<8>(v + 8, am, lut);
  if (e0 < n) {
    // Elements past n were zeros whose row index is the zero row; clear those
    // nibbles so the padding nibble of an odd count is 0.
    const int64_t valid = n - e0;
    uint64_t word = ((uint64_t)hi << 32) | lo;
    if (valid < 16) word &= (1ull << (4 * valid)) - 1ull;
    const int64_t nbytes = (n + 1) / 2, b0 = e0 / 2;
    for (int i = 0; i < 8 && b0 + i < nbytes; ++i) codes[b0 + i] = (uint8_t)(word >> (8 * i));
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const void *__restrict__ W, int64_t n,
                                                            uint8_t *__restrict__ codes,
                                                            float *__restrict__ absmax,
                                                            CodecTables tab) {
  __shared__ float2 lut[32];
  if (threadIdx.x < 32) {
    lut[threadIdx.x] = make_float2(tab.thr[threadIdx.x], __builtin_bit_cast(float, tab.base[threadIdx.x]));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t full = n / kQChunk;
  for (int64_t ch = wave_id; ch < full; ch += nwaves) {
    const int64_t base = ch * kQChunk;
    if constexpr (!BF16) {
      // instruction i: elements base + 4 (64 i + lane) .. +4, block 4 i + lane / 16
      const float *p = static_cast<const float *>(W) + base;
      u32x4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = ld_stream(p + 4 * (64 * i + lane));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // Copy components to scalars before reinterpreting them: a bit_cast
        // applied directly to a vector component reads the wrong element.
        const uint32_t u[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = as_f32(u[j]);
        float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        am = fmaxf(am, dpp_f32<0xB1>(am));    // quad xor 1
        am = fmaxf(am, dpp_f32<0x4E>(am));    // quad xor 2
        am = fmaxf(am, dpp_f32<0x124>(am));   // row rotate by 4
        am = fmaxf(am, dpp_f32<0x128>(am));   // row rotate by 8
        if ((lane & 15) == 0) absmax[base / QN_BLOCK + 4 * i + (lane >> 4)] = am;
        const uint32_t w = encode<4>(v, am, lut);
        *reinterpret_cast<uint16_t *>(codes + base / 2 + 2 * (64 * i + lane)) = (uint16_t)w;
      }
    } else {
      // instruction i: elements base + 8 (64 i + lane) .. +8, block 8 i + lane / 8
      const uint16_t *p = static_cast<const uint16_t *>(W) + base;
      u32x4 raw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) raw[i] = ld_stream(p + 8 * (64 * i + lane));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t u[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
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
        if ((lane & 7) == 0) absmax[base / QN_BLOCK + 8 * i + (lane >> 3)] = am;
        const uint32_t w = encode<8>(v, am, lut);
        *reinterpret_cast<uint32_t *>(codes + base / 2 + 4 * (64 * i + lane)) = w;
      }
    }
  }
  if (full * kQChunk < n && wave_id == nwaves - 1) quantize_tail<BF16>(W, n, full * kQChunk, codes, absmax, lut, lane);
}

// ------------------------------------------------------------ double quant
// One workgroup of 256 lanes per group of 256 block scales.
__global__ __launch_bounds__(kThreads) void double_quant_kernel(const float *__restrict__ absmax, int64_t nb,
                                                                uint8_t *__restrict__ absmax_q,
                                                                float *__restrict__ scale2) {
  __shared__ float wmax[kThreads / 64];
  const int64_t g = blockIdx.x;
  const int64_t b = g * QN_GROUP + threadIdx.x;
  const float a = b < nb ? absmax[b] : 0.0f;
  float m = a;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float c = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float step = c / 255.0f;
  if (threadIdx.x == 0) scale2[g] = step;
  if (b < nb) {
    uint32_t k = 0;
    if (step > 0.0f) {
      const float t = a / step;
      // t - 1/2 is exact in fp32 for t >= 1/2; below that the ceiling is 0 anyway.
      const float kf = ceilf(t - 0.5f);
      k = (uint32_t)fminf(fmaxf(kf, 0.0f), 255.0f);
    }
    absmax_q[b] = (uint8_t)k;
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

hipError_t launch_quantize(const void *W, int w_is_bf16, int64_t n, uint8_t *codes, float *absmax,
                           hipStream_t s) {
  const CodecTables &tab = codec_tables();
  const int grid = grid_for((n + kQChunk - 1) / kQChunk * 64);
  TraceScope tr(QN_TRACE_QUANTIZE, s);
  if (w_is_bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid), dim3(kThreads), 0, s, W, n, codes, absmax, tab);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid), dim3(kThreads), 0, s, W, n, codes, absmax, tab);
  return hipGetLastError();
}

hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *absmax_q, float *scale2,
                               hipStream_t s) {
  const int64_t ng = (nb + QN_GROUP - 1) / QN_GROUP;
  TraceScope tr(QN_TRACE_DOUBLE_QUANT, s);
  hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)ng), dim3(kThreads), 0, s, absmax, nb, absmax_q,
                     scale2);
  return hipGetLastError();
}

hipError_t launch_dequant(const qn_nf4_weight &W, void *out, int out_bf16, hipStream_t s) {
  const CodecTables &tab = codec_tables();
  const int64_t n = W.N * W.K;
  ScaleSrc sc{W.absmax, W.absmax_q, W.scale2};
  const int grid = grid_for((n + 7) / 8, 4);   // a few resident workgroups per CU, each building its table once
  TraceScope tr(QN_TRACE_DEQUANT, s);
  if (out_bf16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid), dim3(kThreads), 0, s, W.codes, sc, n, out, tab);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid), dim3(kThreads), 0, s, W.codes, sc, n, out, tab);
  return hipGetLastError();
}

}  // namespace qn
