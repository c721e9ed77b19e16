// One AdamW step on bf16 adapter parameters with 8-bit block-wise optimizer
// state.
//
// "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", "Why the
// groups are small": block-wise quantisation (blocks of 64, a scale each) is
// what makes 8-bit optimizer state work; "Turn a LoRA script into a QLoRA
// script with one config object": the optimizer is an 8-bit AdamW and its
// state belongs to the adapter only.  AdamW's rule itself (decoupled weight
// decay, bias-corrected moments) is the published one; the pages do not
// restate it.
//
// Per parameter, fp32, each operation rounded once in this order:
//   m  = k_m * step_m,  u = k_u * step_u,  v = u * u          (old state)
//   m' = b1 m + c1 g,  v' = b2 v + c2 (g g)
//   d  = (m' / bc1) / (sqrt(v' / bc2) + eps) + wd p
//   p' = bf16(p - lr d)
//   u' = sqrt(v')
// and per block of 64 parameters the new state:
//   step_m = max|m'| / 127,  k_m = clamp(ceil(m'/step_m - 1/2), -127, 127)
//   step_u = max u' / 255,   k_u = clamp(ceil(u'/step_u - 1/2), 0, 255)
//   (a zero block: step 0, codes 0).
// A lane owns 4 consecutive parameters, 16 lanes a block; the block maxima are
// reduced across those lanes with DPP.  HBM-bound: about 10 bytes per parameter.
// The multi-tensor kernel runs the same span code over several tensors in one
// launch (an adapter's tensors are small: one launch each is latency-bound).

#pragma clang fp contract(off)

#include <algorithm>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int kThreads = 256;
constexpr int kAdamBlock = 64;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Maximum over the 16 lanes of a row (lanes 16q .. 16q + 15).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));    // quad xor 1
  v = fmaxf(v, dpp<0x4E>(v));    // quad xor 2
  v = fmaxf(v, dpp<0x124>(v));   // row rotate by 4
  v = fmaxf(v, dpp<0x128>(v));   // row rotate by 8
  return v;
}

__device__ __forceinline__ int grid_code(float x, float step, float lo, float hi) {
  if (!(step > 0.0f)) return 0;
  const float t = x / step;
  return (int)fminf(fmaxf(ceilf(t - 0.5f), lo), hi);
}

// One span of 256 parameters (four blocks of 64) of one tensor: the wave's
// lane l owns parameters 256 sp + 4 l .. +3.
__device__ __forceinline__ void adam_span(uint16_t *__restrict__ p, const uint16_t *__restrict__ g, int64_t n,
                                          int8_t *__restrict__ mq, float *__restrict__ ms, uint8_t *__restrict__ uq,
                                          float *__restrict__ us, const AdamConsts &c, int64_t sp, int lane) {
  const int64_t e0 = sp * 256 + 4 * lane;
  const int64_t blk = e0 / kAdamBlock;
  const bool full = e0 + 4 <= n;
  float pv[4], gv[4], m[4], u[4];
  int km[4], ku[4];
  if (full) {
    const u32x2 pw = *reinterpret_cast<const u32x2 *>(p + e0);
    const u32x2 gw = *reinterpret_cast<const u32x2 *>(g + e0);
    const uint32_t mw = *reinterpret_cast<const uint32_t *>(mq + e0);
    const uint32_t uw = *reinterpret_cast<const uint32_t *>(uq + e0);
    const uint32_t pa[2] = {pw.x, pw.y}, ga[2] = {gw.x, gw.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      pv[2 * i] = bf16_lo(pa[i]); pv[2 * i + 1] = bf16_hi(pa[i]);
      gv[2 * i] = bf16_lo(ga[i]); gv[2 * i + 1] = bf16_hi(ga[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      km[i] = (int)(int8_t)(mw >> (8 * i));
      ku[i] = (int)((uw >> (8 * i)) & 0xFF);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = e0 + i < n;
      pv[i] = in ? bf16_to_f32(p[e0 + i]) : 0.0f;
      gv[i] = in ? bf16_to_f32(g[e0 + i]) : 0.0f;
      km[i] = in ? (int)mq[e0 + i] : 0;
      ku[i] = in ? (int)uq[e0 + i] : 0;
    }
  }
  const bool bin = e0 < n;
  const float sm = bin ? ms[blk] : 0.0f, su = bin ? us[blk] : 0.0f;
  float m1[4], u1[4], p1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = (float)km[i] * sm;
    u[i] = (float)ku[i] * su;
    const float v = u[i] * u[i];
    m1[i] = c.b1 * m[i] + c.c1 * gv[i];
    const float v1 = c.b2 * v + c.c2 * (gv[i] * gv[i]);
    const float mh = m1[i] / c.bc1;
    const float vh = v1 / c.bc2;
    const float den = __builtin_sqrtf(vh) + c.eps;
    const float d = mh / den + c.wd * pv[i];
    p1[i] = pv[i] - c.lr * d;
    u1[i] = __builtin_sqrtf(v1);
  }
  float am = fmaxf(fmaxf(fabsf(m1[0]), fabsf(m1[1])), fmaxf(fabsf(m1[2]), fabsf(m1[3])));
  float au = fmaxf(fmaxf(u1[0], u1[1]), fmaxf(u1[2], u1[3]));
  am = row16_max(am);
  au = row16_max(au);
  const float step_m = am / 127.0f, step_u = au / 255.0f;
  if (bin && (lane & 15) == 0) {
    ms[blk] = step_m;
    us[blk] = step_u;
  }
  uint32_t mw = 0, uw = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mw |= (uint32_t)(uint8_t)(int8_t)grid_code(m1[i], step_m, -127.0f, 127.0f) << (8 * i);
    uw |= (uint32_t)grid_code(u1[i], step_u, 0.0f, 255.0f) << (8 * i);
  }
  if (full) {
    *reinterpret_cast<u32x2 *>(p + e0) = u32x2{pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
    *reinterpret_cast<uint32_t *>(mq + e0) = mw;
    *reinterpret_cast<uint32_t *>(uq + e0) = uw;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (e0 + i < n) {
        p[e0 + i] = f32_to_bf16(p1[i]);
        mq[e0 + i] = (int8_t)(mw >> (8 * i));
        uq[e0 + i] = (uint8_t)(uw >> (8 * i));
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void adamw8_kernel(uint16_t *__restrict__ p, const uint16_t *__restrict__ g,
                                                          int64_t n, int8_t *__restrict__ mq,
                                                          float *__restrict__ ms, uint8_t *__restrict__ uq,
                                                          float *__restrict__ us, AdamConsts c) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t spans = (n + 255) / 256;   // 256 parameters (4 blocks) per wave step
  for (int64_t sp = wave; sp < spans; sp += nwaves) adam_span(p, g, n, mq, ms, uq, us, c, sp, lane);
}

// Several tensors in one launch: their spans are numbered one after another
// (tensor i owns spans [first[i], first[i + 1])), and the waves walk the
// whole range with a grid stride; each span belongs to one tensor, found by a
// scan of the (at most QN_ADAMW_MULTI) boundaries.
__global__ __launch_bounds__(kThreads) void adamw8_multi_kernel(AdamMulti mt, AdamConsts c) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t total = mt.first[mt.n];
  for (int64_t sp = wave; sp < total; sp += nwaves) {
    int ti = 0;
    for (int k = 1; k < mt.n; ++k) ti += sp >= mt.first[k] ? 1 : 0;
    ti = __builtin_amdgcn_readfirstlane(ti);
    const AdamTensor &t = mt.t[ti];
    adam_span(t.p, t.g, t.n, t.mq, t.ms, t.uq, t.us, c, sp - mt.first[ti], lane);
  }
}

}  // namespace

hipError_t launch_adamw8(uint16_t *p, const uint16_t *g, int64_t n, int8_t *mq, float *ms, uint8_t *uq, float *us,
                         const AdamConsts &c, hipStream_t st) {
  const int64_t spans = (n + 255) / 256;
  const int64_t waves = std::min<int64_t>(spans, (int64_t)device_cus() * 32);
  const int grid = (int)((waves + 3) / 4);
  TraceScope tr(QN_TRACE_ADAMW8, st);
  hipLaunchKernelGGL(adamw8_kernel, dim3(grid), dim3(kThreads), 0, st, p, g, n, mq, ms, uq, us, c);
  return hipGetLastError();
}

hipError_t launch_adamw8_multi(const AdamMulti &mt, const AdamConsts &c, hipStream_t st) {
  const int64_t spans = mt.first[mt.n];
  const int64_t waves = std::min<int64_t>(spans, (int64_t)device_cus() * 32);
  const int grid = (int)std::max<int64_t>(1, (waves + 3) / 4);
  TraceScope tr(QN_TRACE_ADAMW8, st);
  hipLaunchKernelGGL(adamw8_multi_kernel, dim3(grid), dim3(kThreads), 0, st, mt, c);
  return hipGetLastError();
}

}  // namespace qn
