// Upstream fused norm: residual add + RMSNorm + dual cast / dynamic MXFP8.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// 融合算子优化: the residual add, the RMSNorm and the conversion of its
// output run as one operator so that the sum and the normalised rows are not
// written and read back in between -- either with a dual output (fp32 for
// the router, bf16 for the experts; 融合RMSNorm Cast) or as dynamic MXFP8
// with round mode "rint" to float8_e4m3fn (融合RMSNorm MX量化, without a
// residual on the first layer); section RmsNorm算子优化: RMSNorm is LayerNorm
// without the mean subtraction.
//
// One wave per token row, HBM bound (each input byte read once, each output
// byte written once; the norm weight stays in L2). Lane l owns the 16-byte
// chunks c = l + 64 j of the row (8 consecutive columns each), all of them
// loaded before any arithmetic: the fp32 sum s = x + residual stays in
// registers, the sum of squares is reduced across the wave, and the outputs
// are written from the same registers. An MX block (32 columns) is 4
// consecutive chunks = 4 adjacent lanes, so its amax takes two shuffles.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

MOE_DEV void unpack8(const uint4 v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y);
  f[3] = bf16_hi(v.y); f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

MOE_DEV uint4 pack8(const float f[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

}  // namespace

// MX: 0 -> y_f32 / y_bf16 (either may be null), 1 -> e4m3 codes + e8m0
// scales. CPL: 16-byte chunks per lane (H <= 512 * CPL).
template <int MX, int CPL>
__global__ __launch_bounds__(256) void add_rms_norm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ residual,
    const uint16_t* __restrict__ wn, float eps, int T, int H,
    float* __restrict__ y32, uint16_t* __restrict__ y16,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    uint16_t* __restrict__ res_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const int C = H / 8;
  const size_t row = (size_t)t * C;
  uint4 xv[CPL], rv[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    const bool ok = c < C;
    xv[j] = ok ? ((const uint4*)x)[row + c] : make_uint4(0, 0, 0, 0);
    rv[j] = ok && residual ? ((const uint4*)residual)[row + c]
                           : make_uint4(0, 0, 0, 0);
  }
  float s[CPL][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float a[8], b[8];
    unpack8(xv[j], a);
    unpack8(rv[j], b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s[j][i] = residual ? a[i] + b[i] : a[i];  // fp32 add; x as is alone
      ss = fmaf(s[j][i], s[j][i], ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float rstd = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    const bool ok = c < C;
    if (ok && res_out) ((uint4*)res_out)[row + c] = pack8(s[j]);
    float w[8];
    unpack8(ok ? ((const uint4*)wn)[c] : make_uint4(0, 0, 0, 0), w);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = s[j][i] * rstd * w[i];
    if (MX == 0) {
      if (ok && y32) {
        float4* p = (float4*)(y32 + (row + c) * 8);
        p[0] = make_float4(y[0], y[1], y[2], y[3]);
        p[1] = make_float4(y[4], y[5], y[6], y[7]);
      }
      if (ok && y16) ((uint4*)y16)[row + c] = pack8(y);
    } else {
      // every lane of a 4-lane group is valid or none is (C % 4 == 0)
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int se = mx_e4m3_scale_exp(amax);
      const uint32_t lo = e4m3x4_hw(y, se), hi = e4m3x4_hw(y + 4, se);
      if (ok) {
        *(uint2*)(codes + (row + c) * 8) = make_uint2(lo, hi);
        if ((c & 3) == 0) scales[(size_t)t * (H / 32) + (c >> 2)] = (uint8_t)(se + 127);
      }
    }
  }
}

template <int MX>
static hipError_t launch_norm_mode(int cpl, const uint16_t* x,
                                   const uint16_t* r, const uint16_t* w,
                                   float eps, int T, int H, float* y32,
                                   uint16_t* y16, uint8_t* codes,
                                   uint8_t* scales, uint16_t* res_out,
                                   hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
#define MOE_NORM_CASE(N)                                                     \
  if (cpl <= N) {                                                            \
    hipLaunchKernelGGL((add_rms_norm_kernel<MX, N>), grid, block, 0, s, x, r, \
                       w, eps, T, H, y32, y16, codes, scales, res_out);      \
    return hipGetLastError();                                                \
  }
  MOE_NORM_CASE(1)
  MOE_NORM_CASE(2)
  MOE_NORM_CASE(4)
  MOE_NORM_CASE(8)
  MOE_NORM_CASE(12)
  MOE_NORM_CASE(16)
#undef MOE_NORM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_add_rms_norm(int mx, const uint16_t* x, const uint16_t* r,
                               const uint16_t* w, float eps, int T, int H,
                               float* y32, uint16_t* y16, uint8_t* codes,
                               uint8_t* scales, uint16_t* res_out,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpl = (H / 8 + 63) / 64;
  return mx ? launch_norm_mode<1>(cpl, x, r, w, eps, T, H, y32, y16, codes,
                                  scales, res_out, s)
            : launch_norm_mode<0>(cpl, x, r, w, eps, T, H, y32, y16, codes,
                                  scales, res_out, s);
}

}  // namespace moe
