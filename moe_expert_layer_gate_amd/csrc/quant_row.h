// Per-row dynamic quantisation by one wavefront, shared by the row kernels
// (quant_i8.hip, routing.hip) and the fused gate + per-token quantisation
// of the layer (gate_topk.hip).
//
// int8 ([P3] "NPU Qwen3-Next inference practice", 量化策略: int8 activations
// with a dynamic scale per token): amax = max |v|; scale = amax / 127
// rounded to nearest fp32; code = rint(v / scale) with the quotient rounded
// to nearest fp32 and rint taking ties to even, clipped to [-127, 127]; an
// all-zero row gets scale 0 and codes 0. Divisions are the correctly rounded
// fp32 division (__fdiv_rn), so codes and scales are bit-identical to any
// other IEEE evaluation of that rule.
//
// MXFP8 ([P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// W4A8: dynamic MXFP8 e4m3 activations, one e8m0 scale per 32 values; scale
// and element rounding as in common.h).
#pragma once
#include "common.h"

namespace moe {

template <bool F32>
MOE_DEV void load8(const void* src, size_t off, float (&v)[8]) {
  if (F32) {
    const float4 a = *(const float4*)((const float*)src + off);
    const float4 b = *(const float4*)((const float*)src + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 a = *(const uint4*)((const uint16_t*)src + off);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  }
}

MOE_DEV uint32_t code_byte(float v, float scale) {
  float q = rintf(__fdiv_rn(v, scale));
  q = fminf(fmaxf(q, -127.f), 127.f);
  return (uint32_t)(int)q & 0xFFu;
}

// One wave quantises one row of K values (bf16, or fp32 when F32) read at
// element offset so of src: codes to orow, the scale to *scale_out (lane 0).
// CPL > 0: the row (at most 512 * CPL elements) is held in registers and
// read once; CPL == 0: any length, read twice (amax, then codes).
template <bool F32, int CPL>
MOE_DEV void quant_i8_row(const void* __restrict__ src, int K, size_t so,
                          int8_t* __restrict__ orow,
                          float* __restrict__ scale_out, int lane) {
  float amax = 0.f;
  if constexpr (CPL > 0) {
    float v[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = 512 * i + 8 * lane;
      if (c < K) {
        load8<F32>(src, so + c, v[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = __fdiv_rn(amax, 127.f);
    if (lane == 0) *scale_out = scale;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = 512 * i + 8 * lane;
      if (c >= K) break;
      uint2 o = {0u, 0u};
      if (scale > 0.f) {
        o.x = code_byte(v[i][0], scale) | code_byte(v[i][1], scale) << 8 |
              code_byte(v[i][2], scale) << 16 | code_byte(v[i][3], scale) << 24;
        o.y = code_byte(v[i][4], scale) | code_byte(v[i][5], scale) << 8 |
              code_byte(v[i][6], scale) << 16 | code_byte(v[i][7], scale) << 24;
      }
      *(uint2*)(orow + c) = o;
    }
    return;
  }
  for (int c = 8 * lane; c < K; c += 512) {
    float v[8];
    load8<F32>(src, so + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = __fdiv_rn(amax, 127.f);
  if (lane == 0) *scale_out = scale;
  for (int c = 8 * lane; c < K; c += 512) {
    uint2 o = {0u, 0u};
    if (scale > 0.f) {
      float v[8];
      load8<F32>(src, so + c, v);
      o.x = code_byte(v[0], scale) | code_byte(v[1], scale) << 8 |
            code_byte(v[2], scale) << 16 | code_byte(v[3], scale) << 24;
      o.y = code_byte(v[4], scale) | code_byte(v[5], scale) << 8 |
            code_byte(v[6], scale) << 16 | code_byte(v[7], scale) << 24;
    }
    *(uint2*)(orow + c) = o;
  }
}

// One wave quantises one bf16 row of H values (H % 32 == 0) to MXFP8: e4m3
// codes to dst, one e8m0 scale per 32 values to dsc. Eight 16-byte chunks
// per lane are in flight before any encoding; a 32-value block is 4
// consecutive chunks = 4 adjacent lanes, so it never straddles the row end.
MOE_DEV void quant_mx_row_bf16(const uint4* __restrict__ src, int H,
                               uint8_t* __restrict__ dst,
                               uint8_t* __restrict__ dsc, int lane) {
  for (int c0 = lane; c0 < H / 8; c0 += 512) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + 64 * j;
      v[j] = c < H / 8 ? src[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + 64 * j;
      float f[8] = {bf16_lo(v[j].x), bf16_hi(v[j].x), bf16_lo(v[j].y),
                    bf16_hi(v[j].y), bf16_lo(v[j].z), bf16_hi(v[j].z),
                    bf16_lo(v[j].w), bf16_hi(v[j].w)};
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int s = mx_e4m3_scale_exp(amax);
      const uint32_t lo = e4m3x4_hw(f, s), hi = e4m3x4_hw(f + 4, s);
      if (c < H / 8) {
        *(uint2*)(dst + (size_t)c * 8) = make_uint2(lo, hi);
        if ((c & 3) == 0) dsc[c >> 2] = (uint8_t)(s + 127);
      }
    }
  }
}

}  // namespace moe
