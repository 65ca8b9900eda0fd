// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 bits

// 16 bytes of weights that a weight-streaming GEMM reads exactly once: a
// load with the nontemporal hint (MOE_STREAM_NT 0: a plain load). Measured
// on MI355X, a 4 GB streaming read reaches 7.0 TB/s with the hint against
// 6.2 TB/s without.
#ifndef MOE_STREAM_NT
#define MOE_STREAM_NT 1
#endif
MOE_DEV uint4 load_stream16(const void* p) {
#if MOE_STREAM_NT
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load((const v4u*)p);
  return uint4{v.x, v.y, v.z, v.w};
#else
  return *(const uint4*)p;
#endif
}

MOE_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs), two values
// per instruction (v_cvt_pk_bf16_f32): lo in bits 0-15, hi in 16-31.
// Compared on MI355X with the integer rounding (u + 0x7FFF + lsb) >> 16
// over every finite fp32 value, subnormals included: no difference.
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t,
                            __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
MOE_DEV uint32_t f32_to_bf16_bits(float f) {
  return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}

// ---------------------------------------------------------------- wave ops

MOE_DEV int lane_id() { return __lane_id(); }

MOE_DEV uint64_t ballot(bool p) { return __ballot(p); }

MOE_DEV int popc64(uint64_t m) { return __popcll(m); }

MOE_DEV uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------- MX encode
//
// e8m0 shared exponent of an MX block (OCP MX v1.0): floor(log2(amax)) minus
// the element format's emax (8 for e4m3), clamped to [-127, 127], stored with
// bias 127. An all-zero block gets code 0. Computed from the fp32 bits.
MOE_DEV int floor_log2_f32(float a) {  // a > 0, finite
  uint32_t u = __float_as_uint(a);
  int ex = (int)((u >> 23) & 0xFF);
  if (ex) return ex - 127;
  uint32_t m = u & 0x7FFFFFu;  // subnormal: m * 2^-149
  return (31 - __clz((int)m)) - 149;
}

MOE_DEV int mx_e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int s = floor_log2_f32(amax) - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// Round-to-nearest-even right shift of a non-negative integer.
MOE_DEV uint32_t rne_shift(uint32_t m, int sh) {
  if (sh <= 0) return m << (-sh);
  if (sh >= 32) return 0;
  uint32_t q = m >> sh;
  uint32_t rem = m & ((1u << sh) - 1u);
  uint32_t half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  return q;
}

// e8m0 shared exponent of an MXFP4 block: floor(log2(amax)) - 2 (emax of
// e2m1), clamped to [-127, 127]; an all-zero block gives -127 (code 0).
MOE_DEV int mx_e2m1_scale_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int s = floor_log2_f32(amax) - 2;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// e2m1 code (OCP MX v1.0: 1 sign, 2 exponent bits with bias 1, 1 mantissa
// bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) of v * 2^-s, rounded to nearest
// with ties to even, saturating at 6, sign kept (values that round to zero
// give +0 or -0). Exact integer arithmetic on the fp32 bits of v.
MOE_DEV uint32_t e2m1_encode_scaled(float v, int s) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 28) & 0x8u;
  int ex = (int)((u >> 23) & 0xFF);
  uint32_t M = u & 0x7FFFFFu;
  if (ex) M |= 0x800000u; else ex = 1;
  if (M == 0) return sign;
  int p = ex - 150 - s;                      // |v| * 2^-s = M * 2^p
  int nb = 32 - __clz((int)M);               // bit length of M
  int e = nb - 1 + p;                        // floor(log2(|v| 2^-s))
  if (e >= 0) {                              // normal range (>= 1.0)
    uint32_t r = rne_shift(M, nb - 2);       // 2 significant bits, in [2, 4]
    if (r == 4) { r = 2; ++e; }
    if (e > 2) return sign | 0x7u;           // saturate at 6
    return sign | ((uint32_t)(e + 1) << 1) | (r - 2);
  }
  // subnormal: multiples of 0.5; rounding up to 2 lands on the code of 1.0
  return sign | rne_shift(M, -(p + 1));
}

// Two e4m3fn codes, of a * 2^-s and b * 2^-s, by the hardware conversion
// (OCP e4m3, round to nearest even) after clamping to +-448 (saturation):
// into bytes 0-1 of the result, or with hi into bytes 2-3 keeping bytes 0-1
// of old. This is the exact rounding (ties to even, saturating at 448, sign
// kept, subnormals included) wherever |v * 2^-s| < 512, which the MX block
// scale guarantees: compared on MI355X with an exact integer encoder over
// every fp32 value of magnitude below 512, with no difference. Not for NaN
// or infinite inputs.
MOE_DEV uint32_t e4m3x2_hw(float a, float b, int s, uint32_t old = 0,
                           bool hi = false) {
  const float wa =
      fminf(fmaxf(__builtin_amdgcn_ldexpf(a, -s), -448.0f), 448.0f);
  const float wb =
      fminf(fmaxf(__builtin_amdgcn_ldexpf(b, -s), -448.0f), 448.0f);
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(wa, wb, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(wa, wb, (int)old, false);
}

// Four codes of v[0..3] * 2^-s, v[i] in byte i.
MOE_DEV uint32_t e4m3x4_hw(const float* v, int s) {
  return e4m3x2_hw(v[2], v[3], s, e4m3x2_hw(v[0], v[1], s), true);
}

// ---------------------------------------------------------------- misc

MOE_DEV float silu(float z) { return z / (1.0f + expf(-z)); }

// SiLU with the hardware exp2 and reciprocal (a few ulp; for epilogues whose
// result is rounded to bf16 or quantised right away).
MOE_DEV float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace moe
