// MXFP4 quantisation of bf16 expert weights (a load-time step, like packing).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// MoE EP优化 / AllGather方案(W4A8量化): the routed experts of the W4A8 scheme
// hold MXFP4 weights. The pages give no encoding rule; the OCP MX v1.0 one is
// used: blocks of 32 consecutive K of one output column share an e8m0 scale
// 2^s with s = floor(log2(amax)) - 2 (clamped to [-127, 127], an all-zero
// block gets code 0), and every element is the e2m1 code of v / 2^s rounded
// to nearest with ties to even, saturating at 6, sign kept.
//
// In:  w bf16 [E, K, N], N contiguous (the bf16 layout of w13 [E, H, 2I] and
//      w2 [E, I, H]).
// Out: codes [E, N, K/2] bytes (K contiguous per output column, two codes per
//      byte, the low nibble holds the even k) and scales [E, N, K/32] e8m0.
// One thread per (expert, column, 32-K block): the 64 lanes of a wave take 64
// consecutive columns, so each of the 32 bf16 loads of a thread is part of a
// 128-byte row segment shared by the wave; each thread writes its 16 code
// bytes and its scale byte.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void quant_mxfp4_weights_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, long long nthreads, int K, int N) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nthreads) return;
  const int n = (int)(i % N);
  const long long rest = i / N;
  const int nkb = K / 32;
  const int kb = (int)(rest % nkb);
  const long long e = rest / nkb;
  const uint16_t* src = w + (e * K + 32LL * kb) * N + n;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    v[j] = bf16_to_f32(src[(long long)j * N]);
    amax = fmaxf(amax, __builtin_fabsf(v[j]));
  }
  const int s = mx_e2m1_scale_exp(amax);
  uint32_t word[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) b |= e2m1_encode_scaled(v[8 * q + j], s) << (4 * j);
    word[q] = b;
  }
  const long long col = e * N + n;
  *(uint4*)(codes + col * (K / 2) + 16LL * kb) =
      make_uint4(word[0], word[1], word[2], word[3]);
  scales[col * nkb + kb] = (uint8_t)(s + 127);
}

}  // namespace

hipError_t launch_quant_mxfp4_weights(int E, int K, int N, const uint16_t* w,
                                      uint8_t* codes, uint8_t* scales,
                                      hipStream_t s) {
  const long long nthreads = (long long)E * N * (K / 32);
  if (nthreads == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_mxfp4_weights_kernel,
                     dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, s,
                     w, codes, scales, nthreads, K, N);
  return hipGetLastError();
}

}  // namespace moe
