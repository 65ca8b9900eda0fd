// Gating top-k softmax: one wavefront per token, 4 tokens per block.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// section 快速选择专家; [P2] "LongCat-Flash inference on Atlas A3 clusters",
// MoE模块 / Router. The per-row routine lives in gate_wave.h.
#include "common.h"
#include "gate_wave.h"
#include "launch.h"
#include "quant_row.h"

#ifndef MOE_GATE_QUANT_ROWS
#define MOE_GATE_QUANT_ROWS 1
#endif

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void gate_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wout) {
  __shared__ uint2 slots[4][64];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  topk_softmax_wave<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k,
                         wout + (size_t)t * k, slots[threadIdx.x >> 6]);
}

hipError_t launch_gate_topk(const float* logits, int T, int E, int k,
                            int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  int vpl = (E + 63) / 64;
#define MOE_GATE_CASE(N)                                                   \
  if (vpl <= N) {                                                          \
    hipLaunchKernelGGL(gate_topk_kernel<N>, grid, block, 0, s, logits, T, \
                       E, k, ids, w);                                      \
    return hipGetLastError();                                              \
  }
  MOE_GATE_CASE(1)
  MOE_GATE_CASE(2)
  MOE_GATE_CASE(4)
  MOE_GATE_CASE(8)
  MOE_GATE_CASE(12)
  MOE_GATE_CASE(16)
  MOE_GATE_CASE(32)
#undef MOE_GATE_CASE
  return hipErrorInvalidValue;
}

// The gate and the per-token quantisation of x that the W4A8 (MXFP8) and
// W8A8 (int8) layers apply before routing, in one launch: blocks [0, gb)
// gate four tokens each (one wave per token), blocks [gb, gb + qb) quantise
// QR rows of x per wave. The two roles run side by side on the chip instead
// of one after the other in each wave, so the gate's latency chain hides
// under the quantisation's HBM traffic. Q = 1: MXFP8 (codes [T, H], e8m0
// [T, H/32]); Q = 2: int8 with CPL chunks of 512 per lane (codes [T, H],
// fp32 scales [T]). The codes equal those of the separate kernels bit for
// bit (same row routines).
template <int VPL, int Q, int CPL, int QR>
__global__ __launch_bounds__(256) void gate_quant_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wout,
    const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq,
    void* __restrict__ xs, int gb) {
  __shared__ uint2 slots[4][64];
  const int lane = threadIdx.x & 63;
  if ((int)blockIdx.x >= gb) {
    const int t0 = ((blockIdx.x - gb) * 4 + (threadIdx.x >> 6)) * QR;
#pragma unroll
    for (int r = 0; r < QR; ++r) {
      const int t = t0 + r;
      if (t >= T) break;  // whole wave
      if (Q == 1)
        quant_mx_row_bf16((const uint4*)(x + (size_t)t * H), H,
                          xq + (size_t)t * H,
                          (uint8_t*)xs + (size_t)t * (H / 32), lane);
      else
        quant_i8_row<false, CPL>(x, H, (size_t)t * H,
                                 (int8_t*)xq + (size_t)t * H, (float*)xs + t,
                                 lane);
    }
    return;
  }
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  topk_softmax_wave<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k,
                         wout + (size_t)t * k, slots[threadIdx.x >> 6]);
}

bool gate_quant_ok(int E, int H, bool mx) {
  return E <= 256 && H % 32 == 0 && (mx || H == 2048 || H == 4096);
}

hipError_t launch_gate_topk_quant(const float* logits, int T, int E, int k,
                                  int32_t* ids, float* w, const uint16_t* x,
                                  int H, bool mx, void* xq, void* xs,
                                  hipStream_t s) {
  if (!gate_quant_ok(E, H, mx)) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  constexpr int QR = MOE_GATE_QUANT_ROWS;  // rows per quantising wave
  const int gb = (T + 3) / 4, qb = (T + 4 * QR - 1) / (4 * QR);
  dim3 grid(gb + qb), block(256);
  const int vpl = (E + 63) / 64;
#define MOE_GQ(V, Q_, C)                                                      \
  hipLaunchKernelGGL((gate_quant_kernel<V, Q_, C, QR>), grid, block, 0, s,   \
                     logits, T, E, k, ids, w, x, H, (uint8_t*)xq, xs, gb)
#define MOE_GQ_V(Q_, C)                                                       \
  do {                                                                        \
    if (vpl <= 1) MOE_GQ(1, Q_, C);                                           \
    else if (vpl <= 2) MOE_GQ(2, Q_, C);                                      \
    else MOE_GQ(4, Q_, C);                                                    \
  } while (0)
  if (mx) MOE_GQ_V(1, 0);
  else if (H == 2048) MOE_GQ_V(2, 4);
  else MOE_GQ_V(2, 8);
#undef MOE_GQ_V
#undef MOE_GQ
  return hipGetLastError();
}

}  // namespace moe
