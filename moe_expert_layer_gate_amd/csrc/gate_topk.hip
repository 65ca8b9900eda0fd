// Gating top-k softmax: one wavefront per token, 4 tokens per block.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// section 快速选择专家; [P2] "LongCat-Flash inference on Atlas A3 clusters",
// MoE模块 / Router. The per-row routine lives in gate_wave.h.
#include "common.h"
#include "gate_wave.h"
#include "launch.h"

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

}  // namespace moe
