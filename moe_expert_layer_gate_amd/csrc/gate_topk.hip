// Gating top-k softmax: one wavefront per token.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// section 快速选择专家: one fused router op replaces top-k followed by softmax.
// [P2] "LongCat-Flash inference on Atlas A3 clusters", MoE模块 / Router: sort
// the router output and keep the top-k experts.
//
// Selection compares the fp32 logits exactly, key (logit desc, id asc); the
// weights are the softmax over the k selected logits (equal to the full
// softmax renormalised over the top-k).
//
// Each lane keeps VPL logits in registers (expert e = lane + 64 * i). Round r
// takes, per lane, the best not-yet-taken entry, reduces (value, id) across
// the wave with xor shuffles, and the owning lane marks the winner taken.
// Lane j keeps winner j; lanes < k then compute exp, a wave sum and the
// weight, and store one (id, weight) each -- a coalesced row write.
#include "common.h"
#include "launch.h"

namespace moe {

MOE_DEV bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int VPL>
__global__ __launch_bounds__(256) void gate_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  const float* row = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.f;
  }
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;

  float my_v = 0.f;
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    // lane-local best among untaken entries
    float bv = 0.f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      bool ok = !((taken >> i) & 1u);
      if (ok && (bi == 0x7FFFFFFF || better(v[i], e, bv, bi))) {
        bv = v[i];
        bi = e;
      }
    }
    // wave arg-max on (value desc, id asc); id 0x7FFFFFFF marks "none"
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      bool take = (bi == 0x7FFFFFFF) ||
                  (oi != 0x7FFFFFFF && better(ov, oi, bv, bi));
      if (take) { bv = ov; bi = oi; }
    }
    if (bi != 0x7FFFFFFF && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) { my_v = bv; my_id = bi; }
  }
  // softmax over the k winners; winner 0 holds the maximum logit
  float vmax = __shfl(my_v, 0);
  float p = lane < k ? expf(my_v - vmax) : 0.f;
  float sum = p;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    wout[(size_t)t * k + lane] = p / sum;
  }
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
