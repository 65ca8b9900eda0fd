// Stand-alone weight prefetch (moe_prefetch_weights): the prefetch.h routine
// on a grid of its own, for a caller to enqueue on a second stream while the
// operators in front of the MoE layer run.
//
// [P2] "LongCat-Flash inference on Atlas A3 clusters", section 权重预取:
// weights of a memory-bound matmul fetched ahead during an earlier operator,
// about bandwidth x that operator's duration of them.
#include "common.h"
#include "launch.h"
#include "prefetch.h"

namespace moe {

__global__ __launch_bounds__(256) void prefetch_kernel(Prefetch pf) {
  __shared__ uint32_t lds[kPrefetchLdsWords];
  prefetch_block(pf, blockIdx.x, gridDim.x, lds, 256);
}

hipError_t launch_prefetch(const Prefetch& pf, int blocks, hipStream_t s) {
  if (blocks <= 0 || pf.lead < 16 || pf.nexp <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefetch_kernel, dim3(blocks), dim3(256), 0, s, pf);
  return hipGetLastError();
}

}  // namespace moe
