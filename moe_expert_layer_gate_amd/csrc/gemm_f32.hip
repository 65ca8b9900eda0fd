// Grouped GEMM for fp32 activations and weights (VALU, LDS-tiled).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// MoE TP优化 / 计算分解: expert(x) = down(SiLU(gate(x)) * up(x)) with gate and
// up merged into one matrix; npu_swiglu splits the last axis into halves and
// returns SiLU(first) * second. Section 高性能专家计算: one grouped operator
// for all experts.
//
// On MI355X fp32 runs at the same dense rate on the vector ALUs as on the
// matrix cores, so the fp32 path uses plain FMAs: a 32-row x 32-column output
// tile per 256-thread block, K staged through LDS 32 at a time, 4 outputs per
// thread (8 FMAs per k with the SwiGLU pair).
#include "common.h"
#include "launch.h"

namespace moe {

template <bool GLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const float* __restrict__ a, const float* __restrict__ w,
    float* __restrict__ out, int K, int Nw, int Nout) {
  constexpr int MT = 32, NT = 32, KT = 32, NB = GLU ? 2 * NT : NT;
  if ((int)blockIdx.x >= tile_count[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int c0 = blockIdx.y * NT;
  const float* we = w + (size_t)tl.expert * K * Nw;
  __shared__ float As[MT][KT + 1];
  __shared__ float Bs[KT][NB + 1];
  const int tid = threadIdx.x, ty = tid >> 3, tx = tid & 7;
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int k0 = 0; k0 < K; k0 += KT) {
    for (int i = tid; i < MT * KT; i += 256) {
      int r = i / KT, kk = i % KT;
      As[r][kk] = r < tl.rows ? a[(size_t)(tl.row0 + r) * K + k0 + kk] : 0.f;
    }
    for (int i = tid; i < KT * NB; i += 256) {
      int kk = i / NB, j = i % NB;
      int col = j < NT ? c0 + j : (Nout + c0 + (j - NT));  // up half at +I
      bool ok = (j < NT ? c0 + j : c0 + (j - NT)) < Nout;
      Bs[kk][j] = ok ? we[(size_t)(k0 + kk) * Nw + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < KT; ++kk) {
      float av = As[ty][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[0][i] = fmaf(av, Bs[kk][tx * 4 + i], acc[0][i]);
        if (GLU) acc[1][i] = fmaf(av, Bs[kk][NT + tx * 4 + i], acc[1][i]);
      }
    }
    __syncthreads();
  }
  if (ty >= tl.rows) return;
  float* o = out + (size_t)(tl.row0 + ty) * Nout;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int col = c0 + tx * 4 + i;
    if (col < Nout) o[col] = GLU ? silu(acc[0][i]) * acc[1][i] : acc[0][i];
  }
}

hipError_t launch_gemm_f32(bool glu, const Tile* tiles,
                           const int32_t* tile_count, int max_tiles,
                           const float* a, const float* w, float* out, int K,
                           int Nw, int Nout, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  dim3 grid(max_tiles, (Nout + 31) / 32), block(256);
  if (glu)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, block, 0, s, tiles,
                       tile_count, a, w, out, K, Nw, Nout);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, block, 0, s, tiles,
                       tile_count, a, w, out, K, Nw, Nout);
  return hipGetLastError();
}

}  // namespace moe
