// Grouped GEMM, MXFP8 activations x MXFP4 weights on the scaled MFMA.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters": the W4A8
// mixed-precision path (overview; prefill section "MXFP8/MXFP4量化"), MoE
// EP优化 / AllGather方案(W4A8量化) (dynamic MXFP8 quantisation of the hidden
// states, grouped matmul over the local experts) and MoE TP优化 / 计算分解
// (expert = down(SiLU(gate(x)) * up(x)), merged gate/up).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = e4m3 (format 0) and B = e2m1
// (format 4). Operand layout on gfx950 (measured with an in-bounds probe of
// one instruction): with q = l/16 and a 128-wide K step,
//   B (e2m1, 4 VGPRs): lane l holds column l%16, K [32q, 32q+32);
//   A (e4m3, 8 VGPRs): lane l holds row l%16, K [16q, 16q+16) in bytes 0-15
//                      and K [64+16q, 64+16q+16) in bytes 16-31;
//   scales: lane l holds the e8m0 scale of row / column l%16 for the K block
//           [32q, 32q+32), whichever lanes hold that block's data.
// Both operands are K-contiguous in memory, so every lane issues 16-byte
// loads straight into registers: two for A, one for B per step.
//
// GEMM1 (glu): each lane carries 4 gate groups and the 4 matching up groups of
// 16 columns (64 h columns per wave); the epilogue forms h = SiLU(g) * u in
// fp32 and quantises it to MXFP8 per 32 columns (amax over 16 lanes x 2
// groups). GEMM2: 8 groups of 16 output columns, stored as bf16.
// KSPLIT waves split K and meet in LDS as in the bf16 streaming kernel.
#include "common.h"
#include "launch.h"

namespace moe {

MOE_DEV f32x4 mfma_mx(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa,
                                                          0, sb);
}

template <bool GLU, int RG, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void gemm_mx_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    void* __restrict__ out, uint8_t* __restrict__ os, int K, int Nw,
    int Nout) {
  constexpr int NG = 8;                       // 16-column groups per lane
  constexpr int SLAB = GLU ? 64 : 128;        // output columns per block
  if ((int)blockIdx.x >= tile_count[0]) return;
  const Tile tl = tiles[blockIdx.x];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & 15, kb = lane >> 4;
  const int c0 = blockIdx.y * SLAB;
  const int KB = K / 32;  // scale blocks per row
  const uint8_t* we = w + (size_t)tl.expert * Nw * (K / 2);
  const uint8_t* wse = ws + (size_t)tl.expert * Nw * KB;

  int col[NG];
  bool cok[NG];
  uint32_t frag[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    int c = GLU ? c0 + 16 * (gi & 3) + g : c0 + 16 * gi + g;
    cok[gi] = c < Nout;
    col[gi] = (GLU && gi >= 4) ? Nout + c : c;  // up columns at +I
    if (!cok[gi]) col[gi] = 0;
    // packed codes: chunk c of 16-column group n16 at c * Nw * 64 + n16 KB
    frag[gi] = (uint32_t)(cok[gi] ? (col[gi] - g) / 16 : 0) * 1024u + 16u * lane;
  }
  int arow[RG];
  bool aok[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    int r = 16 * rg + g;
    aok[rg] = r < tl.rows;
    arow[rg] = tl.row0 + (aok[rg] ? r : 0);
  }

  f32x4 acc[NG][RG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[gi][rg] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / 128;
  const int s_begin = wave * nsteps / KSPLIT;
  const int s_end = (wave + 1) * nsteps / KSPLIT;
  for (int s = s_begin; s < s_end; ++s) {
    const int kblk = s * 4 + kb;  // K block of this lane's scales and B data
    i32x8 af[RG];
    int asc[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      // rows past the tile read row 0 of the tile: their outputs are dropped
      const uint8_t* p = a + (size_t)arow[rg] * K + s * 128 + 16 * kb;
      uint4 v0 = *(const uint4*)p;
      uint4 v1 = *(const uint4*)(p + 64);
      af[rg] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                     (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      asc[rg] = as[(size_t)arow[rg] * KB + kblk];
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      // columns past N read column 0: their outputs are never stored
      // lane l: column l%16, K block 4s + l/16 of its 64-byte step chunk
      uint4 v = *(const uint4*)(we + (size_t)s * Nw * 64 + frag[gi]);
      int bsc = wse[(size_t)col[gi] * KB + kblk];
      i32x8 bf = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        acc[gi][rg] = mfma_mx(af[rg], bf, acc[gi][rg], asc[rg], bsc);
    }
  }

  if (KSPLIT > 1) {
    __shared__ float red[(KSPLIT > 1 ? KSPLIT - 1 : 1) * 16 * 64];
    constexpr int NREG = NG * RG * 4;
#pragma unroll
    for (int q = 0; q < NREG / 16; ++q) {
      if (wave > 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int x = q * 16 + j;
          red[((wave - 1) * 16 + j) * 64 + lane] = acc[x / (RG * 4)][(x / 4) % RG][x % 4];
        }
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int x = q * 16 + j;
          float sum = acc[x / (RG * 4)][(x / 4) % RG][x % 4];
#pragma unroll
          for (int ww = 0; ww < KSPLIT - 1; ++ww)
            sum += red[(ww * 16 + j) * 64 + lane];
          acc[x / (RG * 4)][(x / 4) % RG][x % 4] = sum;
        }
      }
      __syncthreads();
    }
    if (wave > 0) return;
  }

  // epilogue: lane holds rows 16*rg + 4*kb + e, column group gi -> col[gi]
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rg + 4 * kb + e;
      const bool rok = r < tl.rows;
      const size_t orow = (size_t)(tl.row0 + (rok ? r : 0));
      if (GLU) {
        // h columns c0 + 16*gi + g for gi = 0..3; MX blocks {0,1} and {2,3}
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float h0 = silu(acc[2 * b][rg][e]) * acc[2 * b + 4][rg][e];
          float h1 = silu(acc[2 * b + 1][rg][e]) * acc[2 * b + 5][rg][e];
          float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
          for (int off = 1; off < 16; off <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off));
          const int sx = mx_e4m3_scale_exp(amax);
          const int cb = c0 + 32 * b;  // first column of the MX block
          if (rok && cb < Nout) {
            uint8_t* o = (uint8_t*)out + orow * Nout + cb;
            o[g] = (uint8_t)e4m3_encode_scaled(h0, sx);
            o[16 + g] = (uint8_t)e4m3_encode_scaled(h1, sx);
            if (g == 0) os[orow * (Nout / 32) + cb / 32] = (uint8_t)(sx + 127);
          }
        }
      } else if (rok) {
        uint16_t* o = (uint16_t*)out + orow * Nout;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          if (cok[gi]) o[col[gi]] = (uint16_t)f32_to_bf16_bits(acc[gi][rg][e]);
      }
    }
  }
}

template <bool GLU, int RG>
static hipError_t launch_mx(int ksplit, dim3 grid, const Tile* tiles,
                            const int32_t* tile_count, const uint8_t* a,
                            const uint8_t* as, const uint8_t* w,
                            const uint8_t* ws, void* out, uint8_t* os, int K,
                            int Nw, int Nout, hipStream_t s) {
  switch (ksplit) {
    case 1:
      hipLaunchKernelGGL((gemm_mx_kernel<GLU, RG, 1>), grid, dim3(64), 0, s,
                         tiles, tile_count, a, as, w, ws, out, os, K, Nw, Nout);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_mx_kernel<GLU, RG, 2>), grid, dim3(128), 0, s,
                         tiles, tile_count, a, as, w, ws, out, os, K, Nw, Nout);
      break;
    default:
      hipLaunchKernelGGL((gemm_mx_kernel<GLU, RG, 4>), grid, dim3(256), 0, s,
                         tiles, tile_count, a, as, w, ws, out, os, K, Nw, Nout);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mx(bool glu, int rg, const Tile* tiles,
                          const int32_t* tile_count, int max_tiles,
                          const uint8_t* a, const uint8_t* a_scale,
                          const uint8_t* w, const uint8_t* w_scale, void* out,
                          uint8_t* out_scale, int K, int Nw, int Nout,
                          hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const int slab = glu ? 64 : 128;
  dim3 grid(max_tiles, (Nout + slab - 1) / slab);
  int steps = K / 128;
  int ksplit = steps >= 16 ? 4 : steps >= 8 ? 2 : 1;
  if (glu)
    return rg == 1 ? launch_mx<true, 1>(ksplit, grid, tiles, tile_count, a,
                                        a_scale, w, w_scale, out, out_scale, K,
                                        Nw, Nout, s)
                   : launch_mx<true, 2>(ksplit, grid, tiles, tile_count, a,
                                        a_scale, w, w_scale, out, out_scale, K,
                                        Nw, Nout, s);
  return rg == 1 ? launch_mx<false, 1>(ksplit, grid, tiles, tile_count, a,
                                       a_scale, w, w_scale, out, out_scale, K,
                                       Nw, Nout, s)
                 : launch_mx<false, 2>(ksplit, grid, tiles, tile_count, a,
                                       a_scale, w, w_scale, out, out_scale, K,
                                       Nw, Nout, s);
}

}  // namespace moe
