// Grouped GEMM, bf16 x bf16 -> fp32 on MFMA, LDS-tiled schedule for
// prefill-size batches (many rows per expert).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// MoE TP优化 / 计算分解 (expert = down(SiLU(gate(x)) * up(x)), merged gate/up
// weights, npu_swiglu = SiLU(first half) * second half) and 高性能专家计算
// (all experts in one grouped operator); prefill operators are compute-bound
// (Prefill优化 / 并行策略选择).
//
// Block = 256 threads (2 x 2 waves) computing a 128-row x 256-weight-column
// tile of one expert, K in steps of 32 through double-buffered LDS:
//   * A (activation rows, K contiguous) is copied to LDS as [row][k];
//   * B (weights [K, N], N contiguous) is loaded as 4x8 blocks (4 rows x 16
//     bytes per thread, 128 contiguous bytes per 8 threads) and transposed in
//     registers into [n][k] so both MFMA operands are single 16-byte LDS reads;
//   * v_mfma_f32_32x32x16_bf16: each wave owns 64 rows x 128 weight columns
//     (2 x 4 blocks of 32 x 32, 128 fp32 accumulators);
//   * GEMM1 tiles hold 128 gate columns and the 128 matching up columns; a
//     wave takes 64 of each, so SwiGLU is lane-local in the epilogue;
//   * the epilogue stages each wave's 32-row slice through LDS and writes
//     16-byte rows to HBM;
//   * blocks are remapped so each XCD works on a contiguous range of
//     (tile, slab) pairs: the m-tiles of one expert and one weight slab run on
//     the same XCD and share its L2.
// The next K step's global loads are issued before the current step's MFMAs.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BNW = 256, BK = 32, LDK = BK + 8;  // LDS row: 80 B

MOE_DEV f32x16 mfma32(u32x4_t a, u32x4_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

struct Smem {
  uint16_t a[2][BM][LDK];
  uint16_t b[2][BNW][LDK];
};

}  // namespace

template <bool GLU>
// two blocks per CU: 2 waves per SIMD, LDS for two double-buffered tiles
__global__ __launch_bounds__(256, 2) void gemm_bf16_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ out, int K, int Nw, int Nout, int nslabs) {
  __shared__ __align__(16) Smem sm;
  // XCD-aware remap of the active blocks (dispatch is round-robin over 8 XCDs)
  const int nb = tile_count[0] * nslabs;
  const int b = blockIdx.x;
  if (b >= nb) return;
  const int per = nb / 8, rem = nb % 8, xcd = b % 8;
  const int L = xcd * per + min(xcd, rem) + b / 8;
  const Tile tl = tiles[L / nslabs];
  const int slab = L % nslabs;
  const int c0 = slab * (GLU ? BNW / 2 : BNW);  // first output column

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* we = w + (size_t)tl.expert * K * Nw;

  // global -> register assignment
  // A: rows tid/4 and 64 + tid/4, 8 halves at k = 8*(tid%4)
  const int a_kc = tid & 3;
  const uint16_t* a_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (tid >> 2) + 64 * j;
    a_src[j] = a + (size_t)(tl.row0 + (r < tl.rows ? r : 0)) * K + 8 * a_kc;
  }
  // B: weight columns 8*cg .. +8 of the tile, rows 4*kg .. +4 of the step
  const int cg = tid >> 3, kg = tid & 7;
  int bcol;
  {
    const int j = 8 * cg;  // tile column
    int col, oc;
    if (GLU) {
      oc = c0 + (j & (BNW / 2 - 1));
      col = j < BNW / 2 ? oc : Nout + oc;
    } else {
      oc = c0 + j;
      col = oc;
    }
    bcol = oc < Nout ? col : 0;  // unused columns read column 0
  }
  const uint16_t* b_src = we + (size_t)(4 * kg) * Nw + bcol;

  uint4 ra[2], rb[4];
  auto gload = [&](int s) {
    const int k0 = s * BK;
#pragma unroll
    for (int j = 0; j < 2; ++j) ra[j] = *(const uint4*)(a_src[j] + k0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      rb[r] = *(const uint4*)(b_src + (size_t)(k0 + r) * Nw);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *(uint4*)&sm.a[buf][(tid >> 2) + 64 * j][8 * a_kc] = ra[j];
    // transpose 4 rows x 8 columns -> 8 columns x 4 k (8 bytes each)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      auto dw = [&](int r) -> uint32_t {
        const int d = i >> 1;
        return d == 0 ? rb[r].x : d == 1 ? rb[r].y : d == 2 ? rb[r].z : rb[r].w;
      };
      uint2 v;
      v.x = __builtin_amdgcn_perm(dw(1), dw(0), sel);
      v.y = __builtin_amdgcn_perm(dw(3), dw(2), sel);
      *(uint2*)&sm.b[buf][8 * cg + i][4 * kg] = v;
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // B-tile column block of wave column wn, block nb (0..3)
  auto bblock = [&](int nbk) -> int {
    if (GLU) return (nbk < 2 ? 0 : BNW / 2) + wn * 64 + (nbk & 1) * 32;
    return wn * 128 + nbk * 32;
  };
  const int lr = lane & 31, lk = 8 * (lane >> 5);
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4_t fa[2], fb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        uint4 v = *(const uint4*)&sm.a[buf][wm * 64 + mb * 32 + lr][kk * 16 + lk];
        fa[mb] = u32x4_t{v.x, v.y, v.z, v.w};
      }
#pragma unroll
      for (int nbk = 0; nbk < 4; ++nbk) {
        uint4 v = *(const uint4*)&sm.b[buf][bblock(nbk) + lr][kk * 16 + lk];
        fb[nbk] = u32x4_t{v.x, v.y, v.z, v.w};
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nbk = 0; nbk < 4; ++nbk)
          acc[mb][nbk] = mfma32(fa[mb], fb[nbk], acc[mb][nbk]);
    }
  };

  const int nsteps = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
    compute(buf);
    if (s + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue through LDS: each wave stages 32 rows at a time in its own
  // region of the (now free) B buffers
  uint16_t* stage = &sm.b[0][0][0] + wave * (32 * 128);
  const int ncols = GLU ? 64 : 128;  // output columns of this wave
  const int oc0 = c0 + wn * ncols;   // first output column of this wave
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    // acc element e of a 32x32 block: row 8*(e/4) + 4*(lane/32) + e%4,
    // column lane%32
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (GLU) {
#pragma unroll
        for (int gb = 0; gb < 2; ++gb) {
          const float hv = silu(acc[mb][gb][e]) * acc[mb][gb + 2][e];
          stage[r * 128 + gb * 32 + lr] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int nbk = 0; nbk < 4; ++nbk)
          stage[r * 128 + nbk * 32 + lr] =
              (uint16_t)f32_to_bf16_bits(acc[mb][nbk][e]);
      }
    }
    // each lane writes 16-byte pieces of the staged rows
    const int chunks = ncols / 8;  // 16-byte pieces per row
#pragma unroll
    for (int it = 0; it < 32 * (GLU ? 8 : 16) / 64; ++it) {
      const int q = it * 64 + lane;
      const int r = q / chunks, c = q % chunks;
      const int row = wm * 64 + mb * 32 + r;
      const int col = oc0 + 8 * c;
      if (row < tl.rows && col < Nout)
        *(uint4*)(out + (size_t)(tl.row0 + row) * Nout + col) =
            *(const uint4*)&stage[r * 128 + 8 * c];
    }
  }
}

hipError_t launch_gemm_bf16_tiled(bool glu, const Tile* tiles,
                                  const int32_t* tile_count, int max_tiles,
                                  const uint16_t* a, const uint16_t* w,
                                  uint16_t* out, int K, int Nw, int Nout,
                                  hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const int slab = glu ? BNW / 2 : BNW;
  const int nslabs = (Nout + slab - 1) / slab;
  dim3 grid((unsigned)max_tiles * nslabs);
  if (glu)
    hipLaunchKernelGGL(gemm_bf16_tiled_kernel<true>, grid, dim3(256), 0, s,
                       tiles, tile_count, a, w, out, K, Nw, Nout, nslabs);
  else
    hipLaunchKernelGGL(gemm_bf16_tiled_kernel<false>, grid, dim3(256), 0, s,
                       tiles, tile_count, a, w, out, K, Nw, Nout, nslabs);
  return hipGetLastError();
}

}  // namespace moe
