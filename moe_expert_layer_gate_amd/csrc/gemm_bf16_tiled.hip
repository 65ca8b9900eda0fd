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
//   * B (weights [K, N], N contiguous) is copied to LDS unchanged, [k][n],
//     with 512 contiguous bytes per row and 16-byte stores, and read back
//     K-packed with ds_read_b64_tr_b16: within each group of 16 lanes, source
//     lane s supplies row kb + s/4, columns n0 + 4*(s%4) .. +3, and lane j
//     receives column n0 + j at rows kb .. kb+3 (transpose semantics measured
//     with an in-bounds probe of the instruction); two such reads give the
//     8 consecutive K of an MFMA B fragment;
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
typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BNW = 256, BK = 32;
constexpr int LDK = BK + 8;      // A row in LDS: 80 B
constexpr int LDN = BNW + 16;    // B row in LDS: 544 B

MOE_DEV f32x16 mfma32(u32x4_t a, u32x4_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

MOE_DEV v4i16_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(p));
}

struct Smem {
  uint16_t a[2][BM][LDK];
  uint16_t b[2][BK][LDN];
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
  // B: 16-byte pieces p = tid + 256*j: row p/32 of the step, tile columns
  // 8*(p%32) .. +8 (32 lanes per 512-byte row)
  const int bc = tid & 31, bk = tid >> 5;
  int bcol;
  {
    const int j = 8 * bc;  // tile column
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
  const uint16_t* b_src = we + (size_t)bk * Nw + bcol;

  // the prefetch registers are plain locals written and read in fully
  // unrolled code (no lambda captures), so they stay in VGPRs
#define MOE_TILED_GLOAD(s_)                                                 \
  do {                                                                      \
    const int k0_ = (s_) * BK;                                              \
    ra0 = *(const uint4*)(a_src[0] + k0_);                                  \
    ra1 = *(const uint4*)(a_src[1] + k0_);                                  \
    rb0 = *(const uint4*)(b_src + (size_t)(k0_ + 0) * Nw);                  \
    rb1 = *(const uint4*)(b_src + (size_t)(k0_ + 8) * Nw);                  \
    rb2 = *(const uint4*)(b_src + (size_t)(k0_ + 16) * Nw);                 \
    rb3 = *(const uint4*)(b_src + (size_t)(k0_ + 24) * Nw);                 \
  } while (0)
#define MOE_TILED_LSTORE(buf_)                                              \
  do {                                                                      \
    *(uint4*)&sm.a[buf_][(tid >> 2)][8 * a_kc] = ra0;                       \
    *(uint4*)&sm.a[buf_][(tid >> 2) + 64][8 * a_kc] = ra1;                  \
    *(uint4*)&sm.b[buf_][bk + 0][8 * bc] = rb0;                             \
    *(uint4*)&sm.b[buf_][bk + 8][8 * bc] = rb1;                             \
    *(uint4*)&sm.b[buf_][bk + 16][8 * bc] = rb2;                            \
    *(uint4*)&sm.b[buf_][bk + 24][8 * bc] = rb3;                            \
  } while (0)
  uint4 ra0, ra1, rb0, rb1, rb2, rb3;

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
  // transpose-read coordinates: group g = lane/16, source lane s = lane%16
  const int tr_k = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_n = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
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
        const uint16_t* p = &sm.b[buf][kk * 16 + tr_k][bblock(nbk) + tr_n];
        const v4i16_t lo = lds_read_tr(p);
        const v4i16_t hi = lds_read_tr(p + 4 * LDN);
        fb[nbk] = __builtin_bit_cast(
            u32x4_t, (short __attribute__((ext_vector_type(8)))){
                         lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nbk = 0; nbk < 4; ++nbk)
          acc[mb][nbk] = mfma32(fa[mb], fb[nbk], acc[mb][nbk]);
    }
  };

  const int nsteps = K / BK;
  MOE_TILED_GLOAD(0);
  MOE_TILED_LSTORE(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) MOE_TILED_GLOAD(s + 1);
    compute(buf);
    if (s + 1 < nsteps) MOE_TILED_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef MOE_TILED_GLOAD
#undef MOE_TILED_LSTORE

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
