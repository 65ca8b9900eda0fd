// Grouped GEMM, MXFP8 activations x MXFP4 weights on the scaled MFMA,
// LDS-tiled schedule for prefill-size batches.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters": W4A8
// (MXFP4 weights, MXFP8 activations) on the prefill path (overview; Prefill
// optimisation "MXFP8/MXFP4量化"), the AllGather scheme's grouped matmul over
// the local experts (MoE EP优化 / AllGather方案(W4A8量化)) and the expert FFN
// of MoE TP优化 / 计算分解 (down(SiLU(gate(x)) * up(x)), merged gate/up).
//
// Block = 256 threads (2 x 2 waves), tile = 128 rows x 256 weight columns of
// one expert, K steps of 128 through double-buffered LDS. Both operands are
// K-contiguous in HBM and in LDS ([row][128 B] for e4m3 activations,
// [column][64 B] for e2m1 weights, plus one 4-byte word of e8m0 scales per
// row / column and step), so no transposition is needed anywhere.
// v_mfma_scale_f32_16x16x128_f8f6f4 operand layout (lane l, q = l/16; see the
// streaming MX kernel): A row l%16 bytes from K [16q,+16) and [64+16q,+16); B
// column l%16 bytes from K [32q,+32); scales of K block q. Each wave owns
// 64 rows x 128 weight columns: 4 x 8 MFMAs per step, 128 fp32 accumulators.
// GEMM1 tiles hold 128 gate and the 128 matching up columns; a wave takes 64
// of each so SwiGLU and the MXFP8 quantisation of h (amax over 32 columns =
// 16 lanes x 2 groups) stay inside the wave. Epilogues stage through LDS and
// store 16-byte rows. Blocks are remapped XCD-contiguously as in the bf16
// tiled kernel.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int MBM = 128, MBNW = 256, MBK = 128;
constexpr int LDA = MBK + 16;      // 144 B per activation row in LDS
constexpr int LDB = MBK / 2 + 16;  // 80 B per weight column in LDS

struct MxSmem {
  uint8_t a[2][MBM][LDA];
  uint8_t b[2][MBNW][LDB];
  uint32_t as[2][MBM];
  uint32_t bs[2][MBNW];
};

MOE_DEV f32x4 mfma_mx(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa,
                                                          0, sb);
}

}  // namespace

template <bool GLU>
// two blocks per CU: 2 waves per SIMD, LDS for two double-buffered tiles
__global__ __launch_bounds__(256, 2) void gemm_mx_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    void* __restrict__ out, uint8_t* __restrict__ os, int K, int Nw, int Nout,
    int nslabs) {
  __shared__ __align__(16) MxSmem sm;
  const int nb = tile_count[0] * nslabs;
  const int b = blockIdx.x;
  if (b >= nb) return;
  const int per = nb / 8, rem = nb % 8, xcd = b % 8;
  const int L = xcd * per + min(xcd, rem) + b / 8;
  const Tile tl = tiles[L / nslabs];
  const int slab = L % nslabs;
  const int c0 = slab * (GLU ? MBNW / 2 : MBNW);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int KB = K / 32;
  const uint8_t* we = w + (size_t)tl.expert * Nw * (K / 2);
  const uint8_t* wse = ws + (size_t)tl.expert * Nw * KB;

  // global -> register assignment, 16-byte pieces p = tid + 256*j (j < 4):
  // A piece p = row p/8, bytes 16*(p%8) of the step (8 lanes per 128-byte
  // row); B piece p = tile column p/4, bytes 16*(p%4) (4 lanes per 64-byte
  // column slice). Scales: one 4-byte word per row (tid < 128) and column.
  size_t a_off[4];
  int b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = tid + 256 * j;
    const int r = p >> 3;
    a_off[j] = (size_t)(tl.row0 + (r < tl.rows ? r : 0)) * K + 16 * (p & 7);
    const int t = p >> 2;
    int oc, col;
    if (GLU) {
      oc = c0 + (t & (MBNW / 2 - 1));
      col = t < MBNW / 2 ? oc : Nout + oc;
    } else {
      oc = c0 + t;
      col = oc;
    }
    if (oc >= Nout) col = 0;  // unused columns read column 0
    b_off[j] = col * (K / 2) + 16 * (p & 3);
  }
  const int sr = tid & (MBM - 1);
  const uint32_t* as_src = (const uint32_t*)(as + (size_t)(tl.row0 + (sr < tl.rows ? sr : 0)) * KB);
  int scol, soc;
  if (GLU) {
    soc = c0 + (tid & (MBNW / 2 - 1));
    scol = tid < MBNW / 2 ? soc : Nout + soc;
  } else {
    soc = c0 + tid;
    scol = soc;
  }
  if (soc >= Nout) scol = 0;
  const uint32_t* bs_src = (const uint32_t*)(wse + (size_t)scol * KB);

  // prefetch registers: plain locals in fully unrolled code (no lambda
  // captures), so they stay in VGPRs
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  uint32_t rsa = 0, rsb = 0;
#define MOE_MX_GLOAD(s_)                                                    \
  do {                                                                      \
    const int so_ = (s_);                                                   \
    ra0 = *(const uint4*)(a + a_off[0] + so_ * MBK);                        \
    ra1 = *(const uint4*)(a + a_off[1] + so_ * MBK);                        \
    ra2 = *(const uint4*)(a + a_off[2] + so_ * MBK);                        \
    ra3 = *(const uint4*)(a + a_off[3] + so_ * MBK);                        \
    rb0 = *(const uint4*)(we + (size_t)b_off[0] + so_ * (MBK / 2));         \
    rb1 = *(const uint4*)(we + (size_t)b_off[1] + so_ * (MBK / 2));         \
    rb2 = *(const uint4*)(we + (size_t)b_off[2] + so_ * (MBK / 2));         \
    rb3 = *(const uint4*)(we + (size_t)b_off[3] + so_ * (MBK / 2));         \
    if (tid < MBM) rsa = as_src[so_];                                       \
    rsb = bs_src[so_];                                                      \
  } while (0)
#define MOE_MX_LSTORE(buf_)                                                 \
  do {                                                                      \
    *(uint4*)&sm.a[buf_][(tid >> 3)][16 * (tid & 7)] = ra0;                 \
    *(uint4*)&sm.a[buf_][(tid >> 3) + 32][16 * (tid & 7)] = ra1;            \
    *(uint4*)&sm.a[buf_][(tid >> 3) + 64][16 * (tid & 7)] = ra2;            \
    *(uint4*)&sm.a[buf_][(tid >> 3) + 96][16 * (tid & 7)] = ra3;            \
    *(uint4*)&sm.b[buf_][(tid >> 2)][16 * (tid & 3)] = rb0;                 \
    *(uint4*)&sm.b[buf_][(tid >> 2) + 64][16 * (tid & 3)] = rb1;            \
    *(uint4*)&sm.b[buf_][(tid >> 2) + 128][16 * (tid & 3)] = rb2;           \
    *(uint4*)&sm.b[buf_][(tid >> 2) + 192][16 * (tid & 3)] = rb3;           \
    if (tid < MBM) sm.as[buf_][tid] = rsa;                                  \
    sm.bs[buf_][tid] = rsb;                                                 \
  } while (0)

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, q = lane >> 4;
  // tile column of wave column wn, group g (0..7)
  auto bcolumn = [&](int g) -> int {
    if (GLU) return (g < 4 ? 0 : MBNW / 2) + wn * 64 + (g & 3) * 16 + lr;
    return wn * 128 + g * 16 + lr;
  };
  auto compute = [&](int buf) {
    i32x8 fa[4];
    int sa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = wm * 64 + mb * 16 + lr;
      const uint4 v0 = *(const uint4*)&sm.a[buf][r][16 * q];
      const uint4 v1 = *(const uint4*)&sm.a[buf][r][64 + 16 * q];
      fa[mb] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                     (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      sa[mb] = (sm.as[buf][r] >> (8 * q)) & 0xFF;
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int c = bcolumn(g);
      const uint4 v = *(const uint4*)&sm.b[buf][c][16 * q];
      const i32x8 fb = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      const int sb = (sm.bs[buf][c] >> (8 * q)) & 0xFF;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][g] = mfma_mx(fa[mb], fb, acc[mb][g], sa[mb], sb);
    }
  };

  const int nsteps = K / MBK;
  MOE_MX_GLOAD(0);
  MOE_MX_LSTORE(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) MOE_MX_GLOAD(s + 1);
    compute(buf);
    if (s + 1 < nsteps) MOE_MX_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef MOE_MX_GLOAD
#undef MOE_MX_LSTORE

  // epilogue, staged per wave in the (free) operand buffers
  if (GLU) {
    // h: 64 rows x 64 columns of e4m3 codes per wave + 2 scales per row
    uint8_t* st = &sm.a[0][0][0] + wave * (64 * 64);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = mb * 16 + 4 * q + e;  // row within the wave's 64
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const float h0 = silu(acc[mb][2 * bb][e]) * acc[mb][2 * bb + 4][e];
          const float h1 = silu(acc[mb][2 * bb + 1][e]) * acc[mb][2 * bb + 5][e];
          float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
          for (int off = 1; off < 16; off <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off));
          const int sx = mx_e4m3_scale_exp(amax);
          st[r * 64 + 32 * bb + lr] = (uint8_t)e4m3_encode_scaled(h0, sx);
          st[r * 64 + 32 * bb + 16 + lr] = (uint8_t)e4m3_encode_scaled(h1, sx);
          const int row = wm * 64 + r;
          const int cb = c0 + wn * 64 + 32 * bb;
          if (lr == 0 && row < tl.rows && cb < Nout)
            os[(size_t)(tl.row0 + row) * (Nout / 32) + cb / 32] =
                (uint8_t)(sx + 127);
        }
      }
    }
    // 64 rows x 4 pieces of 16 bytes
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int p = it * 64 + lane, r = p >> 2, c = p & 3;
      const int row = wm * 64 + r, colo = c0 + wn * 64 + 16 * c;
      if (row < tl.rows && colo < Nout)
        *(uint4*)((uint8_t*)out + (size_t)(tl.row0 + row) * Nout + colo) =
            *(const uint4*)&st[r * 64 + 16 * c];
    }
  } else {
    // y: 64 rows x 128 bf16 columns per wave (16 KB), staged 32 rows at a time
    uint16_t* st = (uint16_t*)(&sm.a[0][0][0]) + wave * (32 * 128);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int mb2 = 0; mb2 < 2; ++mb2) {
        const int mb = 2 * h + mb2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = mb2 * 16 + 4 * q + e;
#pragma unroll
          for (int g = 0; g < 8; ++g)
            st[r * 128 + g * 16 + lr] = (uint16_t)f32_to_bf16_bits(acc[mb][g][e]);
        }
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int p = it * 64 + lane, r = p >> 4, c = p & 15;
        const int row = wm * 64 + 32 * h + r, colo = c0 + wn * 128 + 8 * c;
        if (row < tl.rows && colo < Nout)
          *(uint4*)((uint16_t*)out + (size_t)(tl.row0 + row) * Nout + colo) =
              *(const uint4*)&st[r * 128 + 8 * c];
      }
    }
  }
}

hipError_t launch_gemm_mx_tiled(bool glu, const Tile* tiles,
                                const int32_t* tile_count, int max_tiles,
                                const uint8_t* a, const uint8_t* a_scale,
                                const uint8_t* w, const uint8_t* w_scale,
                                void* out, uint8_t* out_scale, int K, int Nw,
                                int Nout, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const int slab = glu ? MBNW / 2 : MBNW;
  const int nslabs = (Nout + slab - 1) / slab;
  dim3 grid((unsigned)max_tiles * nslabs);
  if (glu)
    hipLaunchKernelGGL(gemm_mx_tiled_kernel<true>, grid, dim3(256), 0, s, tiles,
                       tile_count, a, a_scale, w, w_scale, out, out_scale, K,
                       Nw, Nout, nslabs);
  else
    hipLaunchKernelGGL(gemm_mx_tiled_kernel<false>, grid, dim3(256), 0, s,
                       tiles, tile_count, a, a_scale, w, w_scale, out,
                       out_scale, K, Nw, Nout, nslabs);
  return hipGetLastError();
}

}  // namespace moe
