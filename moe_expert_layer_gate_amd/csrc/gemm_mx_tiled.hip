// Grouped GEMM, MXFP8 activations x MXFP4 weights on the scaled MFMA,
// LDS-tiled schedule for prefill-size batches.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters": W4A8
// (MXFP4 weights, MXFP8 activations) on the prefill path (overview; Prefill
// optimisation "MXFP8/MXFP4量化"), the AllGather scheme's grouped matmul over
// the local experts (MoE EP优化 / AllGather方案(W4A8量化)) and the expert FFN
// of MoE TP优化 / 计算分解 (down(SiLU(gate(x)) * up(x)), merged gate/up).
//
// Block = WMW x 2 waves, tile = 64*WMW rows x 256 weight columns of one
// expert, K steps of 128 through an LDS ring filled by direct global -> LDS
// copies (16 bytes per lane, no VGPRs involved):
//   * WMW = 2: 128-row tiles, 256 threads, 2-stage ring (one step in
//     flight), two blocks per CU;
//   * WMW = 4: 256-row tiles, 512 threads, 3-stage ring (two steps in flight,
//     150 KB of LDS), one block per CU: 1.5x the bytes in flight per CU and
//     half the weight bytes per flop of the 128-row shape.
// Both operands are K-contiguous in HBM and in LDS, so nothing is transposed:
//   * A (e4m3 codes): LDS [row][8 x 16 B], the 16-byte piece index XOR-ed
//     with (row / 2) % 8: with 128-byte rows, the 16 rows one MFMA operand
//     read touches then cover all 64 banks once (row parity picks the half);
//   * B (e2m1 codes): LDS [column][4 x 16 B], piece index XOR-ed with
//     (column / 4) % 4 for the same reason;
//   * the e8m0 scales (one word = the step's four 32-K blocks per row or
//     column) ride along in the same stage, 4 bytes per lane, and each lane
//     reads back the byte of its K block.
// v_mfma_scale_f32_16x16x128_f8f6f4 operand layout (lane l, q = l/16; see the
// streaming MX kernel): A row l%16 bytes from K [16q,+16) and [64+16q,+16); B
// column l%16 bytes from K [32q,+32); scales of K block q. Each wave owns
// 64 rows x 128 weight columns: 4 x 8 MFMAs per step, 128 fp32 accumulators;
// 32-row halves past the tile's rows are skipped.
// GEMM1 tiles hold 128 gate and the 128 matching up columns; a wave takes 64
// of each so SwiGLU and the MXFP8 quantisation of h (amax over 32 columns =
// 16 lanes x 2 groups) stay inside the wave. Epilogues stage through LDS and
// store 16-byte rows. Blocks are remapped XCD-contiguously as in the bf16
// tiled kernel.
#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {

namespace {

constexpr int MBNW = 256, MBK = 128;
constexpr int MB_BYTES = MBNW * MBK / 2;      // 16 KB of e2m1

// Tile geometry for WMW 64-row wave groups.
template <int WMW>
struct MxCfg {
  static constexpr int NW = 2 * WMW;                 // waves
  static constexpr int MBM = 64 * WMW;               // tile rows
  static constexpr int MA_BYTES = MBM * MBK;         // 16 / 32 KB of e4m3
  static constexpr int MSA = MA_BYTES + MB_BYTES;    // row scale words
  static constexpr int MSB = MSA + MBM * 4;          // column scale words
  static constexpr int MSTAGE = MSB + MBNW * 4;      // 33.5 / 50 KB
  static constexpr int NSTAGE = WMW == 4 ? 3 : 2;
  static constexpr int BLOCKS_PER_CU = WMW == 4 ? 1 : 2;
  // copies per wave and step with WMW == 4: 4 (A) + 2 (B) + 1 (scales)
  static constexpr int NI = 7;
};

// 4 bytes per lane, global (base + lane offset) -> LDS at lds_wave_base +
// 4 * lane; same conventions as g2lds
MOE_DEV void g2lds4(const void* base, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_wave_base)
      : "memory");
}

MOE_DEV f32x4 mfma_mx(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa,
                                                          0, sb);
}

}  // namespace

template <bool GLU, int WMW>
__global__ __launch_bounds__(128 * WMW, MxCfg<WMW>::BLOCKS_PER_CU) void gemm_mx_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    void* __restrict__ out, uint8_t* __restrict__ os, int K, int Nw, int Nout,
    int nslabs, const int32_t* __restrict__ gidx,
    const int32_t* __restrict__ gbase, int gk) {
  using C = MxCfg<WMW>;
  constexpr int NW = C::NW, MBM = C::MBM, MA_BYTES = C::MA_BYTES;
  constexpr int MSA = C::MSA, MSB = C::MSB, MSTAGE = C::MSTAGE;
  constexpr int NSTAGE = C::NSTAGE, NI = C::NI;
  static_assert(NSTAGE == 2 || NW == 8, "a 3-stage ring needs uniform copy counts");
  __shared__ __align__(1024) uint8_t smem[NSTAGE * MSTAGE];
  const int nb = tile_count[0] * nslabs;
  const int b = blockIdx.x;
  if (b >= nb) return;
  const int per = nb / 8, rem = nb % 8, xcd = b % 8;
  const int L = xcd * per + min(xcd, rem) + b / 8;
  const Tile tl = tiles[L / nslabs];
  const int slab = L % nslabs;
  const int c0 = slab * (GLU ? MBNW / 2 : MBNW);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int KB = K / 32;
  const uint8_t* we = w + (size_t)tl.expert * Nw * (K / 2);
  const uint8_t* wse = ws + (size_t)tl.expert * Nw * KB;
  // A rows: the tile's rows of the permuted codes, or with a gather index
  // the token rows of the per-token codes (32-bit offsets, checked by the
  // host)
  const uint8_t* a_tile = gidx ? a : a + (size_t)tl.row0 * K;
  const uint8_t* as_tile = gidx ? as : as + (size_t)tl.row0 * KB;
  const int32_t* grow = gidx ? gidx + gbase[0] + tl.row0 : nullptr;

  // weight column of tile column t (0..255); columns past Nout read column 0
  auto wcol = [&](int t) -> int {
    int oc, col;
    if (GLU) {
      oc = c0 + (t & (MBNW / 2 - 1));
      col = t < MBNW / 2 ? oc : Nout + oc;
    } else {
      oc = c0 + t;
      col = oc;
    }
    return oc < Nout ? col : 0;
  };
  // tile rows past the tile read its row 0 (their outputs are never stored)
  auto arow = [&](int r) -> int {
    const int rr = r < tl.rows ? r : 0;
    return grow ? grow[rr] / gk : rr;
  };

  // ---- copy assignment: each instruction of a wave moves 1 KB.
  // A (4 per wave, j = 0..3): rows 8*(NW*j + wave) + lane/8, physical piece
  //    lane%8 <- logical piece (lane%8) ^ ((row/2)%8); (row/2)%8 =
  //    4*(wave%2) + lane/16 here.
  // B (16/NW per wave): columns 16*(NW*j + wave) + lane/4, physical piece
  //    lane%4 <- logical piece (lane%4) ^ ((column/4)%4); (column/4)%4 =
  //    (lane/16)%4 here.
  constexpr int NB = 16 / NW;
  uint32_t a_off[4], b_off[NB];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * (NW * j + wave) + (lane >> 3);
    a_off[j] = (uint32_t)arow(r) * K +
               16 * ((lane & 7) ^ (4 * (wave & 1) + (lane >> 4)));
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int t = 16 * (NW * j + wave) + (lane >> 2);
    b_off[j] = (uint32_t)wcol(t) * (K / 2) + 16 * ((lane & 3) ^ (lane >> 4));
  }
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds0 + 8 * wave * MBK);
  const uint32_t b_dst =
      __builtin_amdgcn_readfirstlane(lds0 + MA_BYTES + 16 * wave * (MBK / 2));

  // scale words: waves w < MBM/64 copy rows 64*w + lane; the last four waves
  // copy tile columns 64*(w - NW + 4) + lane
  const bool sa_wave = wave < MBM / 64;
  const int sbw = wave - (NW - 4);
  const bool sb_wave = sbw >= 0;
  const uint32_t sa_doff = (uint32_t)arow((64 * wave + lane) & (MBM - 1)) * KB;
  const uint32_t sb_doff = (uint32_t)wcol((64 * sbw + lane) & (MBNW - 1)) * KB;
  const uint32_t sa_dst = __builtin_amdgcn_readfirstlane(
      lds0 + MSA + 64 * 4 * (wave & (MBM / 64 - 1)));
  const uint32_t sb_dst = __builtin_amdgcn_readfirstlane(
      lds0 + MSB + 64 * 4 * (sbw & 3));

  // loads of K step s_ into stage st_
#define MOE_MX_ISSUE(s_, st_)                                                 \
  do {                                                                        \
    const uint8_t* ab_ = a_tile + (size_t)(s_) * MBK;                         \
    const uint8_t* bb_ = we + (size_t)(s_) * (MBK / 2);                       \
    const uint32_t o_ = (st_) * MSTAGE;                                       \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                             \
      g2lds(ab_, a_off[j], a_dst + o_ + 8 * NW * j * MBK);                    \
    _Pragma("unroll") for (int j = 0; j < NB; ++j)                            \
      g2lds(bb_, b_off[j], b_dst + o_ + 16 * NW * j * (MBK / 2));             \
    if (sa_wave) g2lds4(as_tile + 4 * (s_), sa_doff, sa_dst + o_);            \
    if (sb_wave) g2lds4(wse + 4 * (s_), sb_doff, sb_dst + o_);                \
  } while (0)

  // ---- operand reads. A of 16-row block mb: row wm*64 + 16*mb + lane%16,
  // logical pieces q and 4+q; B of group g: tile column bcol(g), piece q.
  const int lr = lane & 15, q = lane >> 4;
  uint32_t a_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    a_rd[h] = lds0 + (wm * 64 + lr) * MBK + 16 * ((4 * h + q) ^ (lr >> 1));
  auto bcol = [&](int g) -> int {
    if (GLU) return (g < 4 ? 0 : MBNW / 2) + wn * 64 + (g & 3) * 16 + lr;
    return wn * 128 + g * 16 + lr;
  };
  const uint32_t b_rd =
      lds0 + MA_BYTES + bcol(0) * (MBK / 2) + 16 * (q ^ (lr >> 2));

  // scale bytes of this lane: row wm*64 + 16*mb + lane%16 and tile column
  // bcol(g), byte q (K block 4s + q)
  const uint32_t sa_rd = lds0 + MSA + (wm * 64 + lr) * 4 + q;
  const uint32_t sb_rd = lds0 + MSB + bcol(0) * 4 + q;
#define MOE_MX_LDS_U8(a_) \
  ((int)*(const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(a_))

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one K step from stage st_ with scale words sa_/sb_; NMB_ 16-row blocks.
  // Two halves of four column groups each: the A fragments and the first
  // half's B fragments are read before its MFMAs, the second half's B while
  // they run.
#define MOE_MX_HALF(st_, NMB_, G0_)                                 \
  do {                                                                        \
    u32x4_t fb[4];                                                            \
    _Pragma("unroll") for (int g = 0; g < 4; ++g)                             \
      fb[g] = lds_read_b128(br_ + (bcol((G0_) + g) - bcol(0)) * (MBK / 2));  \
    if ((NMB_) > 0) {                                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, (G0_) ? 8 : 3 * (NMB_) + 8, 0); \
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * (NMB_), 0);             \
    }                                                                         \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                           \
      const i32x8 b8 = i32x8{(int)fb[g].x, (int)fb[g].y, (int)fb[g].z,        \
                             (int)fb[g].w, 0, 0, 0, 0};                       \
      const int sbv = MOE_MX_LDS_U8(sbr_ + (bcol((G0_) + g) - bcol(0)) * 4);  \
      _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb)                   \
        acc[mb][(G0_) + g] = mfma_mx(fa[mb], b8, acc[mb][(G0_) + g],          \
                                     sa[mb], sbv);                            \
    }                                                                         \
  } while (0)
#define MOE_MX_COMPUTE(st_, NMB_)                                             \
  do {                                                                        \
    /* the stage's read bases, recomputed every step (an opaque offset keeps \
       the compiler from holding one set of address registers per stage;     \
       stage offsets past 64 KB do not fit the read's immediate) */          \
    uint32_t so_ = (st_) * MSTAGE;                                            \
    asm volatile("" : "+s"(so_));                                             \
    const uint32_t ar0_ = a_rd[0] + so_, ar1_ = a_rd[1] + so_;                \
    const uint32_t br_ = b_rd + so_, sar_ = sa_rd + so_, sbr_ = sb_rd + so_;  \
    i32x8 fa[4];                                                              \
    int sa[4];                                                                \
    _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb) {                   \
      const u32x4_t v0 = lds_read_b128(ar0_ + mb * 16 * MBK);                 \
      const u32x4_t v1 = lds_read_b128(ar1_ + mb * 16 * MBK);                 \
      fa[mb] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,              \
                     (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};             \
      sa[mb] = MOE_MX_LDS_U8(sar_ + mb * 16 * 4);                             \
    }                                                                         \
    MOE_MX_HALF(st_, NMB_, 0);                                                \
    MOE_MX_HALF(st_, NMB_, 4);                                                \
  } while (0)

  // step t_ (stage st_ = t_ % NSTAGE): wait until its copies landed (the
  // NI copies per wave of step t+1 may still be in flight in a 3-stage
  // ring), then every wave is done with the stage of step t-1; refill it
  // with step t + NSTAGE - 1 and multiply.
#define MOE_MX_STEP(t_, st_, NMB_)                                            \
  do {                                                                        \
    if (NSTAGE == 3 && (t_) + 1 < nsteps) MOE_WAIT_VMCNT(NI);                 \
    else MOE_WAIT_VMCNT(0);                                                   \
    __syncthreads();                                                          \
    if ((t_) + NSTAGE - 1 < nsteps)                                           \
      MOE_MX_ISSUE((t_) + NSTAGE - 1, ((st_) + NSTAGE - 1) % NSTAGE);         \
    MOE_MX_COMPUTE(st_, NMB_);                                                \
  } while (0)
// one step per iteration, the stage index at run time: unrolling over the
// ring's stages keeps a set of address registers per stage alive and spills
#define MOE_MX_PIPE(NMB_)                                                     \
  do {                                                                        \
    for (int t = 0; t < nsteps; ++t) MOE_MX_STEP(t, t % NSTAGE, NMB_);        \
  } while (0)

  const int nsteps = K / MBK;
  MOE_MX_ISSUE(0, 0);
  if (NSTAGE == 3 && nsteps > 1) MOE_MX_ISSUE(1, 1);
  // 16-row blocks of this wave's 64 rows that hold tile rows, in pairs
  const int mrows = __builtin_amdgcn_readfirstlane(tl.rows - wm * 64);
  if (mrows > 32) MOE_MX_PIPE(4);
  else if (mrows > 0) MOE_MX_PIPE(2);
  else MOE_MX_PIPE(0);
#undef MOE_MX_PIPE
#undef MOE_MX_STEP
#undef MOE_MX_COMPUTE
#undef MOE_MX_HALF
#undef MOE_MX_LDS_U8
#undef MOE_MX_ISSUE
  __syncthreads();

  // epilogue, staged per wave in the (free) operand buffers
  if (GLU) {
    // h: 64 rows x 64 columns of e4m3 codes per wave + 2 scales per row
    uint8_t* st = smem + wave * (64 * 64);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = mb * 16 + 4 * q + e;  // row within the wave's 64
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const float h0 = silu_fast(acc[mb][2 * bb][e]) * acc[mb][2 * bb + 4][e];
          const float h1 = silu_fast(acc[mb][2 * bb + 1][e]) * acc[mb][2 * bb + 5][e];
          float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
          for (int off = 1; off < 16; off <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off));
          const int sx = mx_e4m3_scale_exp(amax);
          st[r * 64 + 32 * bb + lr] = (uint8_t)e4m3_encode_fast(h0, sx);
          st[r * 64 + 32 * bb + 16 + lr] = (uint8_t)e4m3_encode_fast(h1, sx);
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
    uint16_t* st = (uint16_t*)smem + wave * (32 * 128);
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

template <int WMW>
static hipError_t launch_mx(bool glu, dim3 grid, const Tile* tiles,
                            const int32_t* tile_count, const uint8_t* a,
                            const uint8_t* a_scale, const uint8_t* w,
                            const uint8_t* w_scale, void* out,
                            uint8_t* out_scale, int K, int Nw, int Nout,
                            int nslabs, const int32_t* gidx,
                            const int32_t* gbase, int gk, hipStream_t s) {
  if (glu)
    hipLaunchKernelGGL((gemm_mx_tiled_kernel<true, WMW>), grid,
                       dim3(128 * WMW), 0, s, tiles, tile_count, a, a_scale, w,
                       w_scale, out, out_scale, K, Nw, Nout, nslabs, gidx,
                       gbase, gk);
  else
    hipLaunchKernelGGL((gemm_mx_tiled_kernel<false, WMW>), grid,
                       dim3(128 * WMW), 0, s, tiles, tile_count, a, a_scale, w,
                       w_scale, out, out_scale, K, Nw, Nout, nslabs, gidx,
                       gbase, gk);
  return hipGetLastError();
}

hipError_t launch_gemm_mx_tiled(bool glu, int mt, const Tile* tiles,
                                const int32_t* tile_count, int max_tiles,
                                const uint8_t* a, const uint8_t* a_scale,
                                const uint8_t* w, const uint8_t* w_scale,
                                void* out, uint8_t* out_scale, int K, int Nw,
                                int Nout, const int32_t* gidx,
                                const int32_t* gbase, int gk, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  if (mt != 128 && mt != 256) return hipErrorInvalidValue;
  const int slab = glu ? MBNW / 2 : MBNW;
  const int nslabs = (Nout + slab - 1) / slab;
  dim3 grid((unsigned)max_tiles * nslabs);
  return mt == 256 ? launch_mx<4>(glu, grid, tiles, tile_count, a, a_scale, w,
                                  w_scale, out, out_scale, K, Nw, Nout, nslabs,
                                  gidx, gbase, gk, s)
                   : launch_mx<2>(glu, grid, tiles, tile_count, a, a_scale, w,
                                  w_scale, out, out_scale, K, Nw, Nout, nslabs,
                                  gidx, gbase, gk, s);
}

}  // namespace moe
