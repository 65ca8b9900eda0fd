// Grouped GEMM, MXFP8 activations x MXFP4 weights on the scaled MFMA,
// LDS-tiled schedule: the W4A8 path at every batch size (on the 4096 x 1536
// experts of the W4A8 workload it beat streaming the weights through
// registers from a single token on).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters": W4A8
// (MXFP4 weights, MXFP8 activations) on the prefill path (overview; Prefill
// optimisation "MXFP8/MXFP4量化"), the AllGather scheme's grouped matmul over
// the local experts (MoE EP优化 / AllGather方案(W4A8量化)) and the expert FFN
// of MoE TP优化 / 计算分解 (down(SiLU(gate(x)) * up(x)), merged gate/up).
//
// Block = 256 threads (2 x 2 waves), tile = 128 rows x 256 weight columns of
// one expert, K steps of 128 through a two-stage LDS ring filled by direct
// global -> LDS copies (16 bytes per lane, no VGPRs involved). Both operands
// are K-contiguous in HBM and in LDS, so nothing is transposed:
//   * A (e4m3 codes): LDS [row][8 x 16 B], the 16-byte piece index XOR-ed
//     with (row / 2) % 8: with 128-byte rows, the 16 rows one MFMA operand
//     read touches then cover all 64 banks once (row parity picks the half);
//   * B (e2m1 codes, packed: 1 KB fragments of 16 columns x one 64-byte K
//     step, 16 bytes of column c, K piece p at 16 (16 p + c)): each copy
//     instruction moves one fragment as it is (one contiguous 1 KB), so LDS
//     holds [16-column group][piece][column]; 16 consecutive lanes reading
//     16 consecutive columns of one piece touch 256 contiguous bytes;
//   * the e8m0 scales have a two-slot ring of their own. When K/32 is a
//     multiple of 16, one 16-byte copy per row (and per column) brings the
//     scales of four K steps at once -- a copy per row or column costs an L2
//     request however few bytes it moves, so batching cuts the requests of
//     the scales fourfold (measured: without any scale copies GEMM1 runs
//     16 % faster); otherwise one 4-byte word per row and step.
// v_mfma_scale_f32_16x16x128_f8f6f4 operand layout on gfx950 (lane l,
// q = l/16; measured with an in-bounds probe of one instruction): A (8
// VGPRs) holds row l%16, bytes 0-15 from K [16q, +16) and bytes 16-31 from
// K [64+16q, +16); B (e2m1, 4 VGPRs) holds column l%16, K [32q, +32); each
// lane's e8m0 scale is that of K block q (K [32q, +32)) of its row / column. Each wave owns
// 64 rows x 128 weight columns: 4 x 8 MFMAs per step, 128 fp32 accumulators;
// 32-row halves past the tile's rows are skipped.
// GEMM1 tiles hold 128 gate and the 128 matching up columns; a wave takes 64
// of each so SwiGLU and the MXFP8 quantisation of h (amax over 32 columns =
// 16 lanes x 2 groups) stay inside the wave. Epilogues stage through LDS and
// store 16-byte rows. Blocks are remapped XCD-contiguously as in the bf16
// tiled kernel. GEMM2 runs a second kernel below on the same tile, ring and
// copies with the 32x32x64 form of the scaled MFMA and fragments double
// buffered across the step's barrier.
#include "common.h"
#include "launch.h"
#include "lds_dma.h"

// Slabs per group of the item order (tile_item): groups of 3 slabs of an
// expert, tile-major inside a group, measured against plain tile-major order
// (every slab of a tile before the next) on the skewed prefills and the W4A8
// rank: layer 479.6 -> 469.3 us (bf16), 332.0 -> 329.6 us (W8A8), 244.8 ->
// 240.0 us (W4A8; its GEMM2 65.6 -> 61.9 us), 1530.6 -> 1507.2 us at 16384
// tokens; groups of 1 (slab-major) or 2 were no better.
// Weights of single-tile experts copied with the nontemporal hint (0: never).
#ifndef MOE_MX_NT_SINGLE
#define MOE_MX_NT_SINGLE 1
#endif

#ifndef MOE_MX_SLAB_GROUP
#define MOE_MX_SLAB_GROUP 3
#endif

namespace moe {

namespace {

constexpr int MBM = 128, MBNW = 256, MBK = 128;
constexpr int MA_BYTES = MBM * MBK;           // 16 KB of e4m3
constexpr int MB_BYTES = MBNW * MBK / 2;      // 16 KB of e2m1
constexpr int MSTAGE = MA_BYTES + MB_BYTES;   // 32 KB per code stage
constexpr int MCODES = 2 * MSTAGE;            // the two code stages

// Scale slot for SCB K steps per copy: [row][4*SCB bytes] then
// [column][4*SCB bytes].
template <int SCB>
struct MxScales {
  static constexpr int ROW = 4 * SCB;                 // bytes per row / column
  static constexpr int SB = MBM * ROW;                // column scales offset
  static constexpr int SLOT = (MBM + MBNW) * ROW;     // 1.5 / 6 KB
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

// GEMM1 + SwiGLU + MXFP8 quantisation of h.
template <int SCB>
// two blocks per CU: 2 waves per SIMD, 67 / 76 KB of LDS each
__global__ __launch_bounds__(256, 2) void gemm_mx_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    void* __restrict__ out, uint8_t* __restrict__ os, int K, int Nw, int Nout,
    int nslabs, int sgroup, const int32_t* __restrict__ gidx,
    const int32_t* __restrict__ gbase, int gk) {
  using S = MxScales<SCB>;
  __shared__ __align__(1024) uint8_t smem[MCODES + 2 * S::SLOT];
  const int nb = tile_count[0] * nslabs;
  const int b = blockIdx.x;
  if (b >= nb) return;
  const int per = nb / 8, rem = nb % 8, xcd = b % 8;
  const int L = xcd * per + min(xcd, rem) + b / 8;
  Tile tl;
  int slab;
  tile_item(tiles, L, nslabs, sgroup, tl, slab);
  const int c0 = slab * (MBNW / 2);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int KB = K / 32;
  const uint8_t* we = w + (size_t)tl.expert * Nw * (K / 2);
  // an expert with one tile is the only reader of its weights: stream them
  const bool wnt = MOE_MX_NT_SINGLE &&
                   __builtin_amdgcn_readfirstlane(tl.count) == 1;
  const uint8_t* wse = ws + (size_t)tl.expert * Nw * KB;
  // A rows: the tile's rows of the permuted codes, or with a gather index
  // the token rows of the per-token codes (32-bit offsets, checked by the
  // host)
  const uint8_t* a_tile = gidx ? a : a + (size_t)tl.row0 * K;
  const uint8_t* as_tile = gidx ? as : as + (size_t)tl.row0 * KB;
  const int32_t* grow = gidx ? gidx + gbase[0] + tl.row0 : nullptr;

  // weight column of tile column t (0..255): gate columns c0 + t for
  // t < 128, the matching up columns at +Nout; columns past Nout read
  // column 0
  auto wcol = [&](int t) -> int {
    const int oc = c0 + (t & (MBNW / 2 - 1));
    const int col = t < MBNW / 2 ? oc : Nout + oc;
    return oc < Nout ? col : 0;
  };
  // tile rows past the tile read its row 0 (their outputs are never stored)
  auto arow = [&](int r) -> int {
    const int rr = r < tl.rows ? r : 0;
    return grow ? grow[rr] / gk : rr;
  };

  // ---- copy assignment: instruction j (0..3) of a wave moves 1 KB.
  // A: rows 8*(4j + wave) + lane/8, physical piece lane%8 <- logical piece
  //    (lane%8) ^ ((row/2)%8); (row/2)%8 = 4*(wave%2) + lane/16 here.
  // B: the packed fragment of tile columns 16*(4j + wave) .. +15, lane l
  //    taking bytes 16 l.
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * (4 * j + wave) + (lane >> 3);
    a_off[j] = (uint32_t)arow(r) * K +
               16 * ((lane & 7) ^ (4 * (wave & 1) + (lane >> 4)));
    b_off[j] = (uint32_t)wcol(16 * (4 * j + wave)) / 16 * 1024u + 16u * lane;
  }
  // A copies whose 8 rows all lie past the tile's rows are skipped: those
  // LDS rows feed only accumulator rows that are never stored
  const int na = __builtin_amdgcn_readfirstlane(
      min(4, (tl.rows - 8 * wave + 31) / 32));
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds0 + 8 * wave * MBK);
  const uint32_t b_dst =
      __builtin_amdgcn_readfirstlane(lds0 + MA_BYTES + 16 * wave * (MBK / 2));

  // scales: waves 0-1 copy rows 64*wave + lane, every wave copies tile
  // columns 64*wave + lane; 4*SCB bytes each, lane l landing at 4*SCB*l
  const uint32_t sa_doff = (uint32_t)arow((64 * wave + lane) & (MBM - 1)) * KB;
  const uint32_t sb_doff = (uint32_t)wcol(64 * wave + lane) * KB;
  const uint32_t ss0 = lds0 + MCODES;
  const uint32_t sa_dst =
      __builtin_amdgcn_readfirstlane(ss0 + 64 * S::ROW * (wave & 1));
  const uint32_t sb_dst =
      __builtin_amdgcn_readfirstlane(ss0 + S::SB + 64 * S::ROW * wave);

  // codes of K step s_ into stage st_ (8 instructions per wave)
#define MOE_MX_ISSUE(s_, st_)                                                 \
  do {                                                                        \
    const uint8_t* ab_ = a_tile + (size_t)(s_) * MBK;                         \
    const uint8_t* bb_ = we + (size_t)(s_) * Nw * (MBK / 2);                  \
    const uint32_t o_ = (st_) * MSTAGE;                                       \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                             \
      if (j < na) g2lds(ab_, a_off[j], a_dst + o_ + 32 * j * MBK);            \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                             \
      g2lds_w(bb_, b_off[j], b_dst + o_ + 64 * j * (MBK / 2), wnt);           \
  } while (0)
  // scales of K steps [SCB*g_, SCB*g_ + SCB) into slot g_ % 2 (1 or 2
  // instructions per wave)
#define MOE_MX_ISSUE_SCALES(g_)                                               \
  do {                                                                        \
    const uint32_t so_ = ((g_) & 1) * S::SLOT;                                \
    const size_t go_ = (size_t)(g_) * S::ROW;                                 \
    if (SCB == 4) {                                                           \
      if (wave < 2) g2lds(as_tile + go_, sa_doff, sa_dst + so_);              \
      g2lds(wse + go_, sb_doff, sb_dst + so_);                                \
    } else {                                                                  \
      if (wave < 2) g2lds4(as_tile + go_, sa_doff, sa_dst + so_);             \
      g2lds4(wse + go_, sb_doff, sb_dst + so_);                               \
    }                                                                         \
  } while (0)

  // ---- operand reads. A of 16-row block mb: row wm*64 + 16*mb + lane%16,
  // logical pieces q and 4+q; B of group g: tile column bcol(g), piece q.
  const int lr = lane & 15, q = lane >> 4;
  uint32_t a_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    a_rd[h] = lds0 + (wm * 64 + lr) * MBK + 16 * ((4 * h + q) ^ (lr >> 1));
  auto bcol = [&](int g) -> int {
    return (g < 4 ? 0 : MBNW / 2) + wn * 64 + (g & 3) * 16 + lr;
  };
  // packed B in LDS: [16-column group][piece][column], 16 B each
  const uint32_t b_rd =
      lds0 + MA_BYTES + (bcol(0) - lr) * (MBK / 2) + 16 * (16 * q + lr);

  // scale bytes of this lane: row wm*64 + 16*mb + lane%16 and tile column
  // bcol(g), byte 4*(s % SCB) + q of the slot (K block 4s + q)
  const uint32_t sa_rd = ss0 + (wm * 64 + lr) * S::ROW + q;
  const uint32_t sb_rd = ss0 + S::SB + bcol(0) * S::ROW + q;
#define MOE_MX_LDS_U8(a_) \
  ((int)*(const __attribute__((address_space(3))) uint8_t*)(uintptr_t)(a_))

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one K step from stage st_; NMB_ 16-row blocks. Every LDS read of the
  // step is issued before its MFMAs: the twelve scale bytes first (each into
  // a register of its own, so no read waits on an MFMA that still needs the
  // previous value), the first four B fragments and the A fragments, then
  // the second four B fragments after the first four MFMAs; the MFMAs go row
  // block by row block, so the first ones wait only for their own operands
  // (LDS reads complete in order). Measured against reading each half's B
  // fragments and scales just before its MFMAs: GEMM1 of the W4A8 rank
  // 130.1 -> 127.7 us (the compiler had put the second half's scale bytes
  // in one register, each read waiting on the MFMAs before it).
#define MOE_MX_COMPUTE(t_, NMB_)                                              \
  do {                                                                        \
    /* read bases of step t_, recomputed every step (opaque offsets keep the \
       compiler from holding a set of address registers per stage) */        \
    uint32_t so_ = ((t_) & 1) * MSTAGE;                                       \
    uint32_t sso_ = (((t_) / SCB) & 1) * S::SLOT + 4 * ((t_) % SCB);          \
    asm volatile("" : "+s"(so_), "+s"(sso_));                                 \
    const uint32_t ar0_ = a_rd[0] + so_, ar1_ = a_rd[1] + so_;                \
    const uint32_t br_ = b_rd + so_, sar_ = sa_rd + sso_, sbr_ = sb_rd + sso_; \
    if ((NMB_) > 0) {                                                         \
      int sa[4], sb[8];                                                       \
      _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb)                   \
        sa[mb] = MOE_MX_LDS_U8(sar_ + mb * 16 * S::ROW);                      \
      _Pragma("unroll") for (int g = 0; g < 8; ++g)                           \
        sb[g] = MOE_MX_LDS_U8(sbr_ + (bcol(g) - bcol(0)) * S::ROW);           \
      u32x4_t fb[8];                                                          \
      _Pragma("unroll") for (int g = 0; g < 4; ++g)                           \
        fb[g] = lds_read_b128(br_ + (bcol(g) - bcol(0)) * (MBK / 2));         \
      i32x8 fa[4];                                                            \
      _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb) {                 \
        const u32x4_t v0 = lds_read_b128(ar0_ + mb * 16 * MBK);               \
        const u32x4_t v1 = lds_read_b128(ar1_ + mb * 16 * MBK);               \
        fa[mb] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,            \
                       (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};           \
      }                                                                       \
      _Pragma("unroll") for (int g = 4; g < 8; ++g)                           \
        fb[g] = lds_read_b128(br_ + (bcol(g) - bcol(0)) * (MBK / 2));         \
      __builtin_amdgcn_sched_group_barrier(0x100, 3 * (NMB_) + 12, 0);        \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 8 * (NMB_) - 4, 0);         \
      _Pragma("unroll") for (int h = 0; h < 2; ++h)                           \
        _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb)                 \
          _Pragma("unroll") for (int g = 4 * h; g < 4 * h + 4; ++g) {         \
            const i32x8 b8 = i32x8{(int)fb[g].x, (int)fb[g].y, (int)fb[g].z,  \
                                   (int)fb[g].w, 0, 0, 0, 0};                 \
            acc[mb][g] = mfma_mx(fa[mb], b8, acc[mb][g], sa[mb], sb[g]);      \
          }                                                                   \
    }                                                                         \
  } while (0)

  // step t_ (stage t_ % 2): its copies landed (issued one step earlier, with
  // the scales of the next batch when t_ + 1 starts one) and every wave is
  // done with the other stage and the other scale slot; refill them, multiply
#define MOE_MX_STEP(t_, NMB_)                                                 \
  do {                                                                        \
    MOE_WAIT_VMCNT(0);                                                        \
    __syncthreads();                                                          \
    if ((t_) + 1 < nsteps) {                                                  \
      MOE_MX_ISSUE((t_) + 1, ((t_) + 1) & 1);                                 \
      if (((t_) + 1) % SCB == 0) MOE_MX_ISSUE_SCALES(((t_) + 1) / SCB);       \
    }                                                                         \
    MOE_MX_COMPUTE(t_, NMB_);                                                 \
  } while (0)
// one step per iteration, stage offsets at run time: unrolling over the
// ring's stages keeps a set of address registers per stage alive and spills
#define MOE_MX_PIPE(NMB_)                                                     \
  do {                                                                        \
    for (int t = 0; t < nsteps; ++t) MOE_MX_STEP(t, NMB_);                    \
  } while (0)

  const int nsteps = K / MBK;
  MOE_MX_ISSUE(0, 0);
  MOE_MX_ISSUE_SCALES(0);
  // 16-row blocks of this wave's 64 rows that hold tile rows, in pairs
  const int mrows = __builtin_amdgcn_readfirstlane(tl.rows - wm * 64);
  if (mrows > 32) MOE_MX_PIPE(4);
  else if (mrows > 0) MOE_MX_PIPE(2);
  else MOE_MX_PIPE(0);
#undef MOE_MX_PIPE
#undef MOE_MX_STEP
#undef MOE_MX_COMPUTE
#undef MOE_MX_LDS_U8
#undef MOE_MX_ISSUE_SCALES
#undef MOE_MX_ISSUE
  __syncthreads();

  // epilogue, staged per wave in the (free) operand buffers
  {
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
          const uint32_t c2 = e4m3x2_hw(h0, h1, sx);
          st[r * 64 + 32 * bb + lr] = (uint8_t)c2;
          st[r * 64 + 32 * bb + 16 + lr] = (uint8_t)(c2 >> 8);
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
  }
}

// ---------------------------------------------------------------------------
// The same tile, ring and copies with v_mfma_scale_f32_32x32x64_f8f6f4.
// Operand layout on gfx950 (measured with an in-bounds probe of one
// instruction; lane l, q = l/32, K relative to the instruction's 64):
//   A (e4m3, 8 VGPRs): row l%32, K [16q, 16q+16) in bytes 0-15 and
//                      [32+16q, 32+16q+16) in bytes 16-31;
//   B (e2m1, 4 VGPRs): column l%32, K [32q, 32q+32);
//   scales: lane l holds the e8m0 of row / column l%32 for K block q.
// Used for GEMM2 (bf16 y). A K step of 128 is two such instructions
// (substeps s = 0, 1). Each wave owns 64 rows x 128 weight columns = 2 x 4
// blocks of 32 x 32; the fragments
// of one substep are 32 registers, so two sets fit: while the MFMAs of one
// substep run, the other's fragments are read, across the step's barrier too
// (read s=1 | multiply s=0 | barrier, refill | read next s=0 | multiply s=1).
// The scale bytes of a step come as one 32-bit LDS read per row / column
// block, repacked per lane (v_perm) so that byte s is block 2s + q; the
// instruction's op_sel picks byte s.
template <int S_>
MOE_DEV f32x16 mfma_mx32(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, S_, sa,
                                                         S_, sb);
}

template <int SCB>
__global__ __launch_bounds__(256, 2) void gemm_mx32_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    uint16_t* __restrict__ out, int K, int Nw, int Nout, int nslabs,
    int sgroup) {
  using S = MxScales<SCB>;
  __shared__ __align__(1024) uint8_t smem[MCODES + 2 * S::SLOT];
  const int nb = tile_count[0] * nslabs;
  const int b = blockIdx.x;
  if (b >= nb) return;
  const int per = nb / 8, rem = nb % 8, xcd = b % 8;
  const int L = xcd * per + min(xcd, rem) + b / 8;
  Tile tl;
  int slab;
  tile_item(tiles, L, nslabs, sgroup, tl, slab);
  const int c0 = slab * MBNW;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int KB = K / 32;
  const uint8_t* we = w + (size_t)tl.expert * Nw * (K / 2);
  // an expert with one tile is the only reader of its weights: stream them
  const bool wnt = MOE_MX_NT_SINGLE &&
                   __builtin_amdgcn_readfirstlane(tl.count) == 1;
  const uint8_t* wse = ws + (size_t)tl.expert * Nw * KB;
  const uint8_t* a_tile = a + (size_t)tl.row0 * K;
  const uint8_t* as_tile = as + (size_t)tl.row0 * KB;
  // weight columns past Nout and tile rows past the tile read column / row 0
  auto wcol = [&](int t) -> int { return c0 + t < Nout ? c0 + t : 0; };
  auto arow = [&](int r) -> int { return r < tl.rows ? r : 0; };

  // copies: as in gemm_mx_tiled_kernel
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 8 * (4 * j + wave) + (lane >> 3);
    a_off[j] = (uint32_t)arow(r) * K +
               16 * ((lane & 7) ^ (4 * (wave & 1) + (lane >> 4)));
    b_off[j] = (uint32_t)wcol(16 * (4 * j + wave)) / 16 * 1024u + 16u * lane;
  }
  // A copies whose 8 rows all lie past the tile's rows are skipped: those
  // LDS rows feed only accumulator rows that are never stored
  const int na = __builtin_amdgcn_readfirstlane(
      min(4, (tl.rows - 8 * wave + 31) / 32));
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds0 + 8 * wave * MBK);
  const uint32_t b_dst =
      __builtin_amdgcn_readfirstlane(lds0 + MA_BYTES + 16 * wave * (MBK / 2));
  const uint32_t sa_doff = (uint32_t)arow((64 * wave + lane) & (MBM - 1)) * KB;
  const uint32_t sb_doff = (uint32_t)wcol(64 * wave + lane) * KB;
  const uint32_t ss0 = lds0 + MCODES;
  const uint32_t sa_dst =
      __builtin_amdgcn_readfirstlane(ss0 + 64 * S::ROW * (wave & 1));
  const uint32_t sb_dst =
      __builtin_amdgcn_readfirstlane(ss0 + S::SB + 64 * S::ROW * wave);

#define MOE_MX_ISSUE(s_, st_)                                                 \
  do {                                                                        \
    const uint8_t* ab_ = a_tile + (size_t)(s_) * MBK;                         \
    const uint8_t* bb_ = we + (size_t)(s_) * Nw * (MBK / 2);                  \
    const uint32_t o_ = (st_) * MSTAGE;                                       \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                             \
      if (j < na) g2lds(ab_, a_off[j], a_dst + o_ + 32 * j * MBK);            \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                             \
      g2lds_w(bb_, b_off[j], b_dst + o_ + 64 * j * (MBK / 2), wnt);           \
  } while (0)
#define MOE_MX_ISSUE_SCALES(g_)                                               \
  do {                                                                        \
    const uint32_t so_ = ((g_) & 1) * S::SLOT;                                \
    const size_t go_ = (size_t)(g_) * S::ROW;                                 \
    if (SCB == 4) {                                                           \
      if (wave < 2) g2lds(as_tile + go_, sa_doff, sa_dst + so_);              \
      g2lds(wse + go_, sb_doff, sb_dst + so_);                                \
    } else {                                                                  \
      if (wave < 2) g2lds4(as_tile + go_, sa_doff, sa_dst + so_);             \
      g2lds4(wse + go_, sb_doff, sb_dst + so_);                               \
    }                                                                         \
  } while (0)

  // ---- operand reads. Lane l: r32 = l%32, q = l/32.
  // A block mb: row wm*64 + 32*mb + r32 (its (row/2)%8 = (r32/2)%8), logical
  // pieces 4s + q and 4s + 2 + q of the 128-byte step row.
  // B block nb: tile column bcol(nb), piece 2s + q of the 64-byte step
  // chunk (packed LDS layout, no swizzle).
  // A: physical piece of logical piece c (bit 0 = q): c ^ swizzle =
  // (c - q) ^ (q ^ swizzle); the row base is 128-byte aligned, so the lane's
  // base ORed with 16 * (q ^ swizzle) only needs the compile-time
  // 16 * (c - q) XORed in per read.
  const int r32 = lane & 31, q = lane >> 5;
  const uint32_t a_rd =
      (lds0 + (wm * 64 + r32) * MBK) | (16 * (q ^ ((r32 >> 1) & 7)));
  auto bcol = [&](int n) -> int { return wn * 128 + n * 32 + r32; };
  // packed B in LDS: [16-column group][piece][column]; piece 2s + q of
  // column bcol(n) at group (bcol/16) KB + 16 (16 (2s + q) + bcol % 16)
  const uint32_t b_rd = lds0 + MA_BYTES + (bcol(0) & ~15) * (MBK / 2) +
                        16 * (16 * q + (bcol(0) & 15));
  // scale words: row / column, bytes 4*(t % SCB) .. +3 of the slot
  const uint32_t sa_rd = ss0 + (wm * 64 + r32) * S::ROW;
  const uint32_t sb_rd = ss0 + S::SB + bcol(0) * S::ROW;
  const uint32_t psel = q ? 0x0c0c0301u : 0x0c0c0200u;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#define MOE_MX32_LDS_U32(a_) \
  (*(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(a_))
  // scales of step t_ (slot of its batch, word t_ % SCB), repacked
#define MOE_MX32_SCALES(t_, sa_, sb_)                                         \
  do {                                                                        \
    uint32_t so_ = (((t_) / SCB) & 1) * S::SLOT + 4 * ((t_) % SCB);           \
    asm volatile("" : "+s"(so_));                                             \
    _Pragma("unroll") for (int mb = 0; mb < 2; ++mb) {                        \
      const uint32_t w_ = MOE_MX32_LDS_U32(sa_rd + so_ + mb * 32 * S::ROW);   \
      sa_[mb] = (int)__builtin_amdgcn_perm(w_, w_, psel);                     \
    }                                                                         \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) {                           \
      const uint32_t w_ =                                                     \
          MOE_MX32_LDS_U32(sb_rd + so_ + (bcol(n) - bcol(0)) * S::ROW);       \
      sb_[n] = (int)__builtin_amdgcn_perm(w_, w_, psel);                      \
    }                                                                         \
  } while (0)
  // fragments of substep ss_ of the step in stage st_ (NMB_ row blocks)
#define MOE_MX32_READ(fa_, fb_, st_, ss_, NMB_)                               \
  do {                                                                        \
    uint32_t so_ = (st_) * MSTAGE;                                            \
    asm volatile("" : "+s"(so_));                                             \
    _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb) {                   \
      const uint32_t r_ = a_rd + so_ + mb * 32 * MBK;                         \
      const u32x4_t v0 = lds_read_b128(r_ ^ (64 * (ss_)));                    \
      const u32x4_t v1 = lds_read_b128(r_ ^ (64 * (ss_) + 32));               \
      fa_[mb] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,             \
                      (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};            \
    }                                                                         \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) {                           \
      const u32x4_t v_ = lds_read_b128(                                       \
          b_rd + so_ + (bcol(n) - bcol(0)) * (MBK / 2) + 512 * (ss_));        \
      fb_[n] = i32x8{(int)v_.x, (int)v_.y, (int)v_.z, (int)v_.w, 0, 0, 0, 0}; \
    }                                                                         \
  } while (0)
#define MOE_MX32_MMA(fa_, fb_, ss_, sa_, sb_, NMB_)                           \
  do {                                                                        \
    _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb)                     \
      _Pragma("unroll") for (int n = 0; n < 4; ++n)                           \
        acc[mb][n] = mfma_mx32<ss_>(fa_[mb], fb_[n], acc[mb][n], sa_[mb],     \
                                    sb_[n]);                                  \
  } while (0)
  // order of a half step: the next fragments' LDS reads first, then the MFMAs
#define MOE_MX32_ORDER(NMB_)                                                  \
  do {                                                                        \
    if ((NMB_) > 0) {                                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (NMB_) + 4, 0);         \
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * (NMB_), 0);             \
    }                                                                         \
  } while (0)
  // One K step t_. NEXT_: a step t_+1 follows (wait for its copies, barrier,
  // read its first fragments); CODES_: refill the freed stage with step t_+2;
  // SC_: with one step per scale batch, also refill the scale slot with step
  // t_+2's scales (its slot held step t_'s, which every wave read before this
  // barrier). All are compile-time, so a step is one basic block: the
  // compiler cannot sink the first half's MFMAs below the barrier (it would,
  // past a branch, since their only use is the second half's MFMAs).
#define MOE_MX32_STEP(t_, NEXT_, CODES_, SC_, NMB_)                           \
  do {                                                                        \
    const int tt_ = __builtin_amdgcn_readfirstlane(t_);                       \
    const int st_ = tt_ & 1;                                                  \
    MOE_MX32_READ(f1a, f1b, st_, 1, NMB_);                                    \
    MOE_MX32_MMA(f0a, f0b, 0, sa, sb, NMB_);                                  \
    MOE_MX32_ORDER(NMB_);                                                     \
    /* the first half's MFMAs are issued before the barrier and run while   \
       the wave waits there */                                                \
    __builtin_amdgcn_sched_barrier(0);                                        \
    if (NEXT_) {                                                              \
      MOE_WAIT_VMCNT(0);                                                      \
      __syncthreads();                                                        \
      if (CODES_) MOE_MX_ISSUE(tt_ + 2, st_);                                 \
      if (SC_) MOE_MX_ISSUE_SCALES(tt_ + 2);                                  \
      MOE_MX32_READ(f0a, f0b, st_ ^ 1, 0, NMB_);                              \
    }                                                                         \
    MOE_MX32_MMA(f1a, f1b, 1, sa, sb, NMB_);                                  \
    MOE_MX32_ORDER(NMB_);                                                     \
    /* next step's scales, read once this step's MFMAs are issued */          \
    if (NEXT_) MOE_MX32_SCALES(tt_ + 1, sa, sb);                              \
  } while (0)
  // steps 0 .. nsteps-3 refill the ring; the last two refill nothing. With
  // four steps per scale batch, the batch that starts at step t+2 is copied
  // at the start of step t: its slot held the batch of steps t-6 .. t-3,
  // which every wave read before step t-2's barrier, and step t's wait
  // covers the copy. The branch comes first in the step so that nothing
  // after it can be sunk.
#define MOE_MX32_PIPE(NMB_)                                                   \
  do {                                                                        \
    i32x8 f0a[2], f0b[4], f1a[2], f1b[4];                                     \
    int sa[2], sb[4];                                                         \
    MOE_MX32_SCALES(0, sa, sb);                                               \
    MOE_MX32_READ(f0a, f0b, 0, 0, NMB_);                                      \
    for (int t = 0; t + 3 <= nsteps; ++t) {                                   \
      if (SCB > 1 && (t + 2) % SCB == 0) MOE_MX_ISSUE_SCALES((t + 2) / SCB);  \
      MOE_MX32_STEP(t, 1, 1, SCB == 1, NMB_);                                 \
    }                                                                         \
    if (nsteps >= 2) MOE_MX32_STEP(nsteps - 2, 1, 0, 0, NMB_);                \
    MOE_MX32_STEP(nsteps - 1, 0, 0, 0, NMB_);                                 \
  } while (0)

  const int nsteps = K / MBK;
  // prologue: step 0 (codes and the first scale batch) landed, step 1 in
  // flight
  MOE_MX_ISSUE(0, 0);
  MOE_MX_ISSUE_SCALES(0);
  MOE_WAIT_VMCNT(0);
  __syncthreads();
  if (nsteps > 1) {
    MOE_MX_ISSUE(1, 1);
    if (1 % SCB == 0) MOE_MX_ISSUE_SCALES(1);
  }
  const int mrows = __builtin_amdgcn_readfirstlane(tl.rows - wm * 64);
  // every wave runs the loop (its copies and barriers), with the MFMAs of
  // row blocks past the tile's rows left out
  if (mrows > 32) MOE_MX32_PIPE(2);
  else if (mrows > 0) MOE_MX32_PIPE(1);
  else MOE_MX32_PIPE(0);
#undef MOE_MX32_PIPE
#undef MOE_MX32_STEP
#undef MOE_MX32_ORDER
#undef MOE_MX32_MMA
#undef MOE_MX32_READ
#undef MOE_MX32_SCALES
#undef MOE_MX32_LDS_U32
#undef MOE_MX_ISSUE_SCALES
#undef MOE_MX_ISSUE
  MOE_WAIT_VMCNT(0);
  __syncthreads();

  // epilogue: acc element e of block (mb, n) is row 32*mb + 8*(e/4) + 4*q +
  // e%4 of the wave's 64, tile column bcol(n). y: 32 rows x 128 bf16 columns
  // per wave and row block (8 KB), staged in the (free) code ring
  uint16_t* st = (uint16_t*)smem + wave * (32 * 128);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * q + (e & 3);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        st[r * 128 + n * 32 + r32] = (uint16_t)f32_to_bf16_bits(acc[mb][n][e]);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int p = it * 64 + lane, r = p >> 4, c = p & 15;
      const int row = wm * 64 + 32 * mb + r, colo = c0 + wn * 128 + 8 * c;
      if (row < tl.rows && colo < Nout)
        *(uint4*)(out + (size_t)(tl.row0 + row) * Nout + colo) =
            *(const uint4*)&st[r * 128 + 8 * c];
    }
  }
}

// GEMM2 runs the 32x32x64 kernel (measured 5-9 % faster at the W4A8 rank's
// shapes); GEMM1 keeps the 16x16x128 one (the 32x32x64 form was 12-19 %
// slower there: its compute loop alone reached 36 % of the fp8 peak against
// 43 %, and 768 blocks leave the second of two rounds half empty).

template <int SCB>
static hipError_t launch_mx(bool glu, dim3 grid, const Tile* tiles,
                            const int32_t* tile_count, const uint8_t* a,
                            const uint8_t* a_scale, const uint8_t* w,
                            const uint8_t* w_scale, void* out,
                            uint8_t* out_scale, int K, int Nw, int Nout,
                            int nslabs, const int32_t* gidx,
                            const int32_t* gbase, int gk, hipStream_t s) {
  const int sgroup = MOE_MX_SLAB_GROUP < nslabs ? MOE_MX_SLAB_GROUP : nslabs;
  if (glu)
    hipLaunchKernelGGL((gemm_mx_tiled_kernel<SCB>), grid, dim3(256), 0, s,
                       tiles, tile_count, a, a_scale, w, w_scale, out,
                       out_scale, K, Nw, Nout, nslabs, sgroup, gidx, gbase,
                       gk);
  else
    hipLaunchKernelGGL((gemm_mx32_tiled_kernel<SCB>), grid, dim3(256), 0, s,
                       tiles, tile_count, a, a_scale, w, w_scale,
                       (uint16_t*)out, K, Nw, Nout, nslabs, sgroup);
  return hipGetLastError();
}

hipError_t launch_gemm_mx_tiled(bool glu, const Tile* tiles,
                                const int32_t* tile_count, int max_tiles,
                                const uint8_t* a, const uint8_t* a_scale,
                                const uint8_t* w, const uint8_t* w_scale,
                                void* out, uint8_t* out_scale, int K, int Nw,
                                int Nout, const int32_t* gidx,
                                const int32_t* gbase, int gk, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const int slab = glu ? MBNW / 2 : MBNW;
  const int nslabs = (Nout + slab - 1) / slab;
  dim3 grid((unsigned)max_tiles * nslabs);
  // four steps of scales per copy when every row's scales split into whole
  // 16-byte pieces (no copy reads past a row, so none past the array)
  return (K / 32) % 16 == 0
             ? launch_mx<4>(glu, grid, tiles, tile_count, a, a_scale, w,
                            w_scale, out, out_scale, K, Nw, Nout, nslabs, gidx,
                            gbase, gk, s)
             : launch_mx<1>(glu, grid, tiles, tile_count, a, a_scale, w,
                            w_scale, out, out_scale, K, Nw, Nout, nslabs, gidx,
                            gbase, gk, s);
}

}  // namespace moe
