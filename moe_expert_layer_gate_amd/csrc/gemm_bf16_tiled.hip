// Grouped GEMM, bf16 x bf16 -> fp32 on MFMA, LDS-tiled schedule for
// prefill-size batches (many rows per expert).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// MoE TP优化 / 计算分解 (expert = down(SiLU(gate(x)) * up(x)), merged gate/up
// weights, npu_swiglu = SiLU(first half) * second half) and 高性能专家计算
// (all experts in one grouped operator); prefill operators are compute-bound
// (Prefill优化 / 并行策略选择).
//
// Two tile geometries, both 256 weight columns wide with K in steps of 32
// through an LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane l of a wave lands at the wave's LDS base +
// 16*l, no VGPRs involved):
//   * 128 rows: 4 waves (2 x 2), each 64 rows x 128 columns, 3-stage ring,
//     two blocks per CU -- for batches of 64 to 127 rows per expert;
//   * 256 rows: 8 waves (2 x 4), each 128 rows x 64 columns, 3-stage ring,
//     one block per CU -- for larger batches. Per K step a CU then issues
//     160 LDS instructions (copies in, fragment reads out) for 32 MFMAs per
//     SIMD, against 208 for the same work in 128-row tiles: on gfx950 an LDS
//     instruction occupies the CU's LDS for about 6.5 clocks whether it moves
//     16 bytes per lane (ds_read_b128) or 8 (the transposing reads of B), and
//     a 32x32x16 MFMA takes about 36, so the 128-row tile is bound by LDS
//     instruction issue and the 256-row tile by the MFMAs. Its L2 traffic per
//     flop is a quarter lower as well.
// In both, each SIMD holds two waves, and the tile's layout in LDS is:
//   * A (activation rows, K contiguous): LDS [row][4 x 16 B], the 16-byte
//     piece index XOR-swizzled with (row/4)%4 so the MFMA reads of 8
//     consecutive rows hit 8 different bank groups;
//   * B (weights [K, N], N contiguous): LDS [k][32 x 16 B] as in HBM, piece
//     index XOR-swizzled with 4*(k%4); read K-packed with ds_read_b64_tr_b16:
//     within each group of 16 lanes, source lane s supplies row kb + s/4,
//     columns n0 + 4*(s%4) .. +3, and lane j receives column n0 + j at rows
//     kb .. kb+3 (transpose semantics measured with an in-bounds probe); two
//     such reads form the 8 consecutive K of an MFMA B fragment;
//   * v_mfma_f32_32x32x16_bf16: each wave owns WR rows x WC weight columns
//     (WR/32 x WC/32 blocks of 32 x 32);
//   * GEMM1 tiles hold 128 gate columns and the 128 matching up columns; a
//     wave takes WC/2 of each, so SwiGLU is lane-local in the epilogue;
//   * the epilogue stages each wave's 32-row slice through LDS and writes
//     16-byte rows to HBM;
//   * blocks are remapped so each XCD works on a contiguous range of
//     (tile, slab) pairs: the m-tiles of one expert and one weight slab run on
//     the same XCD and share its L2.
//
// The same schedule runs the W8A8 experts ([P3] "NPU Qwen3-Next inference
// practice", 量化策略: int8 weights with static per-channel scales, int8
// activations with dynamic per-token scales): a step is 64 bytes of every row
// either way (32 bf16 or 64 int8 K), so the LDS ring, the copies of A and
// the fragment reads are byte for byte those of bf16. The int8 weights come
// packed in 1 KB fragments (16 columns x 64 K bytes each); they are staged
// like A, [column][4 x 16 B] with the same swizzle, each copy instruction
// reading one whole fragment, and read with plain 16-byte reads;
// v_mfma_i32_32x32x32_i8
// takes the place of the bf16 MFMA (same operand bytes, same issue cycles,
// twice the K); the int32 sums are dequantised in the epilogue with the row
// scales (staged in LDS per tile) and the weight column scales.
#include <type_traits>

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
#ifndef MOE_TILED_NT_SINGLE
#define MOE_TILED_NT_SINGLE 1
#endif

#ifndef MOE_TILED_SLAB_GROUP
#define MOE_TILED_SLAB_GROUP 3
#endif

namespace moe {

namespace {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int BNW = 256, BK = 32;
constexpr int B_BYTES = BK * BNW * 2;           // 16 KB
constexpr int B_ROW = BNW * 2;                  // 512 B

// Tile geometry: WAVES_M x WAVES_N waves of WR rows x WC = 256 / WAVES_N
// weight columns each.
template <int WR_, int WAVES_M_, int WAVES_N_, int NSTAGE_, int BPC_>
struct TiledCfg {
  static constexpr int WR = WR_;                         // rows per wave
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int WC = BNW / WAVES_N;               // columns per wave
  static constexpr int BM = WAVES_M * WR;                // tile rows
  static constexpr int NMB = WR / 32;                    // 32-row blocks per wave
  static constexpr int NNB = WC / 32;                    // 32-column blocks per wave
  static constexpr int NSTAGE = NSTAGE_;                 // LDS ring depth
  static constexpr int A_BYTES = BM * BK * 2;            // 8 / 16 KB
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;  // 24 / 32 KB
  static constexpr int NA = BM / 16 / NWAVES;            // A copies per wave and step
  static constexpr int NB = 16 / NWAVES;                 // B copies per wave and step
  static constexpr int NI = NA + NB;                     // copies per wave and step
  static constexpr int BLOCKS_PER_CU = BPC_;
  static_assert(NA * 16 * NWAVES == BM && NB * NWAVES == 16, "copy split");
  static_assert(NNB % 2 == 0, "GLU splits a wave's columns in halves");
};
using Tiles128 = TiledCfg<64, 2, 2, 3, 2>;
using Tiles256 = TiledCfg<128, 2, 4, 3, 1>;

MOE_DEV f32x16 mfma32(u32x4_t a, u32x4_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

// int8 x int8 -> int32: 32 K per instruction, the same 16 bytes per lane and
// operand as the bf16 form; A and B lanes hold the same K offsets, so the sum
// over K is exact whatever order the hardware takes them in.
MOE_DEV i32x16 mfma32(u32x4_t a, u32x4_t b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a),
                                               __builtin_bit_cast(i32x4_t, b),
                                               c, 0, 0, 0);
}

MOE_DEV v4i16_t lds_read_tr(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(uintptr_t)a);
}

MOE_DEV int swz_a(int row) { return (row >> 2) & 3; }
MOE_DEV int swz_b(int k) { return 4 * (k & 3); }

}  // namespace

// One (tile, slab) work item L of the grid's list (tile_item: slab groups of
// sgroup within an expert). smem is the block's LDS ring (plus, for int8, 128 row
// scales after it); the item starts and ends with every wave past its LDS
// accesses of the previous item.
// PKB: bf16 weights slab-packed (pack_bf16.hip): the 32 x 256 block of a
// K step is one contiguous 16 KB, [k][column] with the tile's columns in
// order, so the copies read it in place of 32 rows 2N bytes apart (same LDS
// layout and swizzle).
// I8: W8A8 -- A int8 codes [rows, K] with one fp32 scale per row (a_scale,
// indexed like the rows), weights int8 [E_loc, N, K] (K contiguous) with one
// fp32 scale per output channel (w_scale [E_loc, N]); int32 accumulation,
// dequantised in the epilogue; GEMM1 stores h in fp32, GEMM2 y in bf16.
template <bool GLU, class C, bool I8, bool PKB>
MOE_DEV void tiled_item(
    uint8_t* smem, int L, const Tile* __restrict__ tiles,
    const void* __restrict__ a, const void* __restrict__ w,
    void* __restrict__ out, int K, int Nw, int Nout, int nslabs, int sgroup,
    const int32_t* __restrict__ gidx, const int32_t* __restrict__ gbase,
    int gk, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale) {
  using Acc = typename std::conditional<I8, i32x16, f32x16>::type;
  constexpr int EB = I8 ? 1 : 2;      // bytes per element
  constexpr int KS = 64 / EB;         // K per step (64 bytes of every row)
  constexpr int WR = C::WR, WC = C::WC, NW = C::NWAVES;
  constexpr int BM = C::BM, NMB = C::NMB, NNB = C::NNB, NSTAGE = C::NSTAGE;
  constexpr int NBR = I8 ? NNB : 2 * NNB;  // LDS reads of B per half step
  constexpr int A_BYTES = C::A_BYTES, STAGE_BYTES = C::STAGE_BYTES;
  constexpr int NA = C::NA, NB = C::NB, NI = C::NI;
  (void)BM;
  Tile tl;
  int slab;
  tile_item(tiles, L, nslabs, sgroup, tl, slab);
  const int c0 = slab * (GLU ? BNW / 2 : BNW);  // first output column

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const char* we = (const char*)w + (size_t)tl.expert * K * Nw * EB;
  // an expert with one tile is the only reader of its weights: stream them
  const bool wnt = MOE_TILED_NT_SINGLE &&
                   __builtin_amdgcn_readfirstlane(tl.count) == 1;

  // ---- global -> LDS assignment (per wave instruction: 1 KB contiguous)
  // A, instruction j (0..NA-1): tile rows 16*(wave + NW*j) + lane/4, physical
  // piece lane%4 holds logical piece (lane%4) ^ swz_a(row)
  // With a gather index the rows come straight from x (row of sorted copy
  // i = token sorted_copy[i] / k; the host keeps x under 4 GB so 32-bit
  // offsets hold), otherwise from the permuted rows of this tile.
  const char* a_tile =
      (const char*)a + (gidx ? 0 : (size_t)tl.row0 * K * EB);  // uniform
  uint32_t a_off[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = 16 * (wave + NW * j) + (lane >> 2);
    int src = r < tl.rows ? r : 0;
    if (gidx) src = gidx[gbase[0] + tl.row0 + src] / gk;
    a_off[j] = (uint32_t)src * K * EB + 16 * ((lane & 3) ^ swz_a(r));
  }
  // int8: the row scales of the tile, in LDS after the ring (0 past its rows)
  float* rs_lds = (float*)(smem + NSTAGE * STAGE_BYTES);
  if (I8 && tid < BM) {
    float sc = 0.f;
    if (tid < tl.rows)
      sc = a_scale[gidx ? gidx[gbase[0] + tl.row0 + tid] / gk : tl.row0 + tid];
    rs_lds[tid] = sc;
  }
  // weight column of tile column t (0..255); columns past Nout read column 0
  auto wcol = [&](int t) -> int {
    int oc, col;
    if (GLU) {
      oc = c0 + (t & (BNW / 2 - 1));
      col = t < BNW / 2 ? oc : Nout + oc;
    } else {
      oc = c0 + t;
      col = oc;
    }
    return oc < Nout ? col : 0;
  };
  // B (bf16 [K, N]), instruction j (0..NB-1): k-row 2*(wave + NW*j) +
  // lane/32 of the step, physical piece lane%32 holds logical piece
  // (lane%32) ^ swz_b(k); the swizzle only depends on k%4 = 2*(wave&1) +
  // lane/32 (NW is even), the same for all j.
  // B (int8, packed: 1 KB fragments per 64-byte K chunk and 16 columns,
  // 16 bytes of column c, K piece p at 16 * (c + 16 p)), instruction j
  // (0..NB-1): the fragment of tile columns 16*(wave + NW*j) .. +15 for this
  // step, copied as it is (lane l takes bytes 16 l, one contiguous 1 KB), so
  // LDS holds [16-column group][piece][column] -- the MFMA reads (32 lanes
  // on 32 consecutive columns, one piece) are conflict-free without a
  // swizzle. (N % 16 == 0: a 16-column group is in or past N whole, and
  // wcol sends it to group 0 in the latter case.)
  uint32_t b_off[I8 ? NB : 1];
  if constexpr (I8) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      b_off[j] = (uint32_t)wcol(16 * (wave + NW * j)) / 16 * 1024u + 16u * lane;
  } else {
    const int kr = 2 * wave + (lane >> 5);
    const int cl = (lane & 31) ^ swz_b(kr);
    b_off[0] = PKB ? (uint32_t)(kr * B_ROW + 16 * cl)
                   : (uint32_t)(kr * Nw + wcol(8 * cl)) * 2;
  }
  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(
      lds_addr(smem + (16 * wave) * (BK * 2)));
  const uint32_t b_dst = __builtin_amdgcn_readfirstlane(lds_addr(
      smem + A_BYTES + (I8 ? 16 * wave * 64 : (2 * wave) * B_ROW)));
  // bytes per K step of B: 32 rows of bf16 [K, N]; for int8 one packed
  // 64-byte K chunk of all N / 16 column groups (32-bit: N * K < 2^31)
  const size_t b_step = PKB ? (size_t)B_BYTES : (size_t)BK * Nw * 2;
  // packed: this item's slab, K / BK steps of B_BYTES each
  const char* wsl = we + (PKB ? (size_t)slab * (K / BK) * B_BYTES : 0);
  const uint32_t b_step_i8 = (uint32_t)Nw * 64u;
  const uint32_t b_rowj = 2u * NW * (PKB ? B_ROW : Nw * 2);  // 2*NW k-rows

  // loads of K step s_ into stage st_ (NI instructions per wave)
#define MOE_TILED_ISSUE(s_, st_)                                              \
  do {                                                                        \
    const char* ab_ = a_tile + (size_t)(s_) * 64;                             \
    const uint32_t o_ = (st_) * STAGE_BYTES;                                  \
    _Pragma("unroll") for (int j = 0; j < NA; ++j)                            \
      g2lds(ab_, a_off[j], a_dst + o_ + 16 * NW * j * (BK * 2));              \
    if constexpr (I8) {                                                       \
      const char* bb_ = we + (uint32_t)(s_) * b_step_i8;                      \
      _Pragma("unroll") for (int j = 0; j < NB; ++j)                          \
        g2lds_w(bb_, b_off[j], b_dst + o_ + 16 * NW * j * 64, wnt);           \
    } else {                                                                  \
      const char* bb_ = wsl + (size_t)(s_) * b_step;                          \
      _Pragma("unroll") for (int j = 0; j < NB; ++j)                          \
        g2lds_w(bb_, b_off[0] + j * b_rowj, b_dst + o_ + 2 * NW * j * B_ROW,  \
                wnt);                                                         \
    }                                                                         \
  } while (0)

  Acc acc[NMB][NNB];
#pragma unroll
  for (int i = 0; i < NMB; ++i)
#pragma unroll
    for (int j = 0; j < NNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // LDS read offsets, loop invariant (stage offsets are immediates below)
  const int lr = lane & 31, lh = lane >> 5;
  // A: row m = wm*WR + 32*mb + lr; its swizzle (m/4)%4 = (lr/4)%4 is the
  // same for every mb, so block mb sits a constant 32 rows further on
  uint32_t a_rd[2];  // [kk]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int m = wm * WR + lr;
    a_rd[kk] = lds_addr(smem) + m * (BK * 2) + 16 * ((kk * 2 + lh) ^ swz_a(m));
  }
  // bf16 transpose reads: group g = lane/16, source lane s = lane%16
  // supplies row kk*16 + 8*(g/2) + s/4 and columns cb + 16*(g%2) + 4*(s%4)
  // .. +3. int8: lane l reads tile column cb + l%32, logical piece
  // 2*kk + l/32 (the same K bytes as its A read).
  // Column block nbk of the wave: GLU -- gate blocks first (nbk < NNB/2),
  // then the matching up blocks, WC/2 columns of each half of the tile.
  // (a part that depends on the wave, and a constant per nbk)
  auto cdelta = [](int nbk) -> int {
    return GLU ? (nbk < NNB / 2 ? 0 : BNW / 2) + (nbk % (NNB / 2)) * 32
               : nbk * 32;
  };
  const int cwave = wn * (GLU ? WC / 2 : WC);
  auto colblk = [&](int nbk) -> int { return cwave + cdelta(nbk); };
  // int8: column col, piece p sits at (col/16) KB + 16 (16 p + col%16);
  // the 32-column blocks of the wave are whole 16-column groups apart, so
  // only the nbk = 0 offsets are kept (b_rd[kk][0]) and the others are
  // constant distances from them
  uint32_t b_rd[2][I8 ? 1 : NNB];  // [kk][nbk]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int nbk = 0; nbk < (I8 ? 1 : NNB); ++nbk) {
      const int cb = colblk(nbk);
      if constexpr (I8) {
        const int col = cb + lr;
        b_rd[kk][nbk] = lds_addr(smem) + A_BYTES + (col >> 4) * 1024 +
                        16 * (16 * (kk * 2 + lh) + (col & 15));
      } else {
        const int kr = kk * 16 + 8 * lh + ((lane & 15) >> 2);
        const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        b_rd[kk][nbk] = lds_addr(smem) + A_BYTES + kr * B_ROW +
                        16 * ((col >> 3) ^ swz_b(kr)) + 2 * (col & 7);
      }
    }

  // fragments of one half step (16 K): A for the wave's 32-row blocks,
  // B for its 32-column blocks; two register sets so that the LDS reads
  // of the next half step overlap the MFMAs of the current one
#define MOE_TILED_READ(fa_, fb_, st_, kk_)                                    \
  do {                                                                        \
    _Pragma("unroll") for (int mb = 0; mb < NMB; ++mb)                        \
      fa_[mb] = lds_read_b128(a_rd[kk_] + mb * 32 * (BK * 2) + (st_) * STAGE_BYTES); \
    _Pragma("unroll") for (int nbk = 0; nbk < NNB; ++nbk) {                   \
      const uint32_t p_ = (I8 ? b_rd[kk_][0] + cdelta(nbk) * 64               \
                              : b_rd[kk_][I8 ? 0 : nbk]) +                    \
                          (st_) * STAGE_BYTES;                                \
      if constexpr (I8) {                                                     \
        fb_[nbk] = lds_read_b128(p_);                                         \
      } else {                                                                \
        const v4i16_t lo = lds_read_tr(p_);                                   \
        const v4i16_t hi = lds_read_tr(p_ + 4 * B_ROW);                       \
        fb_[nbk] = __builtin_bit_cast(                                        \
            u32x4_t, v8i16_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}); \
      }                                                                       \
    }                                                                         \
  } while (0)
  // NMB_: 32-row blocks of this wave that hold tile rows (blocks past the
  // tile's rows feed no stored output and are skipped)
#define MOE_TILED_MMA(fa_, fb_, NMB_)                                         \
  do {                                                                        \
    _Pragma("unroll") for (int mb = 0; mb < (NMB_); ++mb)                     \
      _Pragma("unroll") for (int nbk = 0; nbk < NNB; ++nbk)                   \
        acc[mb][nbk] = mfma32(fa_[mb], fb_[nbk], acc[mb][nbk]);               \
  } while (0)

  // K step t_ held in stage st_ (= t_ % NSTAGE); fragments of its first half
  // are in f0*. While the second half is read, the first is multiplied; then,
  // once the copies of step t+1 have landed (steps t+2 .. t+NSTAGE-1, NI
  // copies per wave each, may still be in flight) and every wave is past its
  // reads of stage st_, that stage is refilled with step t+NSTAGE and the
  // first half of step t+1 is read while the second half of step t is
  // multiplied. The steady-state form (t + NSTAGE < nsteps) has no branches,
  // so the compiler's wait counts stay exact; the last steps take the
  // guarded form.
#define MOE_TILED_STEP_FULL(t_, st_, NMB_)                                    \
  do {                                                                        \
    MOE_TILED_READ(f1a, f1b, st_, 1);                                         \
    MOE_TILED_MMA(f0a, f0b, NMB_);                                            \
    MOE_TILED_ORDER(NMB_);                                                    \
    MOE_WAIT_VMCNT((NSTAGE - 2) * NI);                                        \
    __syncthreads();                                                          \
    MOE_TILED_ISSUE((t_) + NSTAGE, st_);                                      \
    MOE_TILED_READ(f0a, f0b, ((st_) + 1) % NSTAGE, 0);                        \
    MOE_TILED_MMA(f1a, f1b, NMB_);                                            \
    MOE_TILED_ORDER(NMB_);                                                    \
  } while (0)
  // scheduling order of a half step: all LDS reads of the next fragments
  // first, then the MFMAs on the current ones (otherwise the scheduler sinks
  // each read next to its use and the LDS latency is exposed)
#define MOE_TILED_ORDER(NMB_)                                                 \
  do {                                                                        \
    if ((NMB_) > 0) {                                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, (NMB_) + NBR, 0);           \
      __builtin_amdgcn_sched_group_barrier(0x008, NNB * (NMB_), 0);           \
    }                                                                         \
  } while (0)
  // wait until step t+1 has landed: the copies of steps t+2 .. up to
  // min(t + NSTAGE - 1, nsteps - 1) may stay in flight
#define MOE_TILED_WAIT_NEXT(t_)                                               \
  do {                                                                        \
    const int pend_ = min(NSTAGE - 2, nsteps - 2 - (t_));                     \
    if (NSTAGE > 3 && pend_ >= 2) MOE_WAIT_VMCNT(2 * NI);                     \
    else if (pend_ >= 1) MOE_WAIT_VMCNT(NI);                                  \
    else MOE_WAIT_VMCNT(0);                                                   \
  } while (0)
#define MOE_TILED_STEP(t_, st_, NMB_)                                         \
  do {                                                                        \
    const int t = (t_);                                                       \
    if (t < nsteps) {                                                         \
      MOE_TILED_READ(f1a, f1b, st_, 1);                                       \
      MOE_TILED_MMA(f0a, f0b, NMB_);                                          \
      if (t + 1 < nsteps) {                                                   \
        MOE_TILED_WAIT_NEXT(t);                                               \
        __syncthreads();                                                      \
        if (t + NSTAGE < nsteps) MOE_TILED_ISSUE(t + NSTAGE, st_);            \
        MOE_TILED_READ(f0a, f0b, ((st_) + 1) % NSTAGE, 0);                    \
      }                                                                       \
      MOE_TILED_MMA(f1a, f1b, NMB_);                                          \
    }                                                                         \
  } while (0)
#define MOE_TILED_PIPE(NMB_)                                                  \
  do {                                                                        \
    int s = 0;                                                                \
    for (; s + 2 * NSTAGE - 1 < nsteps; s += NSTAGE) {                        \
      _Pragma("unroll") for (int i = 0; i < NSTAGE; ++i)                      \
        MOE_TILED_STEP_FULL(s + i, i, NMB_);                                  \
    }                                                                         \
    _Pragma("unroll") for (int i = 0; i < 2 * NSTAGE - 1; ++i)                \
      MOE_TILED_STEP(s + i, i % NSTAGE, NMB_);                                \
  } while (0)

  const int nsteps = K / KS;
  // rows of this wave's WR-row part of the tile (wave-uniform)
  const int mrows = __builtin_amdgcn_readfirstlane(tl.rows - wm * WR);
  u32x4_t f0a[NMB], f0b[NNB], f1a[NMB], f1b[NNB];
  // prologue: steps 0 .. NSTAGE-2 in flight, wait for step 0, then the last
  // stage gets step NSTAGE-1
  MOE_TILED_ISSUE(0, 0);
#pragma unroll
  for (int i = 1; i < NSTAGE - 1; ++i)
    if (nsteps > i) MOE_TILED_ISSUE(i, i);
  MOE_TILED_WAIT_NEXT(-1);
  __syncthreads();
  if (nsteps > NSTAGE - 1) MOE_TILED_ISSUE(NSTAGE - 1, NSTAGE - 1);
  MOE_TILED_READ(f0a, f0b, 0, 0);
  if (NMB > 3 && mrows > 96) MOE_TILED_PIPE(4);
  else if (NMB > 2 && mrows > 64) MOE_TILED_PIPE(3);
  else if (mrows > 32) MOE_TILED_PIPE(2);
  else if (mrows > 0) MOE_TILED_PIPE(1);
  else MOE_TILED_PIPE(0);
#undef MOE_TILED_PIPE
#undef MOE_TILED_STEP_FULL
#undef MOE_TILED_WAIT_NEXT
#undef MOE_TILED_ORDER
#undef MOE_TILED_STEP
#undef MOE_TILED_MMA
#undef MOE_TILED_READ
#undef MOE_TILED_ISSUE
  __syncthreads();

  // epilogue through LDS: each wave stages 32 rows at a time
  constexpr int OCOLS = GLU ? WC / 2 : WC;  // output columns of this wave
  const int oc0 = c0 + wn * OCOLS;          // first output column of this wave
  // int8: value = acc * scale of its row * scale of its weight column
  float cs[NNB];
#pragma unroll
  for (int nbk = 0; nbk < NNB; ++nbk) {
    cs[nbk] = 1.f;
    if constexpr (I8)
      cs[nbk] = w_scale[(size_t)tl.expert * Nw + wcol(colblk(nbk) + lr)];
  }
  auto val = [&](int mb, int nbk, int e, int r) -> float {
    if constexpr (I8)
      return (float)acc[mb][nbk][e] * rs_lds[wm * WR + mb * 32 + r] * cs[nbk];
    else
      return acc[mb][nbk][e];
  };
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    // one 32-row block at a time: the scale reads and staging of block mb
    // stay after those of block mb-1 (fewer live registers)
    __builtin_amdgcn_sched_barrier(0);
    // acc element e of a 32x32 block: row 8*(e/4) + 4*(lane/32) + e%4,
    // column lane%32
    if (GLU && I8) {
      // h in fp32: 32 rows x OCOLS (<= 64) columns per wave, rows 64 apart
      float* st = (float*)smem + wave * (32 * 64);
      float* st_lane = st + 4 * lh * 64 + lr;  // constant offsets below
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * lh + (e & 3);
#pragma unroll
        for (int gb = 0; gb < NNB / 2; ++gb)
          st_lane[(8 * (e >> 2) + (e & 3)) * 64 + gb * 32] =
              silu(val(mb, gb, e, r)) * val(mb, gb + NNB / 2, e, r);
      }
      constexpr int CH = OCOLS / 4;  // 16-byte pieces per row
#pragma unroll
      for (int it = 0; it < 32 * CH / 64; ++it) {
        const int q = it * 64 + lane;
        const int r = q / CH, c = q % CH;
        const int row = wm * WR + mb * 32 + r;
        const int col = oc0 + 4 * c;
        if (row < tl.rows && col < Nout)
          *(uint4*)((float*)out + (size_t)(tl.row0 + row) * Nout + col) =
              *(const uint4*)&st[r * 64 + 4 * c];
      }
      continue;
    }
    // bf16: 32 rows x OCOLS (<= 128) columns per wave, rows 128 apart
    uint16_t* stage = (uint16_t*)smem + wave * (32 * 128);
    uint16_t* stage_lane = stage + 4 * lh * 128 + lr;  // constant offsets below
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * lh + (e & 3);
      const int ro = (8 * (e >> 2) + (e & 3)) * 128;
      if (GLU) {
#pragma unroll
        for (int gb = 0; gb < NNB / 2; ++gb) {
          const float hv = silu(val(mb, gb, e, r)) * val(mb, gb + NNB / 2, e, r);
          stage_lane[ro + gb * 32] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int nbk = 0; nbk < NNB; ++nbk)
          stage_lane[ro + nbk * 32] = (uint16_t)f32_to_bf16_bits(val(mb, nbk, e, r));
      }
    }
    // each lane writes 16-byte pieces of the staged rows
    constexpr int CH = OCOLS / 8;  // 16-byte pieces per row
#pragma unroll
    for (int it = 0; it < 32 * CH / 64; ++it) {
      const int q = it * 64 + lane;
      const int r = q / CH, c = q % CH;
      const int row = wm * WR + mb * 32 + r;
      const int col = oc0 + 8 * c;
      if (row < tl.rows && col < Nout)
        *(uint4*)((uint16_t*)out + (size_t)(tl.row0 + row) * Nout + col) =
            *(const uint4*)&stage[r * 128 + 8 * c];
    }
  }
}

// Persistent grid of (a multiple of 8) blocks, dispatched round-robin over the
// 8 XCDs: XCD x owns the contiguous item range [lo_x, hi_x) and its blocks
// walk it in lockstep, block j taking items lo_x + j, lo_x + j + nj, ...
// (nj blocks per XCD). The items running at once on an XCD are therefore
// consecutive: the slabs of a few tiles and the tiles of one expert, whose A
// rows and weight slabs that XCD's L2 serves to all of them.
template <bool GLU, class C, bool I8, bool PKB>
__global__ __launch_bounds__(C::THREADS, C::BLOCKS_PER_CU) void gemm_bf16_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const void* __restrict__ a, const void* __restrict__ w,
    void* __restrict__ out, int K, int Nw, int Nout, int nslabs, int sgroup,
    const int32_t* __restrict__ gidx, const int32_t* __restrict__ gbase,
    int gk, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale) {
  static_assert(C::NSTAGE * C::STAGE_BYTES >= C::NWAVES * 8192,
                "epilogue staging fits the ring");
  __shared__ __align__(1024) uint8_t
      smem[C::NSTAGE * C::STAGE_BYTES + (I8 ? 4 * C::BM : 0)];
  const int nb = tile_count[0] * nslabs;
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8, nj = gridDim.x / 8;
  const int per = nb / 8, rem = nb % 8;
  const int lo = xcd * per + min(xcd, rem);
  const int hi = lo + per + (xcd < rem ? 1 : 0);
  for (int L = lo + j; L < hi; L += nj) {
    tiled_item<GLU, C, I8, PKB>(smem, L, tiles, a, w, out, K, Nw, Nout, nslabs,
                            sgroup, gidx, gbase, gk, a_scale, w_scale);
    __syncthreads();  // LDS staging of this item read before the next fills
  }
}

template <class C, bool I8, bool PKB = false>
static hipError_t launch_tiled(bool glu, const Tile* tiles,
                               const int32_t* tile_count, int max_tiles,
                               const void* a, const void* w, void* out, int K,
                               int Nw, int Nout, const int32_t* gidx,
                               const int32_t* gbase, int gk,
                               const float* a_scale, const float* w_scale,
                               hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const int slab = glu ? BNW / 2 : BNW;
  const int nslabs = (Nout + slab - 1) / slab;
  const int sgroup = MOE_TILED_SLAB_GROUP < nslabs ? MOE_TILED_SLAB_GROUP : nslabs;
  // one resident block per slot, a multiple of 8 (the XCD count), never
  // more blocks than items
  const long long items = (long long)max_tiles * nslabs;
  const long long slots = (long long)device_cus() * C::BLOCKS_PER_CU;
  long long nblk = items < slots ? items : slots;
  nblk = ((nblk + 7) / 8) * 8;
  const dim3 grid((unsigned)nblk), block(C::THREADS);
  if (glu)
    hipLaunchKernelGGL((gemm_bf16_tiled_kernel<true, C, I8, PKB>), grid, block, 0,
                       s, tiles, tile_count, a, w, out, K, Nw, Nout, nslabs,
                       sgroup, gidx, gbase, gk, a_scale, w_scale);
  else
    hipLaunchKernelGGL((gemm_bf16_tiled_kernel<false, C, I8, PKB>), grid, block, 0,
                       s, tiles, tile_count, a, w, out, K, Nw, Nout, nslabs,
                       sgroup, gidx, gbase, gk, a_scale, w_scale);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_tiled(bool glu, int mt, const Tile* tiles,
                                  const int32_t* tile_count, int max_tiles,
                                  const uint16_t* a, const uint16_t* w,
                                  uint16_t* out, int K, int Nw, int Nout,
                                  const int32_t* gidx, const int32_t* gbase,
                                  int gk, hipStream_t s, bool pk) {
  // packed slabs are whole: 256 weight columns, K in steps of 32
  if (pk && (K % BK || Nw % BNW)) return hipErrorInvalidValue;
  if (mt == 256)
    return pk ? launch_tiled<Tiles256, false, true>(
                    glu, tiles, tile_count, max_tiles, a, w, out, K, Nw, Nout,
                    gidx, gbase, gk, nullptr, nullptr, s)
              : launch_tiled<Tiles256, false>(glu, tiles, tile_count,
                                              max_tiles, a, w, out, K, Nw, Nout,
                                              gidx, gbase, gk, nullptr, nullptr,
                                              s);
  return pk ? launch_tiled<Tiles128, false, true>(
                  glu, tiles, tile_count, max_tiles, a, w, out, K, Nw, Nout,
                  gidx, gbase, gk, nullptr, nullptr, s)
            : launch_tiled<Tiles128, false>(glu, tiles, tile_count, max_tiles,
                                            a, w, out, K, Nw, Nout, gidx, gbase,
                                            gk, nullptr, nullptr, s);
}

hipError_t launch_gemm_i8_tiled(bool glu, int mt, const Tile* tiles,
                                const int32_t* tile_count, int max_tiles,
                                const int8_t* a, const float* a_scale,
                                const int8_t* w, const float* w_scale,
                                void* out, int K, int Nw, int Nout,
                                const int32_t* gidx, const int32_t* gbase,
                                int gk, hipStream_t s) {
  if (mt == 256)
    return launch_tiled<Tiles256, true>(glu, tiles, tile_count, max_tiles, a,
                                        w, out, K, Nw, Nout, gidx, gbase, gk,
                                        a_scale, w_scale, s);
  return launch_tiled<Tiles128, true>(glu, tiles, tile_count, max_tiles, a, w,
                                      out, K, Nw, Nout, gidx, gbase, gk,
                                      a_scale, w_scale, s);
}

}  // namespace moe
