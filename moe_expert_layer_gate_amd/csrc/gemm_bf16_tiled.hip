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
// tile of one expert, K in steps of 32 through a 3-stage LDS ring filled by
// direct global->LDS loads (global_load_lds_dwordx4: lane l of a wave lands
// at the wave's LDS base + 16*l, no VGPRs involved), two steps in flight:
//   * A (activation rows, K contiguous): LDS [row][4 x 16 B], the 16-byte
//     piece index XOR-swizzled with (row/4)%4 so the MFMA reads of 8
//     consecutive rows hit 8 different bank groups;
//   * B (weights [K, N], N contiguous): LDS [k][32 x 16 B] as in HBM, piece
//     index XOR-swizzled with 4*(k%4); read K-packed with ds_read_b64_tr_b16:
//     within each group of 16 lanes, source lane s supplies row kb + s/4,
//     columns n0 + 4*(s%4) .. +3, and lane j receives column n0 + j at rows
//     kb .. kb+3 (transpose semantics measured with an in-bounds probe); two
//     such reads form the 8 consecutive K of an MFMA B fragment;
//   * v_mfma_f32_32x32x16_bf16: each wave owns 64 rows x 128 weight columns
//     (2 x 4 blocks of 32 x 32, 128 fp32 accumulators);
//   * GEMM1 tiles hold 128 gate columns and the 128 matching up columns; a
//     wave takes 64 of each, so SwiGLU is lane-local in the epilogue;
//   * the epilogue stages each wave's 32-row slice through LDS and writes
//     16-byte rows to HBM;
//   * blocks are remapped so each XCD works on a contiguous range of
//     (tile, slab) pairs: the m-tiles of one expert and one weight slab run on
//     the same XCD and share its L2.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BNW = 256, BK = 32, NSTAGE = 3;
constexpr int A_BYTES = BM * BK * 2;            // 8 KB
constexpr int B_BYTES = BK * BNW * 2;           // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;  // 24 KB
constexpr int B_ROW = BNW * 2;                  // 512 B

MOE_DEV f32x16 mfma32(u32x4_t a, u32x4_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

MOE_DEV u32x4_t lds_read_b128(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)a;
}

MOE_DEV v4i16_t lds_read_tr(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(uintptr_t)a);
}

// 16 bytes per lane, global (base + 32-bit lane offset) -> LDS at
// lds_wave_base + 16 * lane. Issued as inline assembly so that the compiler
// does not track it as an LDS write: it would otherwise drain every
// outstanding copy (vmcnt(0)) before each barrier and LDS read, serialising
// the ring. Completion is ordered by hand with MOE_WAIT_VMCNT before the
// barrier that publishes a stage. M0 holds the wave-uniform LDS destination;
// nothing else in these kernels uses M0. The base is a wave-uniform 64-bit
// SGPR pair, so advancing a step costs scalar adds only.
MOE_DEV void g2lds(const void* base, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_wave_base)
      : "memory");
}

MOE_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum)
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

MOE_DEV int swz_a(int row) { return (row >> 2) & 3; }
MOE_DEV int swz_b(int k) { return 4 * (k & 3); }

}  // namespace

// two blocks per CU: 2 waves per SIMD, LDS for two 3-stage rings
template <bool GLU>
__global__ __launch_bounds__(256, 2) void gemm_bf16_tiled_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ out, int K, int Nw, int Nout, int nslabs,
    const int32_t* __restrict__ gidx, const int32_t* __restrict__ gbase,
    int gk) {
  __shared__ __align__(1024) uint8_t smem[NSTAGE * STAGE_BYTES];
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

  // ---- global -> LDS assignment (per wave instruction: 1 KB contiguous)
  // A, instruction j (0..1): tile rows 16*(wave + 4j) + lane/4, physical
  // piece lane%4 holds logical piece (lane%4) ^ swz_a(row)
  // With a gather index the rows come straight from x (row of sorted copy
  // i = token sorted_copy[i] / k; the host keeps x under 4 GB so 32-bit
  // offsets hold), otherwise from the permuted rows of this tile.
  const uint16_t* a_tile = gidx ? a : a + (size_t)tl.row0 * K;  // uniform
  uint32_t a_off0, a_off1;
  {
    const int r0 = 16 * wave + (lane >> 2), r1 = r0 + 64;
    int s0 = r0 < tl.rows ? r0 : 0, s1 = r1 < tl.rows ? r1 : 0;
    if (gidx) {
      const int g0 = gbase[0] + tl.row0;
      s0 = gidx[g0 + s0] / gk;
      s1 = gidx[g0 + s1] / gk;
    }
    a_off0 = ((uint32_t)s0 * K + 8 * ((lane & 3) ^ swz_a(r0))) * 2u;
    a_off1 = ((uint32_t)s1 * K + 8 * ((lane & 3) ^ swz_a(r1))) * 2u;
  }
  // B, instruction j (0..3): k-row 2*(wave + 4j) + lane/32 of the step,
  // physical piece lane%32 holds logical piece (lane%32) ^ swz_b(k); the
  // swizzle only depends on k%4 = 2*(wave&1) + lane/32, the same for all j
  uint32_t b_off;
  {
    const int kr = 2 * wave + (lane >> 5);
    const int cl = (lane & 31) ^ swz_b(kr);
    const int j = 8 * cl;  // tile column
    int col, oc;
    if (GLU) {
      oc = c0 + (j & (BNW / 2 - 1));
      col = j < BNW / 2 ? oc : Nout + oc;
    } else {
      oc = c0 + j;
      col = oc;
    }
    if (oc >= Nout) col = 0;  // unused columns read column 0
    b_off = (uint32_t)(kr * Nw + col) * 2;
  }
  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(
      lds_addr(smem + (16 * wave) * (BK * 2)));
  const uint32_t b_dst = __builtin_amdgcn_readfirstlane(
      lds_addr(smem + A_BYTES + (2 * wave) * B_ROW));
  const size_t b_step = (size_t)BK * Nw * 2;     // bytes per K step of B
  const uint32_t b_row8 = 8u * Nw * 2;          // 8 k-rows of B

  // loads of K step s_ into stage st_ (6 instructions per wave)
#define MOE_TILED_ISSUE(s_, st_)                                              \
  do {                                                                        \
    const char* ab_ = (const char*)a_tile + (size_t)(s_) * (BK * 2);         \
    const char* bb_ = (const char*)we + (size_t)(s_) * b_step;               \
    const uint32_t o_ = (st_) * STAGE_BYTES;                                  \
    g2lds(ab_, a_off0, a_dst + o_);                                           \
    g2lds(ab_, a_off1, a_dst + o_ + 64 * (BK * 2));                           \
    g2lds(bb_, b_off, b_dst + o_);                                            \
    g2lds(bb_, b_off + b_row8, b_dst + o_ + 8 * B_ROW);                       \
    g2lds(bb_, b_off + 2 * b_row8, b_dst + o_ + 16 * B_ROW);                  \
    g2lds(bb_, b_off + 3 * b_row8, b_dst + o_ + 24 * B_ROW);                  \
  } while (0)

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // LDS read offsets, loop invariant (stage offsets are immediates below)
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t a_rd[2][2];  // [kk][mb]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m = wm * 64 + mb * 32 + lr;
      a_rd[kk][mb] = lds_addr(smem) + m * (BK * 2) + 16 * ((kk * 2 + lh) ^ swz_a(m));
    }
  // transpose reads: group g = lane/16, source lane s = lane%16 supplies row
  // kk*16 + 8*(g/2) + s/4 and columns cb + 16*(g%2) + 4*(s%4) .. +3
  uint32_t b_rd[2][4];  // [kk][nbk]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int nbk = 0; nbk < 4; ++nbk) {
      const int kr = kk * 16 + 8 * lh + ((lane & 15) >> 2);
      const int cb = GLU ? (nbk < 2 ? 0 : BNW / 2) + wn * 64 + (nbk & 1) * 32
                         : wn * 128 + nbk * 32;
      const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      b_rd[kk][nbk] = lds_addr(smem) + A_BYTES + kr * B_ROW +
                      16 * ((col >> 3) ^ swz_b(kr)) + 2 * (col & 7);
    }

#define MOE_TILED_COMPUTE(st_)                                                \
  do {                                                                        \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                        \
      u32x4_t fa[2], fb[4];                                                   \
      _Pragma("unroll") for (int mb = 0; mb < 2; ++mb) {                      \
        fa[mb] = lds_read_b128(a_rd[kk][mb] + (st_) * STAGE_BYTES);           \
      }                                                                       \
      _Pragma("unroll") for (int nbk = 0; nbk < 4; ++nbk) {                   \
        const uint32_t p_ = b_rd[kk][nbk] + (st_) * STAGE_BYTES;              \
        const v4i16_t lo = lds_read_tr(p_);                                   \
        const v4i16_t hi = lds_read_tr(p_ + 4 * B_ROW);                       \
        fb[nbk] = __builtin_bit_cast(                                         \
            u32x4_t, v8i16_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}); \
      }                                                                       \
      _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                        \
        _Pragma("unroll") for (int nbk = 0; nbk < 4; ++nbk)                   \
          acc[mb][nbk] = mfma32(fa[mb], fb[nbk], acc[mb][nbk]);               \
    }                                                                         \
  } while (0)

  // one K step t in stage st_: wait for its copies (at most one later step,
  // 6 copies per wave, still in flight), publish it, multiply, and refill
  // the stage read one step earlier with step t + 2
#define MOE_TILED_STEP(t_, st_)                                               \
  do {                                                                        \
    const int t = (t_);                                                       \
    if (t + 1 < nsteps) MOE_WAIT_VMCNT(6);                                    \
    else MOE_WAIT_VMCNT(0);                                                   \
    __syncthreads();                                                          \
    MOE_TILED_COMPUTE(st_);                                                   \
    if (t + 2 < nsteps) MOE_TILED_ISSUE(t + 2, ((st_) + 2) % NSTAGE);         \
  } while (0)

  const int nsteps = K / BK;
  MOE_TILED_ISSUE(0, 0);
  if (nsteps > 1) MOE_TILED_ISSUE(1, 1);
  int s = 0;
  for (; s + NSTAGE <= nsteps; s += NSTAGE) {
    MOE_TILED_STEP(s, 0);
    MOE_TILED_STEP(s + 1, 1);
    MOE_TILED_STEP(s + 2, 2);
  }
  if (s < nsteps) MOE_TILED_STEP(s, 0);
  if (s + 1 < nsteps) MOE_TILED_STEP(s + 1, 1);
#undef MOE_TILED_STEP
#undef MOE_TILED_COMPUTE
#undef MOE_TILED_ISSUE
  __syncthreads();

  // epilogue through LDS: each wave stages 32 rows at a time
  uint16_t* stage = (uint16_t*)smem + wave * (32 * 128);
  const int ncols = GLU ? 64 : 128;  // output columns of this wave
  const int oc0 = c0 + wn * ncols;   // first output column of this wave
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    // acc element e of a 32x32 block: row 8*(e/4) + 4*(lane/32) + e%4,
    // column lane%32
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * lh + (e & 3);
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
                                  const int32_t* gidx, const int32_t* gbase,
                                  int gk, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const int slab = glu ? BNW / 2 : BNW;
  const int nslabs = (Nout + slab - 1) / slab;
  dim3 grid((unsigned)max_tiles * nslabs);
  if (glu)
    hipLaunchKernelGGL(gemm_bf16_tiled_kernel<true>, grid, dim3(256), 0, s,
                       tiles, tile_count, a, w, out, K, Nw, Nout, nslabs,
                       gidx, gbase, gk);
  else
    hipLaunchKernelGGL(gemm_bf16_tiled_kernel<false>, grid, dim3(256), 0, s,
                       tiles, tile_count, a, w, out, K, Nw, Nout, nslabs,
                       gidx, gbase, gk);
  return hipGetLastError();
}

}  // namespace moe
