// Grouped GEMM, bf16 x bf16 -> fp32 on MFMA, weight-streaming schedule.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// MoE TP优化 / 计算分解 (expert = down(SiLU(gate(x)) * up(x)); merged gate/up
// matrix; npu_swiglu = SiLU(first half) * second half) and section
// 高性能专家计算 (one grouped operator for all experts). [P2] "LongCat-Flash
// inference on Atlas A3 clusters" notes that on the FFN side the grouped
// matmuls of decode are memory-bound.
//
// Decode-size batches give each expert a handful of rows, so every weight byte
// is used by at most 16*RG rows and the kernel is bound by streaming weights
// from HBM. The schedule keeps weights out of LDS entirely:
//   * weights are [K, N] with N contiguous. Lane l of a wave loads an 8x8
//     block -- rows k0 + 8*(l/16) + 0..7, columns col + 8*(l%16) + 0..7 -- as
//     eight 16-byte loads (16 lanes cover 256 contiguous bytes of a row), and
//     transposes it in registers (v_perm) into eight K-packed fragments, one
//     per column offset i. Fragment i is the B operand of a
//     v_mfma_f32_16x16x32_bf16 whose 16 "columns" are {col + 8g + i}, g=0..15.
//   * each lane carries two such column groups: for GEMM1 the gate columns
//     and the matching up columns (so SwiGLU is lane-local in the epilogue),
//     for GEMM2 two halves of a 256-column slab.
//   * A rows (activations, K contiguous) are loaded straight into the
//     fragment layout: row 16*rg + l%16, k0 + 8*(l/16) + 0..7. With a gather
//     index the rows are read from x itself (row of sorted copy i = token
//     sorted_copy[i] / k), so the permuted copy of x is never written.
//   * KSPLIT waves of a block split K; partial sums meet in LDS in one or
//     two rounds; wave 0 applies SwiGLU / converts and stores 16 bytes per
//     row and lane.
//   * PK: the weights come slab-packed (pack_bf16.hip): the 32 x 256 block
//     a block reads per K step is one contiguous 16 KB, rows of 512 bytes
//     (the 128 columns of the lane's first group, then those of its second);
//     the lane's loads and fragments are the same, only their addresses
//     change.
// Output D of each MFMA: lane l holds rows 4*(l/16) + 0..3 at column
// col + 8*(l%16) + i, so a lane owns 8 consecutive columns of 4 rows.
#include "common.h"
#include "launch.h"

namespace moe {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

MOE_DEV f32x4 mfma_bf16_16x16x32(u32x4_t a, u32x4_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

// Column i (0..7) of an 8x8 bf16 block held as 8 rows of uint4: K-packed.
MOE_DEV u32x4_t column_frag(const uint4 (&r)[8], int i) {
  const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
  auto dw = [&](int row) -> uint32_t {
    const uint4 v = r[row];
    const int d = i >> 1;
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
  };
  u32x4_t f;
  f.x = __builtin_amdgcn_perm(dw(1), dw(0), sel);
  f.y = __builtin_amdgcn_perm(dw(3), dw(2), sel);
  f.z = __builtin_amdgcn_perm(dw(5), dw(4), sel);
  f.w = __builtin_amdgcn_perm(dw(7), dw(6), sel);
  return f;
}

// Two waves per SIMD: left to itself the compiler spends 288 registers per
// lane (accumulators in AGPRs) and runs one wave per SIMD, so a decode launch
// of two thousand waves would take two rounds.
template <bool GLU, int RG, int KSPLIT, bool PK>
__global__ __launch_bounds__(64 * KSPLIT)
__attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_bf16_stream_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ out, int K, int Nw, int Nout,
    const int32_t* __restrict__ gidx, const int32_t* __restrict__ gbase,
    int gk) {
  // The tile entry is read alongside the tile count (entries past the count
  // are in bounds, merely stale): the empty asm keeps both loads ahead of the
  // exit test, so the weight loads start one scalar-load latency after the
  // kernel does.
  // grid: x = column slab, y = tile, so consecutive blocks are the slabs of
  // one expert (measured 2 % faster at decode than tile-major blocks)
  const Tile tl = tiles[blockIdx.y];
  const int ntiles = tile_count[0];
  asm volatile("" ::"s"(ntiles), "s"(tl.expert), "s"(tl.row0), "s"(tl.rows));
  if ((int)blockIdx.y >= ntiles) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & 15, kq = lane >> 4;
  // two column groups per lane
  constexpr int SLAB = GLU ? 128 : 256;
  const int c0 = blockIdx.x * SLAB;
  const int colA = c0 + 8 * g;
  const int colB = GLU ? Nout + colA : colA + 128;
  const bool okA = colA < Nout;
  const bool okB = GLU ? okA : (colA + 128 < Nout);
  // Columns past N and rows past the tile only feed outputs that are never
  // stored (each output column / row depends on its own B column / A row),
  // so their loads are redirected to column / row 0 instead of being
  // predicated: every load stays an unconditional 16-byte load.
  const int ldA = okA ? colA : 0;
  const int ldB = okB ? colB : 0;
  const uint16_t* we = w + (size_t)tl.expert * K * Nw;
  const int nsteps = K / 32;
  const int s_begin = wave * nsteps / KSPLIT;
  const int s_end = (wave + 1) * nsteps / KSPLIT;

  // A rows are resolved after the first step's weight loads are issued
  // (the gather index is two dependent loads away)
  const uint16_t* arow[RG];
  auto resolve_rows = [&]() {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int r = 16 * rg + g;
      int src = tl.row0 + (r < tl.rows ? r : 0);
      // fused gather: the row of the sorted copy is its token's row of x
      if (gidx) src = gidx[gbase[0] + src] / gk;
      arow[rg] = a + (size_t)src * K + 8 * kq;
    }
  };

  f32x4 acc[2][RG][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][rg][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one K step: 8 rows x (8 + 8) columns of weights and the A fragments
  struct Stage {
    uint4 bA[8], bB[8];
    u32x4_t af[RG];
  };
  auto load_w = [&](Stage& st, int s) {
    if constexpr (PK) {
      // slab blockIdx.x, step s: 16 KB of [32 rows][256 columns]
      const uint16_t* pA = we + ((size_t)blockIdx.x * nsteps + s) * 8192 +
                           (8 * kq) * 256 + 8 * g;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        st.bA[r] = load_stream16(pA + r * 256);
        st.bB[r] = load_stream16(pA + r * 256 + 128);
      }
    } else {
      const int k0 = s * 32;
      const uint16_t* pA = we + (size_t)(k0 + 8 * kq) * Nw + ldA;
      const uint16_t* pB = we + (size_t)(k0 + 8 * kq) * Nw + ldB;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        st.bA[r] = load_stream16(pA + (size_t)r * Nw);
        st.bB[r] = load_stream16(pB + (size_t)r * Nw);
      }
    }
  };
  auto load_a = [&](Stage& st, int s) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      uint4 v = *(const uint4*)(arow[rg] + s * 32);
      st.af[rg] = u32x4_t{v.x, v.y, v.z, v.w};
    }
  };
  auto load = [&](Stage& st, int s) {
    load_w(st, s);
    load_a(st, s);
  };
  auto compute = [&](const Stage& st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t fA = column_frag(st.bA, i);
      u32x4_t fB = column_frag(st.bB, i);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        acc[0][rg][i] = mfma_bf16_16x16x32(st.af[rg], fA, acc[0][rg][i]);
        acc[1][rg][i] = mfma_bf16_16x16x32(st.af[rg], fB, acc[1][rg][i]);
      }
    }
  };
  if (RG == 1) {
    // two register stages: the loads of step s+1 are in flight while step s
    // is transposed and multiplied
    Stage st0, st1;
    if (s_begin < s_end) load_w(st0, s_begin);
    resolve_rows();
    if (s_begin < s_end) load_a(st0, s_begin);
    for (int s = s_begin; s < s_end; s += 2) {
      if (s + 1 < s_end) load(st1, s + 1);
      compute(st0);
      if (s + 1 < s_end) {
        if (s + 2 < s_end) load(st0, s + 2);
        compute(st1);
      }
    }
  } else {
    // 32-row tiles carry twice the accumulators: one stage, loads of a step
    // still issued together before its MFMAs
    resolve_rows();
    for (int s = s_begin; s < s_end; ++s) {
      Stage st;
      load(st, s);
      compute(st);
    }
  }

  // cross-wave reduction of the split-K partial sums through LDS, up to 64
  // registers a round (one round for 16-row tiles): every block ends here at
  // about the same time, so the fewer barriers the shorter the exposed tail
  if (KSPLIT > 1) {
    constexpr int NREG = 2 * RG * 8 * 4;
    constexpr int RR = NREG < 64 ? NREG : 64;
    __shared__ float red[(KSPLIT > 1 ? KSPLIT - 1 : 1) * RR * 64];
#pragma unroll
    for (int q = 0; q < NREG / RR; ++q) {
      if (wave > 0) {
#pragma unroll
        for (int j = 0; j < RR; ++j) {
          const int rgi = q * RR + j;
          const int h = rgi / (RG * 32), rg = (rgi / 32) % RG;
          const int i = (rgi / 4) % 8, e = rgi % 4;
          red[((wave - 1) * RR + j) * 64 + lane] = acc[h][rg][i][e];
        }
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int j = 0; j < RR; ++j) {
          const int rgi = q * RR + j;
          const int h = rgi / (RG * 32), rg = (rgi / 32) % RG;
          const int i = (rgi / 4) % 8, e = rgi % 4;
          float sum = acc[h][rg][i][e];
#pragma unroll
          for (int ww = 0; ww < KSPLIT - 1; ++ww)
            sum += red[(ww * RR + j) * 64 + lane];
          acc[h][rg][i][e] = sum;
        }
      }
      if (q + 1 < NREG / RR) __syncthreads();
    }
    if (wave > 0) return;
  }

  // epilogue: lane owns rows 16*rg + 4*kq + e, columns colA + 0..7 (+ colB).
  // 32-row tiles come with outputs of tens of MB (the LongCat-shaped layer's
  // y is 100 MB, its h 33 MB), stored while every other wave streams
  // weights: written nontemporally, its GEMM2 measured 2018 -> 1958 us and
  // GEMM1 3777 -> 3760 us (layer 5844 -> 5781 us, outputs identical). A
  // timing-only build without the y stores ran GEMM2 in 1818 us. The
  // 16-row decode tiles write a few MB, which the next kernel reads from
  // the caches, and keep plain stores (nontemporal: neutral to 0.5 % slower).
  constexpr bool NT_OUT = RG == 2;
  auto store_out = [&](uint16_t* p, uint4 o) {
    if constexpr (NT_OUT)
      __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w}, (u32x4_t*)p);
    else
      *(uint4*)p = o;
  };
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rg + 4 * kq + e;
      if (r >= tl.rows) continue;
      uint16_t* orow = out + (size_t)(tl.row0 + r) * Nout;
      if (GLU) {
        if (okA) {
          float hv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            hv[i] = silu(acc[0][rg][i][e]) * acc[1][rg][i][e];
          uint4 o;
          o.x = pack_bf16x2(hv[0], hv[1]);
          o.y = pack_bf16x2(hv[2], hv[3]);
          o.z = pack_bf16x2(hv[4], hv[5]);
          o.w = pack_bf16x2(hv[6], hv[7]);
          store_out(orow + colA, o);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 0 ? !okA : !okB) continue;
          uint4 o;
          o.x = pack_bf16x2(acc[h][rg][0][e], acc[h][rg][1][e]);
          o.y = pack_bf16x2(acc[h][rg][2][e], acc[h][rg][3][e]);
          o.z = pack_bf16x2(acc[h][rg][4][e], acc[h][rg][5][e]);
          o.w = pack_bf16x2(acc[h][rg][6][e], acc[h][rg][7][e]);
          store_out(orow + (h == 0 ? colA : colB), o);
        }
      }
    }
  }
}

template <bool GLU, int RG, bool PK>
static hipError_t launch_stream(int ksplit, dim3 grid, const Tile* tiles,
                                const int32_t* tile_count, const uint16_t* a,
                                const uint16_t* w, uint16_t* out, int K, int Nw,
                                int Nout, const int32_t* gidx,
                                const int32_t* gbase, int gk, hipStream_t s) {
  switch (ksplit) {  // 1 or 3 (stream_ksplit)
    case 1:
      hipLaunchKernelGGL((gemm_bf16_stream_kernel<GLU, RG, 1, PK>), grid,
                         dim3(64), 0, s, tiles, tile_count, a, w, out, K, Nw,
                         Nout, gidx, gbase, gk);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_stream_kernel<GLU, RG, 3, PK>), grid,
                         dim3(192), 0, s, tiles, tile_count, a, w, out, K, Nw,
                         Nout, gidx, gbase, gk);
      break;
  }
  return hipGetLastError();
}

template <bool GLU, bool PK>
static hipError_t launch_stream_rg(int rg, int ksplit, dim3 grid,
                                   const Tile* tiles, const int32_t* tile_count,
                                   const uint16_t* a, const uint16_t* w,
                                   uint16_t* out, int K, int Nw, int Nout,
                                   const int32_t* gidx, const int32_t* gbase,
                                   int gk, hipStream_t s) {
  return rg == 1 ? launch_stream<GLU, 1, PK>(ksplit, grid, tiles, tile_count,
                                             a, w, out, K, Nw, Nout, gidx,
                                             gbase, gk, s)
                 : launch_stream<GLU, 2, PK>(ksplit, grid, tiles, tile_count,
                                             a, w, out, K, Nw, Nout, gidx,
                                             gbase, gk, s);
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n <= 0)
    return 256;
  return n;
}

// Waves per block that split K. Decode launches have few (tile, slab) blocks;
// splitting K across 3 waves fills the chip, but only as far as every block
// stays resident in one round and each wave keeps at least 4 steps. At two
// waves per SIMD a CU holds 8 waves, i.e. floor(8 / 3) = 2 blocks of 3
// waves: a 3-way split holds 512 blocks per round on 256 CUs, not 2048 / 3
// (counting wave slots let the decode GEMM1's 666 blocks spill into a
// partial second round, which cost it 3-4 %). Beyond that one wave per
// block: with the weights streamed nontemporally, a 2-way split of the
// decode GEMMs' 616-822 blocks was 1.5-2.5 % slower than none (Qwen3-30B
// decode layer 179.2 vs 176.5 us at 32 tokens, 203.3 vs 198.2 us at 64),
// while at 1-6 tokens the 3-way split stays 0.1-20 us ahead. The grid is
// sized for the host's upper bound on the tile count; the tiles that exist
// on the device are typically 3/4 of it.
int stream_ksplit(long long blocks, int steps, int rg) {
  (void)rg;
  if (blocks * 3 / 4 <= (long long)device_cus() * (8 / 3) && steps / 3 >= 4)
    return 3;
  return 1;
}

int stream_bf16_slabs(bool glu, int Nout) {
  const int slab = glu ? 128 : 256;
  return (Nout + slab - 1) / slab;
}

int stream_bf16_ksplit(bool glu, int max_tiles, int K, int Nout, int rg) {
  return stream_ksplit((long long)stream_bf16_slabs(glu, Nout) * max_tiles,
                       K / 32, rg);
}

hipError_t launch_gemm_bf16_stream(bool glu, int rg, const Tile* tiles,
                                   const int32_t* tile_count, int max_tiles,
                                   const uint16_t* a, const uint16_t* w,
                                   uint16_t* out, int K, int Nw, int Nout,
                                   const int32_t* gidx, const int32_t* gbase,
                                   int gk, hipStream_t s, bool pk) {
  if (max_tiles == 0) return hipSuccess;
  // packed slabs are whole: 256 weight columns, K in steps of 32
  if (pk && (K % 32 || Nw % 256)) return hipErrorInvalidValue;
  // (max_tiles < 65536: this schedule serves fewer than 20 rows per expert)
  dim3 grid(stream_bf16_slabs(glu, Nout), max_tiles);
  const int ksplit = stream_bf16_ksplit(glu, max_tiles, K, Nout, rg);
  if (glu)
    return pk ? launch_stream_rg<true, true>(rg, ksplit, grid, tiles,
                                             tile_count, a, w, out, K, Nw, Nout,
                                             gidx, gbase, gk, s)
              : launch_stream_rg<true, false>(rg, ksplit, grid, tiles,
                                              tile_count, a, w, out, K, Nw,
                                              Nout, gidx, gbase, gk, s);
  return pk ? launch_stream_rg<false, true>(rg, ksplit, grid, tiles,
                                            tile_count, a, w, out, K, Nw, Nout,
                                            gidx, gbase, gk, s)
            : launch_stream_rg<false, false>(rg, ksplit, grid, tiles,
                                             tile_count, a, w, out, K, Nw,
                                             Nout, gidx, gbase, gk, s);
}

}  // namespace moe
