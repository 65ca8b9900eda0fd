// Grouped GEMM, W8A8 (int8 x int8 -> int32 on MFMA), weight-streaming
// schedule for decode-size batches.
//
// [P3] "NPU Qwen3-Next inference practice", section 量化策略: routed experts
// in W8A8 -- int8 weights with a static scale per output channel, int8
// activations with a dynamic scale per token. [P1] "Qwen3-MoE low-latency
// inference on Atlas A3 / 950 clusters", MoE TP优化 / 计算分解 (expert =
// down(SiLU(gate(x)) * up(x)), merged gate/up) and 高性能专家计算 (one grouped
// operator); [P2] "LongCat-Flash inference on Atlas A3 clusters": the decode
// grouped matmuls are memory-bound, so this kernel streams weights from HBM
// straight into registers.
//
// v_mfma_i32_16x16x64_i8: lane l holds 16 bytes of row (A) / column (B) l%16.
// Per K step of 128, MFMA m (0, 1) takes from lane l (q = l/16) bytes
// [64m + 16q, +16) of its activation row and of its weight column. A and B
// lanes hold the same K offsets, so the two MFMAs sum every K of the step
// exactly, whatever order the hardware takes them in. Activation rows are
// K-contiguous and read in place; the weights come packed (one 1 KB
// fragment per 64-byte K chunk and 16 columns, in exactly this lane order,
// the column groups of a chunk adjacent: chunk c of group n16 at
// c * N * 64 + n16 * 1024), so every weight load of a wave reads 1 KB
// contiguous; MFMA m of step s takes chunk 2s + m.
//
// Each lane carries 8 groups of 16 weight columns: for GEMM1 4 gate groups and
// the 4 matching up groups (64 h columns per block, SwiGLU lane-local), for
// GEMM2 8 groups (128 output columns). KSPLIT waves split K and add their
// int32 partial sums in LDS; wave 0 dequantises (row scale * column scale),
// applies SwiGLU and stores h in fp32, or y in bf16.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

MOE_DEV i32x4_t mfma_i8(uint4 a, uint4 b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(
      i32x4_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w},
      i32x4_t{(int)b.x, (int)b.y, (int)b.z, (int)b.w}, c, 0, 0, 0);
}

}  // namespace

// Two waves per SIMD, as the bf16 streaming kernel (register budget 256).
template <bool GLU, int RG, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT)
__attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_i8_stream_kernel(
    const Tile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    const int8_t* __restrict__ a, const float* __restrict__ as,
    const int8_t* __restrict__ w, const float* __restrict__ ws,
    void* __restrict__ out, int K, int Nw, int Nout,
    const int32_t* __restrict__ gidx, const int32_t* __restrict__ gbase,
    int gk) {
  constexpr int NG = 8;                 // 16-column groups per lane
  constexpr int SLAB = GLU ? 64 : 128;  // output columns per block
  // tile entry and count read together (entries past the count are in
  // bounds, merely stale); the empty asm keeps both ahead of the exit test
  // grid: x = column slab, y = tile (consecutive blocks: one expert's slabs)
  const Tile tl = tiles[blockIdx.y];
  const int ntiles = tile_count[0];
  asm volatile("" ::"s"(ntiles), "s"(tl.expert), "s"(tl.row0), "s"(tl.rows));
  if ((int)blockIdx.y >= ntiles) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & 15, q = lane >> 4;
  const int c0 = blockIdx.x * SLAB;
  const int8_t* we = w + (size_t)tl.expert * Nw * K;

  // Columns past N and rows past the tile only feed outputs that are never
  // stored; their loads read column group / row 0, so every load is
  // unconditional. (N is a multiple of 16: a group is in or out whole.)
  int col[NG];
  bool cok[NG];
  uint32_t frag[NG];  // byte offset of the group's K-block-0 fragment + lane
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int c = GLU ? c0 + 16 * (gi & 3) + g : c0 + 16 * gi + g;
    cok[gi] = c < Nout;
    col[gi] = cok[gi] ? ((GLU && gi >= 4) ? Nout + c : c) : 0;
    const int n16 = cok[gi] ? (col[gi] - g) / 16 : 0;  // group's column / 16
    frag[gi] = (uint32_t)n16 * 1024u + 16u * lane;
  }
  // A rows are resolved after the first step's weight loads are issued
  // (the gather index is two dependent loads away)
  const int8_t* arow[RG];
  auto resolve_rows = [&]() {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int r = 16 * rg + g;
      int src = tl.row0 + (r < tl.rows ? r : 0);
      if (gidx) src = gidx[gbase[0] + src] / gk;  // fused gather of token rows
      arow[rg] = a + (size_t)src * K + 16 * q;
    }
  };

  i32x4_t acc[NG][RG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) acc[gi][rg] = i32x4_t{0, 0, 0, 0};

  struct Stage {
    uint4 b[NG][2];
    uint4 a[RG][2];
  };
  auto load_w = [&](Stage& st, int s) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int8_t* p = we + frag[gi] + (size_t)(2 * s) * Nw * 64;
      st.b[gi][0] = load_stream16(p);
      st.b[gi][1] = load_stream16(p + (size_t)Nw * 64);
    }
  };
  auto load_a = [&](Stage& st, int s) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      st.a[rg][0] = *(const uint4*)(arow[rg] + (size_t)s * 128);
      st.a[rg][1] = *(const uint4*)(arow[rg] + (size_t)s * 128 + 64);
    }
  };
  auto load = [&](Stage& st, int s) {
    load_w(st, s);
    load_a(st, s);
  };
  auto compute = [&](const Stage& st) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        acc[gi][rg] = mfma_i8(st.a[rg][0], st.b[gi][0], acc[gi][rg]);
        acc[gi][rg] = mfma_i8(st.a[rg][1], st.b[gi][1], acc[gi][rg]);
      }
  };
  const int nsteps = K / 128;
  const int s_begin = wave * nsteps / KSPLIT;
  const int s_end = (wave + 1) * nsteps / KSPLIT;
  if (RG == 1) {
    // two register stages: step s+1's loads are in flight during step s
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
    resolve_rows();
    for (int s = s_begin; s < s_end; ++s) {
      Stage st;
      load(st, s);
      compute(st);
    }
  }

  // exact int32 partial sums of the K-split waves meet in LDS (one round)
  if (KSPLIT > 1) {
    constexpr int NREG = NG * RG * 4;
    __shared__ int red[(KSPLIT > 1 ? KSPLIT - 1 : 1) * NREG * 64];
    if (wave > 0) {
#pragma unroll
      for (int x = 0; x < NREG; ++x)
        red[((wave - 1) * NREG + x) * 64 + lane] = acc[x / (RG * 4)][(x / 4) % RG][x % 4];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int x = 0; x < NREG; ++x) {
      int sum = acc[x / (RG * 4)][(x / 4) % RG][x % 4];
#pragma unroll
      for (int ww = 0; ww < KSPLIT - 1; ++ww) sum += red[(ww * NREG + x) * 64 + lane];
      acc[x / (RG * 4)][(x / 4) % RG][x % 4] = sum;
    }
  }

  // epilogue: lane holds rows 16*rg + 4*q + e of column col[gi]
  float cs[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) cs[gi] = ws[(size_t)tl.expert * Nw + col[gi]];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rg + 4 * q + e;
      if (r >= tl.rows) continue;
      const int orow = tl.row0 + r;
      const float rsc = as[gidx ? gidx[gbase[0] + orow] / gk : orow];
      if (GLU) {
        float* o = (float*)out + (size_t)orow * Nout;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          if (!cok[gi]) continue;
          const float gv = (float)acc[gi][rg][e] * rsc * cs[gi];
          const float uv = (float)acc[gi + 4][rg][e] * rsc * cs[gi + 4];
          o[c0 + 16 * gi + g] = silu(gv) * uv;
        }
      } else {
        uint16_t* o = (uint16_t*)out + (size_t)orow * Nout;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          if (cok[gi])
            o[col[gi]] = (uint16_t)f32_to_bf16_bits((float)acc[gi][rg][e] * rsc * cs[gi]);
      }
    }
  }
}

namespace {

template <bool GLU, int RG>
hipError_t launch_i8s(int ksplit, dim3 grid, const Tile* tiles,
                      const int32_t* tile_count, const int8_t* a,
                      const float* as, const int8_t* w, const float* ws,
                      void* out, int K, int Nw, int Nout, const int32_t* gidx,
                      const int32_t* gbase, int gk, hipStream_t s) {
  switch (ksplit) {  // 1 or 3 (stream_ksplit)
    case 1:
      hipLaunchKernelGGL((gemm_i8_stream_kernel<GLU, RG, 1>), grid, dim3(64), 0,
                         s, tiles, tile_count, a, as, w, ws, out, K, Nw, Nout,
                         gidx, gbase, gk);
      break;
    default:
      hipLaunchKernelGGL((gemm_i8_stream_kernel<GLU, RG, 3>), grid, dim3(192),
                         0, s, tiles, tile_count, a, as, w, ws, out, K, Nw,
                         Nout, gidx, gbase, gk);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int stream_i8_slabs(bool glu, int Nout) {
  const int slab = glu ? 64 : 128;
  return (Nout + slab - 1) / slab;
}

// a step of 128 K moves as many weight bytes per wave (16 KB) as a bf16 step
// of 32, so the bf16 kernel's split rule applies in these steps
int stream_i8_ksplit(bool glu, int max_tiles, int K, int Nout, int rg) {
  return stream_ksplit((long long)stream_i8_slabs(glu, Nout) * max_tiles,
                       K / 128, rg);
}

hipError_t launch_gemm_i8_stream(bool glu, int rg, const Tile* tiles,
                                 const int32_t* tile_count, int max_tiles,
                                 const int8_t* a, const float* a_scale,
                                 const int8_t* w, const float* w_scale,
                                 void* out, int K, int Nw, int Nout,
                                 const int32_t* gidx, const int32_t* gbase,
                                 int gk, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  // (max_tiles < 65536: this schedule serves fewer than 10 rows per expert)
  dim3 grid(stream_i8_slabs(glu, Nout), max_tiles);
  const int ksplit = stream_i8_ksplit(glu, max_tiles, K, Nout, rg);
  // 16-row tiles only: below the tiled kernel's switch (10 rows per expert)
  // 32-row tiles measured 8-12 % slower
  if (rg != 1) return hipErrorInvalidValue;
  if (glu)
    return launch_i8s<true, 1>(ksplit, grid, tiles, tile_count, a, a_scale, w,
                               w_scale, out, K, Nw, Nout, gidx, gbase, gk, s);
  return launch_i8s<false, 1>(ksplit, grid, tiles, tile_count, a, a_scale, w,
                              w_scale, out, K, Nw, Nout, gidx, gbase, gk, s);
}

}  // namespace moe
