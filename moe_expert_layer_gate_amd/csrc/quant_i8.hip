// Dynamic per-row int8 quantisation of activations for the W8A8 experts.
//
// [P3] "NPU Qwen3-Next inference practice", section 量化策略: the routed
// experts run W8A8 -- int8 weights with a static scale per output channel and
// int8 activations with a dynamic scale per token. Applied here to the tokens
// of x (once, before routing; GEMM1 gathers the token rows of the codes) and
// to the rows of h between the two GEMMs.
//
// Row r: amax = max |v|; scale = amax / 127 rounded to nearest fp32; code =
// rint(v / scale) with the quotient rounded to nearest fp32 and rint taking
// ties to even, clipped to [-127, 127]. An all-zero row gets scale 0 and codes
// 0. Divisions are the correctly rounded fp32 division (__fdiv_rn), so codes
// and scales are bit-identical to any other IEEE evaluation of that rule.
//
// One wave per row, 8 elements (16 or 32 bytes) per lane and chunk of 512.
// Rows up to 8192 elements stay in registers between the amax and the codes
// (one read); longer rows are read twice.
#include "common.h"
#include "launch.h"
#include "quant_row.h"

namespace moe {

namespace {

// rows: offs == NULL: nrows rows, row r reads source row r. Otherwise the
// R = offs[fe] - offs[fb] rows of the sorted copies of experts [fb, fe); row r
// reads source row gidx[offs[fb] + r] / gk (gidx != NULL) or r.
template <bool F32, int CPL>
__global__ __launch_bounds__(256) void quant_i8_rows_kernel(
    const void* __restrict__ src, int K, int nrows,
    const int32_t* __restrict__ gidx, const int32_t* __restrict__ offs, int fb,
    int fe, int gk, int8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  int R = nrows, base = 0;
  if (offs) {
    base = offs[fb];
    R = offs[fe] - base;
  }
  if (r >= R) return;
  const int srow = gidx ? gidx[base + r] / gk : r;
  quant_i8_row<F32, CPL>(src, K, (size_t)srow * K, codes + (size_t)r * K,
                         scales + r, lane);
}

template <bool F32>
hipError_t launch_rows(int cpl, dim3 grid, hipStream_t s, const void* src,
                       int K, int nrows, const int32_t* gidx,
                       const int32_t* offs, int fb, int fe, int gk,
                       int8_t* codes, float* scales) {
#define MOE_Q(C)                                                              \
  hipLaunchKernelGGL((quant_i8_rows_kernel<F32, C>), grid, dim3(256), 0, s,   \
                     src, K, nrows, gidx, offs, fb, fe, gk, codes, scales)
  switch (cpl) {
    case 1: MOE_Q(1); break;
    case 2: MOE_Q(2); break;
    case 3: MOE_Q(3); break;
    case 4: MOE_Q(4); break;
    case 6: MOE_Q(6); break;
    case 8: MOE_Q(8); break;
    case 12: MOE_Q(12); break;
    case 16: MOE_Q(16); break;
    default: MOE_Q(0); break;
  }
#undef MOE_Q
  return hipGetLastError();
}

}  // namespace

// Packed weights: thread i moves 16-byte fragment piece i. Piece i of the
// packed buffer is lane l = i % 64 of fragment f = i / 64,
// f = (e * Kb/64 + c) * N/16 + n16; it holds row 16 * n16 + l % 16, bytes
// [64 c + 16 (l / 16), + 16) of expert e's [N, Kb] byte matrix. Writes are
// contiguous; reads gather 16 bytes per lane (a one-time step).
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
    long long npieces, int N, int Kb) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= npieces) return;
  const int l = (int)(i & 63);
  long long f = i >> 6;
  const int n16 = (int)(f % (N / 16));
  f /= N / 16;
  const int nc = Kb / 64;
  const int c = (int)(f % nc);
  const long long e = f / nc;
  const long long so = (e * N + 16 * n16 + (l & 15)) * (long long)Kb + 64 * c +
                       16 * (l >> 4);
  *(uint4*)(dst + 16 * i) = *(const uint4*)(src + so);
}

hipError_t launch_pack_weights(int E, int N, int Kb, const uint8_t* src,
                               uint8_t* dst, hipStream_t s) {
  const long long npieces = (long long)E * N * Kb / 16;
  if (npieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weights_kernel,
                     dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0, s,
                     src, dst, npieces, N, Kb);
  return hipGetLastError();
}

hipError_t launch_quant_i8_rows(bool f32, const void* src, int K, int nrows,
                                const int32_t* gidx, const int32_t* offs,
                                int fb, int fe, int gk, int8_t* codes,
                                float* scales, hipStream_t s) {
  if (nrows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nrows + 3) / 4));
  // chunks of 512 elements per row, rounded up to an instantiated count
  int cpl = (K + 511) / 512;
  for (int c : {1, 2, 3, 4, 6, 8, 12, 16})
    if (cpl <= c) { cpl = c; break; }
  if (cpl > 16) cpl = 0;
  return f32 ? launch_rows<true>(cpl, grid, s, src, K, nrows, gidx, offs, fb,
                                 fe, gk, codes, scales)
             : launch_rows<false>(cpl, grid, s, src, K, nrows, gidx, offs, fb,
                                  fe, gk, codes, scales);
}

}  // namespace moe
