// Slab packing of static bf16 expert weights.
//
// [P2] "LongCat-Flash inference on Atlas A3 clusters" notes that the decode
// grouped matmuls are memory-bound: their time is the time to stream the
// expert weights. The bf16 GEMMs split an expert's weight matrix [K, N] into
// slabs of 256 columns (GEMM1: 128 gate columns and the 128 matching up
// columns; GEMM2: 256 consecutive columns) and walk each slab along K in
// steps of 32 rows. Row-major, the 32 x 256 block of one step is 32 pieces of
// 512 bytes at a stride of 2N bytes, and the blocks reading the slabs of one
// expert share each DRAM row; once their MFMA work makes them drift apart
// that sharing is lost (measured on MI355X with the LongCat-shaped GEMM1
// pattern: 6.55 TB/s row-major against 7.05 TB/s with each slab stored
// contiguously). While the blocks run in step -- one round of equal blocks,
// as at decode batch sizes on small experts -- the shared rows pay instead,
// and row-major stays ahead. Packed, step s of slab j is one contiguous
// 16 KB block:
//   dst[e][j][s][r][c] = W[e][32 s + r][col_j(c)],  r < 32, c < 256,
//   col_j(c) = 128 j + c (c < 128) and N/2 + 128 j + c - 128 (c >= 128)
//   for a gate/up matrix, 256 j + c otherwise.
// Packed once, when the weights are loaded.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// one 16-byte piece (8 columns of one row) per thread
__global__ __launch_bounds__(256) void pack_bf16_kernel(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
    long long npieces, int K, int N, int glu) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= npieces) return;
  const int p = (int)(i & 31);               // piece of the 512-byte row
  const int r = (int)((i >> 5) & 31);        // row of the step
  long long f = i >> 10;                     // (e, j, s)
  const int nst = K / 32;
  const int s = (int)(f % nst);
  f /= nst;
  const int nsl = N / 256;
  const int j = (int)(f % nsl);
  const long long e = f / nsl;
  const int c = 8 * p;
  const int col = glu ? (c < 128 ? 128 * j + c : N / 2 + 128 * j + c - 128)
                      : 256 * j + c;
  const long long so = (e * K + 32LL * s + r) * N + col;
  *(uint4*)(dst + 8 * i) = *(const uint4*)(src + so);
}

}  // namespace

hipError_t launch_pack_bf16_weights(int E, int K, int N, bool glu,
                                    const uint16_t* src, uint16_t* dst,
                                    hipStream_t s) {
  const long long npieces = (long long)E * K * N / 8;
  if (npieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_bf16_kernel,
                     dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0, s,
                     src, dst, npieces, K, N, glu ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
