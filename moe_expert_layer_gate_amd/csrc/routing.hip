// Routing: expert histogram, offsets, stable permutation, gather (+ MXFP8).
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// section 高效排序和token路由: sort the token copies by expert (init_routing)
// and count the tokens of each expert (compute_expert_tokens); section MoE
// EP优化 / AllGather方案(W4A8量化): quantise hidden states to MXFP8 and keep
// only the copies of the local expert range.
//
// Copies c = t * k + j are cut into chunks of 256 (one wavefront each).
//   count   : per-chunk LDS histogram -> chunk_counts[chunk][E]
//   scan    : one block; per expert an exclusive scan over chunks (in place,
//             giving each chunk its first slot inside the expert), the
//             expert totals, their exclusive scan (offsets) and, optionally,
//             the GEMM tile list of the local FFN experts
//   scatter : each wave re-reads its chunk 64 copies at a time in order; the
//             lanes holding equal ids are found by intersecting one ballot
//             per bit of the id, and a copy's rank is the number of equal
//             lanes below it, so copies of one expert keep ascending c: the
//             sort key is (expert, c) and the result is deterministic
//   gather  : one wave per routed row copies (or MXFP8-quantises) x[t]
#include "common.h"
#include "launch.h"
#include "quant_row.h"

namespace moe {

constexpr int kChunk = 256;
constexpr int kMaxE = 2048;
constexpr int kScanRegs = 16;  // chunk counts a scan thread keeps in registers

int route_num_chunks(int N) { return (N + kChunk - 1) / kChunk; }

__global__ __launch_bounds__(256) void route_count_kernel(
    const int32_t* __restrict__ ids, int N, int E, int nchunks,
    int32_t* __restrict__ cc) {
  extern __shared__ int32_t sh[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + w;
  int32_t* h = sh + w * E;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  if (c < nchunks) {
#pragma unroll
    for (int it = 0; it < kChunk / 64; ++it) {
      int i = c * kChunk + it * 64 + lane;
      if (i < N) {
        int e = ids[i];
        if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
      }
    }
  }
  __syncthreads();
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) cc[(size_t)c * E + e] = h[e];
}

// Exclusive scan of a[0..n) in LDS by a block of 1024 threads, n <= 2048.
// Returns the total to every thread.
__device__ int block_exclusive_scan(int32_t* a, int n, int32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = 2 * tid, i1 = i0 + 1;
  int v0 = i0 < n ? a[i0] : 0;
  int v1 = i1 < n ? a[i1] : 0;
  int s = v0 + v1, x = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int z = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      int y = __shfl_up(z, off);
      if (lane >= off) z += y;
    }
    if (lane < 16) wsum[lane] = z;
  }
  __syncthreads();
  int base = (w ? wsum[w - 1] : 0) + x - s;
  int total = wsum[15];
  if (i0 < n) a[i0] = base;
  if (i1 < n) a[i1] = base + v0;
  __syncthreads();
  return total;
}

// Tile list of the FFN experts [fb, fe): expert e gets ceil(count/mt) tiles.
__device__ void build_tiles_block(const int32_t* cnt_lds, const int32_t* off_lds,
                                  int fb, int fe, int mt, Tile* tiles,
                                  int max_tiles, int32_t* tile_count,
                                  int32_t* tmp, int32_t* wsum) {
  const int El = fe - fb;
  for (int i = threadIdx.x; i < El; i += blockDim.x)
    tmp[i] = (cnt_lds[fb + i] + mt - 1) / mt;
  __syncthreads();
  const int total = block_exclusive_scan(tmp, El, wsum);
  const int r0 = off_lds[fb];
  // one thread per tile: its expert is the last one whose first tile is at
  // or before it (experts without tiles share their successor's start)
  const int nt = min(total, max_tiles);
  for (int ti = threadIdx.x; ti < nt; ti += blockDim.x) {
    int lo = 0, hi = El - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tmp[mid] <= ti) lo = mid;
      else hi = mid - 1;
    }
    const int n = cnt_lds[fb + lo], m = ti - tmp[lo];
    Tile tl;
    tl.expert = lo;
    tl.row0 = off_lds[fb + lo] - r0 + m * mt;
    tl.rows = min(mt, n - m * mt);
    tl.first = tmp[lo];
    tl.count = (n + mt - 1) / mt;
    tl.pad[0] = tl.pad[1] = tl.pad[2] = 0;
    tiles[ti] = tl;
  }
  if (threadIdx.x == 0) tile_count[0] = nt;
}

// Optional per-token quantisation of x riding along with the scan (RowQuant
// with nrows > 0): blocks 1, 2, ... quantise 16 rows each (one wave per
// row) while block 0 scans. The scan is one latency-bound block, so the
// quantisation -- which the routing does not need -- fills the idle chip.
// Q = 1: MXFP8 (e4m3 codes [T, H] + e8m0 [T, H/32]); Q = 2: int8 with CPL
// chunks of 512 per lane (CPL = 0: any H, read twice).
struct RowQuant {
  const uint16_t* x;
  int H, nrows;
  void* codes;
  void* scales;
};

template <int Q, int CPL>
__global__ __launch_bounds__(1024) void route_scan_kernel(
    int32_t* __restrict__ cc, int nchunks, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int fb, int fe, int mt, Tile* tiles,
    int max_tiles, int32_t* tile_count, RowQuant rq) {
  if (Q != 0 && blockIdx.x > 0) {
    const int t = (blockIdx.x - 1) * 16 + (threadIdx.x >> 6);
    if (t >= rq.nrows) return;  // whole wave
    const int lane = threadIdx.x & 63;
    if (Q == 1)
      quant_mx_row_bf16((const uint4*)(rq.x + (size_t)t * rq.H), rq.H,
                        (uint8_t*)rq.codes + (size_t)t * rq.H,
                        (uint8_t*)rq.scales + (size_t)t * (rq.H / 32), lane);
    else
      quant_i8_row<false, CPL>(rq.x, rq.H, (size_t)t * rq.H,
                               (int8_t*)rq.codes + (size_t)t * rq.H,
                               (float*)rq.scales + t, lane);
    return;
  }
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int32_t tmp[kMaxE];
  __shared__ int32_t wsum[16];
  __shared__ int32_t part[1024];
  // tpe threads per expert split the chunks into contiguous ranges of at
  // most kScanRegs: each thread loads its range once into registers (all
  // loads in flight together), the range sums are scanned in LDS, and every
  // chunk count is rewritten as its exclusive prefix within the expert. Only
  // if a range cannot fit (more than 1024 * kScanRegs / E chunks) are the
  // counts read a second time.
  int tpe = 1;
  while (tpe * 2 * E <= (int)blockDim.x) tpe *= 2;
  while (tpe < (int)blockDim.x && (nchunks + tpe - 1) / tpe > kScanRegs) tpe *= 2;
  const int per = (nchunks + tpe - 1) / tpe;
  // consecutive threads take consecutive experts of one chunk range, so each
  // load and store of a wave covers 64 adjacent counts of one chunk row
  const int epp = (int)blockDim.x / tpe;  // experts per pass
  for (int e0 = 0; e0 < E; e0 += epp) {
    const int e = e0 + (int)threadIdx.x % epp, q = (int)threadIdx.x / epp;
    const bool act = e < E;
    const int c0 = q * per, c1 = min(nchunks, c0 + per);
    int sum = 0;
    int v[kScanRegs];
    if (per <= kScanRegs) {
#pragma unroll
      for (int j = 0; j < kScanRegs; ++j)
        v[j] = act && c0 + j < c1 ? cc[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanRegs; ++j) sum += v[j];
    } else if (act) {
      for (int c = c0; c < c1; c += 8) {
        int u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          u[j] = c + j < c1 ? cc[(size_t)(c + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += u[j];
      }
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    if (act) {
      int base = 0;
      for (int j = 0; j < q; ++j) base += part[j * epp + (int)threadIdx.x % epp];
      if (q == tpe - 1) { cnt[e] = base + sum; off[e] = base + sum; counts[e] = base + sum; }
      if (per <= kScanRegs) {
#pragma unroll
        for (int j = 0; j < kScanRegs; ++j)
          if (c0 + j < c1) {
            cc[(size_t)(c0 + j) * E + e] = base;
            base += v[j];
          }
      } else {
        for (int c = c0; c < c1; c += 8) {
          int u[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            u[j] = c + j < c1 ? cc[(size_t)(c + j) * E + e] : 0;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c + j < c1) {
              cc[(size_t)(c + j) * E + e] = base;
              base += u[j];
            }
        }
      }
    }
    __syncthreads();
  }
  int total = block_exclusive_scan(off, E, wsum);
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = off[e];
  if (threadIdx.x == 0) { offsets[E] = total; off[E] = total; }
  __syncthreads();
  if (tiles) build_tiles_block(cnt, off, fb, fe, mt, tiles, max_tiles,
                               tile_count, tmp, wsum);
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(
    const int32_t* __restrict__ offsets, int fb, int fe, int mt, Tile* tiles,
    int max_tiles, int32_t* tile_count) {
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t off[kMaxE + 1];
  __shared__ int32_t tmp[kMaxE];
  __shared__ int32_t wsum[16];
  for (int e = fb + threadIdx.x; e <= fe; e += blockDim.x) {
    off[e] = offsets[e];
    if (e < fe) cnt[e] = offsets[e + 1] - offsets[e];
  }
  __syncthreads();
  build_tiles_block(cnt, off, fb, fe, mt, tiles, max_tiles, tile_count, tmp,
                    wsum);
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int N, int E, int nchunks,
    const int32_t* __restrict__ cc, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_copy, int32_t* __restrict__ copy_pos) {
  extern __shared__ int32_t sh[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + w;
  volatile int32_t* base = sh + w * E;
  if (c < nchunks)
    for (int e = lane; e < E; e += 64)
      base[e] = offsets[e] + cc[(size_t)c * E + e];
  __syncthreads();
  if (c >= nchunks) return;
  const uint64_t lt = lanemask_lt();
  const uint64_t gt = ~lt & ~(1ull << lane);
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int it = 0; it < kChunk / 64; ++it) {
    const int i = c * kChunk + it * 64 + lane;
    const int e = i < N ? ids[i] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    if (i < N && !valid) copy_pos[i] = -1;
    // lanes holding the same expert id: intersect one ballot per id bit
    uint64_t m = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = ballot(valid && bit);
      m &= bit ? ones : ~ones;
    }
    if (valid) {
      const int b0 = base[e];  // every reader sees the value before this step
      const int pos = b0 + popc64(m & lt);
      sorted_copy[pos] = i;
      copy_pos[i] = pos;
      if ((m & gt) == 0) base[e] = b0 + popc64(m);  // last lane of its group
    }
  }
}

// Single-block routing for small problems (N <= 4096 copies, E <= 1024):
// per-wave histograms over contiguous chunks of copies, the scans, the GEMM
// tile list and the stable scatter, all in one launch with the counts kept
// in LDS. Same results as count + scan + scatter. (Running the gate inside
// this block as well was measured slower at T = 32: 13.2 us against 4.6 us
// for the gate kernel spread over 8 CUs plus 5.0 us for this one.)
constexpr int kSmallMaxN = 4096, kSmallMaxE = 1024;

template <int PER>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const int32_t* __restrict__ ids, int N, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_copy, int32_t* __restrict__ copy_pos, int fb,
    int fe, int mt, Tile* tiles, int max_tiles, int32_t* tile_count) {
  __shared__ int32_t hist[16][kSmallMaxE];
  __shared__ int32_t cnt[kSmallMaxE];
  __shared__ int32_t off[kSmallMaxE + 1];
  __shared__ int32_t tmp[kSmallMaxE];
  __shared__ int32_t wsum[16];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // wave w owns copies [c0, c1), a multiple of 64 long
  const int C = ((N + 16 * 64 - 1) / (16 * 64)) * 64;
  const int c0 = min(N, w * C), c1 = min(N, c0 + C);
  // the wave's ids stay in registers: all loads issue back to back, and the
  // count and the scatter both read them from there
  constexpr int kPerLane = PER;  // copies per lane: N <= 1024 * PER
  int idr[kPerLane];
#pragma unroll
  for (int it = 0; it < kPerLane; ++it) {
    const int i = c0 + it * 64 + lane;
    const int v = N > 0 ? ids[min(i, N - 1)] : -1;
    idr[it] = i < c1 ? v : -1;
  }
  for (int e = lane; e < E; e += 64) hist[w][e] = 0;
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kPerLane; ++it)
    if ((unsigned)idr[it] < (unsigned)E) atomicAdd(&hist[w][idr[it]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) {
      const int v = hist[ww][e];
      hist[ww][e] = run;
      run += v;
    }
    cnt[e] = run;
    off[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(off, E, wsum);
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = off[e];
  if (threadIdx.x == 0) { offsets[E] = total; off[E] = total; }
  __syncthreads();
  if (tiles) build_tiles_block(cnt, off, fb, fe, mt, tiles, max_tiles,
                               tile_count, tmp, wsum);
  // this wave's first slot of each expert, then the stable scatter
  volatile int32_t* base = hist[w];
  for (int e = lane; e < E; e += 64) base[e] = base[e] + off[e];
  const uint64_t lt = lanemask_lt();
  const uint64_t gt = ~lt & ~(1ull << lane);
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
#pragma unroll
  for (int it = 0; it < kPerLane; ++it) {
    if (c0 + it * 64 >= c1) break;
    const int i = c0 + it * 64 + lane;
    const int e = idr[it];
    const bool valid = (unsigned)e < (unsigned)E;
    if (i < c1 && !valid) copy_pos[i] = -1;
    // lanes holding the same expert id: intersect one ballot per id bit
    uint64_t m = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = ballot(valid && bit);
      m &= bit ? ones : ~ones;
    }
    if (valid) {
      const int b0 = base[e];
      const int pos = b0 + popc64(m & lt);
      sorted_copy[pos] = i;
      copy_pos[i] = pos;
      if ((m & gt) == 0) base[e] = b0 + popc64(m);
    }
  }
}

// One wave per routed row. bf16 rows move as 16-byte chunks of 8 values.
template <int ACT, bool MX>
__global__ __launch_bounds__(256) void route_gather_kernel(
    const void* __restrict__ x, int H, int k,
    const int32_t* __restrict__ sorted_copy,
    const int32_t* __restrict__ offsets, int fb, int fe,
    void* __restrict__ xp, uint8_t* __restrict__ xs, int nrows) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  // without a permutation row r is token r (rows quantised in place order)
  int t = r;
  if (sorted_copy) {
    const int r0 = offsets[fb];
    if (r >= offsets[fe] - r0) return;
    t = sorted_copy[r0 + r] / k;
  } else if (r >= nrows) {
    return;
  }
  if (ACT == 0) {  // fp32: 8 floats = two 16-byte chunks per step
    const uint4* src = (const uint4*)((const float*)x + (size_t)t * H);
    uint4* dst = (uint4*)((float*)xp + (size_t)r * H);
    for (int c = lane; c < H / 4; c += 64) dst[c] = src[c];
    return;
  }
  const uint4* src = (const uint4*)((const uint16_t*)x + (size_t)t * H);
  if (!MX) {
    uint4* dst = (uint4*)((uint16_t*)xp + (size_t)r * H);
    for (int c = lane; c < H / 8; c += 64) dst[c] = src[c];
    return;
  }
  quant_mx_row_bf16(src, H, (uint8_t*)xp + (size_t)r * H,
                    xs + (size_t)r * (H / 32), lane);
}

hipError_t launch_route_count(const int32_t* ids, int N, int E,
                              int32_t* chunk_counts, hipStream_t s) {
  int nch = route_num_chunks(N);
  if (nch == 0) return hipSuccess;
  hipLaunchKernelGGL(route_count_kernel, dim3((nch + 3) / 4), dim3(256),
                     4 * E * sizeof(int32_t), s, ids, N, E, nch, chunk_counts);
  return hipGetLastError();
}

hipError_t launch_route_scan(int32_t* chunk_counts, int nchunks, int E,
                             int32_t* counts, int32_t* offsets, int fb, int fe,
                             int mt, Tile* tiles, int max_tiles,
                             int32_t* tile_count, hipStream_t s,
                             const uint16_t* qx, int qH, int qrows, int qmode,
                             void* qcodes, void* qscales) {
  RowQuant rq{qx, qH, qrows, qcodes, qscales};
  const int qb = qmode ? (qrows + 15) / 16 : 0;
  const dim3 grid(1 + qb), block(1024);
#define MOE_SCAN(Q_, C_)                                                    \
  hipLaunchKernelGGL((route_scan_kernel<Q_, C_>), grid, block, 0, s,        \
                     chunk_counts, nchunks, E, counts, offsets, fb, fe, mt, \
                     tiles, max_tiles, tile_count, rq)
  if (qmode == 1) MOE_SCAN(1, 0);
  else if (qmode == 2 && qH == 2048) MOE_SCAN(2, 4);
  else if (qmode == 2 && qH == 4096) MOE_SCAN(2, 8);
  else if (qmode == 2) MOE_SCAN(2, 0);
  else MOE_SCAN(0, 0);
#undef MOE_SCAN
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int fb, int fe, int mt,
                              Tile* tiles, int max_tiles, int32_t* tile_count,
                              hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets,
                     fb, fe, mt, tiles, max_tiles, tile_count);
  return hipGetLastError();
}

hipError_t launch_route_scatter(const int32_t* ids, int N, int E,
                                const int32_t* chunk_base,
                                const int32_t* offsets, int32_t* sorted_copy,
                                int32_t* copy_pos, hipStream_t s) {
  int nch = route_num_chunks(N);
  if (nch == 0) return hipSuccess;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((nch + 3) / 4), dim3(256),
                     4 * E * sizeof(int32_t), s, ids, N, E, nch, chunk_base,
                     offsets, sorted_copy, copy_pos);
  return hipGetLastError();
}

bool route_small_ok(int N, int E) { return N <= kSmallMaxN && E <= kSmallMaxE; }

hipError_t launch_route_small(const int32_t* ids, int N, int E,
                              int32_t* counts, int32_t* offsets,
                              int32_t* sorted_copy, int32_t* copy_pos, int fb,
                              int fe, int mt, Tile* tiles, int max_tiles,
                              int32_t* tile_count, hipStream_t s) {
  if (!route_small_ok(N, E)) return hipErrorInvalidValue;
  if (N <= 1024)
    hipLaunchKernelGGL((route_small_kernel<1>), dim3(1), dim3(1024), 0, s, ids,
                       N, E, counts, offsets, sorted_copy, copy_pos, fb, fe,
                       mt, tiles, max_tiles, tile_count);
  else
    hipLaunchKernelGGL((route_small_kernel<4>), dim3(1), dim3(1024), 0, s, ids,
                       N, E, counts, offsets, sorted_copy, copy_pos, fb, fe,
                       mt, tiles, max_tiles, tile_count);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const void* x, int T, int H, uint8_t* xq,
                              uint8_t* xq_scale, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL((route_gather_kernel<1, true>), dim3((T + 3) / 4),
                     dim3(256), 0, s, x, H, 1, nullptr, nullptr, 0, 0, xq,
                     xq_scale, T);
  return hipGetLastError();
}

hipError_t launch_route_gather(const void* x, int act, int mx, int H, int k,
                               const int32_t* sorted_copy,
                               const int32_t* offsets, int fb, int fe,
                               int max_rows, void* x_perm, uint8_t* x_scale,
                               hipStream_t s) {
  if (max_rows == 0 || fe <= fb) return hipSuccess;
  dim3 grid((max_rows + 3) / 4), block(256);
  if (act == 0)
    hipLaunchKernelGGL((route_gather_kernel<0, false>), grid, block, 0, s, x,
                       H, k, sorted_copy, offsets, fb, fe, x_perm, x_scale, 0);
  else if (!mx)
    hipLaunchKernelGGL((route_gather_kernel<1, false>), grid, block, 0, s, x,
                       H, k, sorted_copy, offsets, fb, fe, x_perm, x_scale, 0);
  else
    hipLaunchKernelGGL((route_gather_kernel<1, true>), grid, block, 0, s, x,
                       H, k, sorted_copy, offsets, fb, fe, x_perm, x_scale, 0);
  return hipGetLastError();
}

}  // namespace moe
