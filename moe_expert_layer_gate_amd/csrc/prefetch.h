// Weight prefetch: reads the leading bytes of the experts' weight matrices so
// that the lines sit in the caches (the 256 MB memory-side cache in front of
// HBM, and the reading XCD's L2) when the grouped GEMM asks for them.
//
// [P2] "LongCat-Flash inference on Atlas A3 clusters", section 权重预取: a
// memory-bound matmul's weights can be fetched ahead while an earlier,
// latency-bound operator runs, up to about the HBM bandwidth times that
// operator's duration; the AFD section applies the same to the FFN side's
// grouped matmuls in the gaps of communication.
//
// What is read: for each of the first `nexp` selected experts (every local
// expert, or only those some copy routes to, in expert order) and each of
// its `nslab` weight regions (1 for row-major weights; the 256-column slabs
// of slab-packed bf16 weights, `slab_bytes` apart), bytes [skip, skip +
// lead) of the head of each of the region's `nseg` K segments, segment s
// starting at K step s * nsteps / nseg (steps of `step_bytes` bytes: the
// consuming GEMM's K steps and K split; its weights are K-major within a
// region, so a head is contiguous). Those are the bytes the streaming GEMM's
// waves read first -- the only ones still in the cache when asked for, since
// the rest of the weights stream through it meanwhile -- and `nexp` covers
// the experts of its first round of blocks.
// Nothing is written: the loaded words are folded into one value per lane
// that is stored only when `sink` is non-null (never, in the library's calls;
// the conditional store keeps the loads from being optimised away).
#pragma once
#include "common.h"

namespace moe {

struct Prefetch {
  const char* w;         // expert 0's weights; expert i at w + i * ebytes
  long long ebytes;      // bytes per expert
  long long step_bytes;  // bytes per K step of the consuming GEMM
  long long slab_bytes;  // bytes per region (slab) of an expert
  int nslab;             // regions per expert
  int nsteps;            // K steps per expert
  int nseg;              // K split of the consuming GEMM
  int skip;              // bytes skipped at the head of each segment
  int lead;              // bytes read after them (a multiple of 16)
  int nexp;              // selected experts covered, in expert order
  int El;                // local experts (<= 2048)
  const int32_t* ids;    // routed expert ids [nids] (NULL: every expert)
  int nids;
  int fb;                // id of local expert 0
  uint32_t* sink;        // NULL (see above)
};

// LDS words prefetch_block needs (up to 2048 local experts).
constexpr int kPrefetchLdsWords = 64 + 65 + 1024;

// Part `part` of `nparts` of the prefetch described by `d`, run by a whole
// block of `nthr` threads (a multiple of 64, at most 1024); `lds` holds
// kPrefetchLdsWords words of the block's LDS. El <= 2048.
MOE_DEV void prefetch_block(const Prefetch& d, int part, int nparts,
                            uint32_t* lds, int nthr) {
  const int tid = threadIdx.x;
  const int nw = (d.El + 31) / 32;
  uint32_t* bits = lds;                       // selected experts, 1 bit each
  uint32_t* wrank = lds + 64;                 // selected experts before word i
  uint16_t* list = (uint16_t*)(lds + 129);    // the selected experts in order
  for (int i = tid; i < nw; i += nthr) {
    uint32_t b = d.ids ? 0u : ~0u;
    if (i == nw - 1 && (d.El & 31)) b &= (1u << (d.El & 31)) - 1u;
    bits[i] = b;
  }
  __syncthreads();
  if (d.ids) {
    for (int i = tid; i < d.nids; i += nthr) {
      const int e = d.ids[i] - d.fb;
      if ((unsigned)e < (unsigned)d.El) atomicOr(&bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
  }
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < nw; ++i) {
      wrank[i] = r;
      r += __popc(bits[i]);
    }
    wrank[nw] = r;
  }
  __syncthreads();
  for (int i = tid; i < nw; i += nthr) {
    uint32_t b = bits[i];
    for (uint32_t r = wrank[i]; b; ++r, b &= b - 1u)
      list[r] = (uint16_t)(32 * i + __ffs(b) - 1);
  }
  __syncthreads();
  const int nsel = min((int)wrank[nw], d.nexp);
  if (d.lead < 16 || nsel <= 0 || d.nseg <= 0 || d.nslab <= 0)
    return;  // uniform over the block
  // work in chunks of 64 KB (the last one of a segment head may be shorter):
  // chunk c is chunk c % cps of the read part of segment c / cps, segment
  // r = (j * nslab + sl) * nseg + sg of region sl of the j-th selected
  // expert; lanes take consecutive 16-byte pieces of a chunk
  constexpr int kChunkBytes = 65536;
  const int cps = (d.lead + kChunkBytes - 1) / kChunkBytes;
  const int per_exp = d.nslab * d.nseg;
  const int nchunks = nsel * per_exp * cps;
  uint32_t fold = 0;
  for (int c = part; c < nchunks; c += nparts) {
    const int r = c / cps;
    const int j = r / per_exp;
    const int sl = (r - j * per_exp) / d.nseg;
    const int sg = r - j * per_exp - sl * d.nseg;
    const int c0 = (c - r * cps) * kChunkBytes;
    const int len = min(kChunkBytes, d.lead - c0);
    const char* base = d.w + list[j] * d.ebytes + sl * d.slab_bytes +
                       (long long)(sg * d.nsteps / d.nseg) * d.step_bytes +
                       d.skip + c0;
    constexpr int U = 4;  // 16-byte loads in flight per lane
    for (int o = 16 * tid; o < len; o += 16 * U * nthr) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ou = min(o + 16 * u * nthr, len - 16);
        v[u] = *(const uint4*)(base + ou);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (d.sink) d.sink[blockIdx.x * nthr + tid] = fold;
}

}  // namespace moe
