// Host-side launchers of the kernels (one per .hip file), used by api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "prefetch.h"

namespace moe {

// Tile of a grouped GEMM: local expert index and first row (relative to the
// expert's first row). Built on the device from the routing offsets.
struct Tile {
  int32_t expert;  // e - fb
  int32_t row0;    // row of x_perm where the tile starts (absolute)
  int32_t rows;    // rows in the tile (<= tile height)
  int32_t first;   // index of the expert's first tile in the list
  int32_t count;   // tiles of the expert
  int32_t pad[3];
};

// Work item L of a tiled grouped GEMM: a (tile, weight slab) pair. The items
// of one expert's tiles are ordered in groups of `sgroup` slabs, tile-major
// inside a group (sgroup >= nslabs: plain tile-major order, every slab of a
// tile before the next tile). Blocks that run together on an XCD take
// consecutive items, so the group size trades weight-slab reuse (a slab's
// reads from HBM) against activation-tile reuse (a tile's rows, gathered
// from x, which the memory-side cache holds).
__device__ __forceinline__ void tile_item(const Tile* __restrict__ tiles, int L,
                                          int nslabs, int sgroup, Tile& tl,
                                          int& slab) {
  const Tile t0 = tiles[L / nslabs];
  if (sgroup >= nslabs) {
    tl = t0;
    slab = L % nslabs;
    return;
  }
  const int nt = t0.count;
  const int i = L - t0.first * nslabs;  // item within the expert
  const int g = i / (sgroup * nt);      // slab group
  const int j = i - g * sgroup * nt;
  const int gg = min(sgroup, nslabs - g * sgroup);
  slab = g * sgroup + j % gg;
  tl = tiles[t0.first + j / gg];
}

hipError_t launch_gate_topk(const float* logits, int T, int E, int k,
                            int32_t* ids, float* w, hipStream_t s);
// The gate fused with the per-token quantisation of x [T, H] bf16 (mx:
// MXFP8 codes + e8m0 scales; else int8 codes + fp32 scales), for E <= 256
// and (MX) H % 32 == 0 or (int8) H = 2048 or 4096 (gate_quant_ok).
bool gate_quant_ok(int E, int H, bool mx);
hipError_t launch_gate_topk_quant(const float* logits, int T, int E, int k,
                                  int32_t* ids, float* w, const uint16_t* x,
                                  int H, bool mx, void* xq, void* xs,
                                  hipStream_t s);

// Routing. chunk_counts has route_num_chunks(N) * E ints.
int route_num_chunks(int N);
hipError_t launch_route_count(const int32_t* ids, int N, int E,
                              int32_t* chunk_counts, hipStream_t s);
// Scans chunk counts (in place, to per-chunk bases), writes counts and
// offsets. When tiles != NULL also builds the GEMM tile list for the FFN
// experts [fb, fe) with tile height mt (tile_count[0] = number of tiles).
// qmode 1 (MXFP8) / 2 (int8): the launch also quantises the qrows bf16 rows
// of qx [qrows, qH] into qcodes / qscales (per token, as the gate-fused
// quantisation does), on blocks beside the scanning one; 0: no quantisation.
hipError_t launch_route_scan(int32_t* chunk_counts, int nchunks, int E,
                             int32_t* counts, int32_t* offsets, int fb, int fe,
                             int mt, Tile* tiles, int max_tiles,
                             int32_t* tile_count, hipStream_t s,
                             const uint16_t* qx = nullptr, int qH = 0,
                             int qrows = 0, int qmode = 0,
                             void* qcodes = nullptr, void* qscales = nullptr);
hipError_t launch_build_tiles(const int32_t* offsets, int fb, int fe, int mt,
                              Tile* tiles, int max_tiles, int32_t* tile_count,
                              hipStream_t s);
hipError_t launch_route_scatter(const int32_t* ids, int N, int E,
                                const int32_t* chunk_base,
                                const int32_t* offsets, int32_t* sorted_copy,
                                int32_t* copy_pos, hipStream_t s);
// Single-block routing (count + scan + tile list + scatter) for N <= 4096
// copies and E <= 1024.
bool route_small_ok(int N, int E);
hipError_t launch_route_small(const int32_t* ids, int N, int E,
                              int32_t* counts, int32_t* offsets,
                              int32_t* sorted_copy, int32_t* copy_pos, int fb,
                              int fe, int mt, Tile* tiles, int max_tiles,
                              int32_t* tile_count, hipStream_t s);
// act: 0 f32, 1 bf16. mx: quantise rows to MXFP8 (bf16 input only).
// MXFP8 codes and e8m0 scales of the T rows of x (bf16), in token order.
hipError_t launch_quantize_mx(const void* x, int T, int H, uint8_t* xq,
                              uint8_t* xq_scale, hipStream_t s);
hipError_t launch_route_gather(const void* x, int act, int mx, int H, int k,
                               const int32_t* sorted_copy,
                               const int32_t* offsets, int fb, int fe,
                               int max_rows, void* x_perm, uint8_t* x_scale,
                               hipStream_t s);

// Compute units of the current device (256 on MI355X if the query fails).
int device_cus();
// Waves per block that split K in the weight-streaming kernels, for a grid
// of `blocks` blocks and `steps` K steps of 16 KB of weights per wave.
int stream_ksplit(long long blocks, int steps, int rg);
// Column slabs (grid x) and K split of the bf16 / int8 weight-streaming
// launches (the launchers use these; the weight prefetch follows them).
int stream_bf16_slabs(bool glu, int Nout);
int stream_bf16_ksplit(bool glu, int max_tiles, int K, int Nout, int rg);
int stream_i8_slabs(bool glu, int Nout);
int stream_i8_ksplit(bool glu, int max_tiles, int K, int Nout, int rg);

// Grouped GEMMs. glu: GEMM1 with SwiGLU epilogue (N = 2*I weight columns,
// I outputs), else GEMM2 (N outputs). Tiles come from the tile list.
// bf16 activations / bf16 weights [E_loc, K, N], row-major or (pk) slab-
// packed as launch_pack_bf16_weights writes them (then K % 32 == 0 and
// N % 256 == 0). When gidx is non-NULL the activation row of tile row i is
// row gidx[gbase[0] + i] / gk of `a` (the gather from x fused into the A
// loads); otherwise row i of `a`.
hipError_t launch_gemm_bf16_stream(bool glu, int rg, const Tile* tiles,
                                   const int32_t* tile_count, int max_tiles,
                                   const uint16_t* a, const uint16_t* w,
                                   uint16_t* out, int K, int Nw, int Nout,
                                   const int32_t* gidx, const int32_t* gbase,
                                   int gk, hipStream_t s, bool pk = false);
// Same operands, LDS-tiled MFMA tiles of mt = 128 or 256 rows (the tile
// list's height). With gidx, `a` must span less than 4 GB.
hipError_t launch_gemm_bf16_tiled(bool glu, int mt, const Tile* tiles,
                                  const int32_t* tile_count, int max_tiles,
                                  const uint16_t* a, const uint16_t* w,
                                  uint16_t* out, int K, int Nw, int Nout,
                                  const int32_t* gidx, const int32_t* gbase,
                                  int gk, hipStream_t s, bool pk = false);
// W8A8: int8 activations [rows, K] with one fp32 scale per row (a_scale,
// indexed like the rows of a, through gidx when it is non-NULL), int8
// weights [E_loc, N, K] with one fp32 scale per output channel
// (w_scale [E_loc, N]); int32 accumulation. glu: fp32 h, else bf16 y.
// LDS-tiled tiles of mt = 128 or 256 rows, K % 64 == 0.
hipError_t launch_gemm_i8_tiled(bool glu, int mt, const Tile* tiles,
                                const int32_t* tile_count, int max_tiles,
                                const int8_t* a, const float* a_scale,
                                const int8_t* w, const float* w_scale,
                                void* out, int K, int Nw, int Nout,
                                const int32_t* gidx, const int32_t* gbase,
                                int gk, hipStream_t s);
// Same operands, weight-streaming tiles of 16 rows (rg = 1; mt = 16),
// K % 128 == 0.
hipError_t launch_gemm_i8_stream(bool glu, int rg, const Tile* tiles,
                                 const int32_t* tile_count, int max_tiles,
                                 const int8_t* a, const float* a_scale,
                                 const int8_t* w, const float* w_scale,
                                 void* out, int K, int Nw, int Nout,
                                 const int32_t* gidx, const int32_t* gbase,
                                 int gk, hipStream_t s);
// Dynamic per-row int8 quantisation (bf16 or fp32 rows of K, K % 8 == 0):
// codes [rows, K] and fp32 scales [rows]. offs == NULL: nrows rows, row r
// from source row r. Else the R = offs[fe] - offs[fb] (<= nrows) rows of the
// copies of experts [fb, fe), row r from source row gidx[offs[fb] + r] / gk
// (gidx != NULL) or r.
// Packed weights (fragments of 16 columns x 64 bytes, [E][Kb/64][N/16]) from
// byte matrices [E, N, Kb] (int8 codes, or two e2m1 codes per byte).
hipError_t launch_pack_weights(int E, int N, int Kb, const uint8_t* src,
                               uint8_t* dst, hipStream_t s);
// Slab-packed bf16 weights (pack_bf16.hip) from row-major [E, K, N]:
// [E][N/256][K/32][32][256]; glu pairs gate column 128 j + c with up column
// N/2 + 128 j + c in slab j. K % 32 == 0, N % 256 == 0.
hipError_t launch_pack_bf16_weights(int E, int K, int N, bool glu,
                                    const uint16_t* src, uint16_t* dst,
                                    hipStream_t s);
// MXFP4 (e2m1 + e8m0 per 32 along K) of bf16 weights [E, K, N] (N
// contiguous): codes [E, N, K/2] (low nibble = even k), scales [E, N, K/32].
// K % 32 == 0.
hipError_t launch_quant_mxfp4_weights(int E, int K, int N, const uint16_t* w,
                                      uint8_t* codes, uint8_t* scales,
                                      hipStream_t s);
hipError_t launch_quant_i8_rows(bool f32, const void* src, int K, int nrows,
                                const int32_t* gidx, const int32_t* offs,
                                int fb, int fe, int gk, int8_t* codes,
                                float* scales, hipStream_t s);

// fp32 activations / fp32 weights [E_loc, K, N], VALU.
hipError_t launch_gemm_f32(bool glu, const Tile* tiles,
                           const int32_t* tile_count, int max_tiles,
                           const float* a, const float* w, float* out, int K,
                           int Nw, int Nout, hipStream_t s);
// MXFP8 activations [rows, K] + e8m0 [rows, K/32]; MXFP4 weights
// [E_loc, N, K/2] + e8m0 [E_loc, N, K/32]. glu: output MXFP8 h (+ scales);
// else bf16 y. 128-row LDS-tiled scaled-MFMA tiles (tile list mt=128).
// With gidx non-NULL, A rows (and their scales) are read from the per-token
// codes: row of sorted copy i = gidx[gbase[0] + i] / gk (offsets < 2^31).
hipError_t launch_gemm_mx_tiled(bool glu, const Tile* tiles,
                                const int32_t* tile_count, int max_tiles,
                                const uint8_t* a, const uint8_t* a_scale,
                                const uint8_t* w, const uint8_t* w_scale,
                                void* out, uint8_t* out_scale, int K, int Nw,
                                int Nout, const int32_t* gidx,
                                const int32_t* gbase, int gk, hipStream_t s);

// The weight prefetch of pf (prefetch.h) on `blocks` blocks of its own.
hipError_t launch_prefetch(const Prefetch& pf, int blocks, hipStream_t s);

// Residual add + RMSNorm; mx = 0: fp32 and/or bf16 outputs, mx = 1: MXFP8
// codes + e8m0 scales. H % 32 == 0, H <= 8192; residual / outputs may be null.
hipError_t launch_add_rms_norm(int mx, const uint16_t* x, const uint16_t* r,
                               const uint16_t* w, float eps, int T, int H,
                               float* y32, uint16_t* y16, uint8_t* codes,
                               uint8_t* scales, uint16_t* res_out,
                               hipStream_t s);

// fp32 router logits [T, E] = y [T, H] @ w [E, H]^T; H % 16 == 0,
// E % 32 == 0.
hipError_t launch_router_logits(const float* y, const float* w, float* out,
                                int T, int H, int E, hipStream_t s);

hipError_t launch_finalize(const int32_t* ids, const float* w,
                           const int32_t* copy_pos, const int32_t* offsets,
                           int fb, int n_ffn, int lb, int le, const void* y,
                           const void* x, const void* residual, void* out,
                           int act, int T, int H, int k, hipStream_t s);

}  // namespace moe
