// C ABI of the MoE expert layer: argument checks, workspace layout and the
// launch sequence. No allocation and no host synchronisation; the only global
// state is the per-device address of moe_layer_noalloc's static scratch.
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "launch.h"

// Workspace of moe_layer_noalloc, for callers that cannot allocate: one copy
// on every GPU the library runs on, held until the process ends. Host code
// never names it directly (on the host the name is only a stand-in); it uses
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::Tile;

constexpr int kMaxE = 2048;
constexpr int kMaxK = 64;
constexpr int kMaxNormH = 8192;  // fused norm: 16 chunks of 8 columns per lane

struct Prob {
  int T, H, I, nffn, nzero, k, lb, le, act, wt, actq;
  int E, fb, fe, El;
  long long N;  // T * k copies
  bool mx;      // MXFP8 activations x MXFP4 weights
  bool i8;      // W8A8: int8 activations and weights, fp32 scales
  bool pk;      // bf16 weights slab-packed (moe_pack_bf16_weights)
};

moe_status check(const moe_problem* p, Prob* q) {
  if (!p) return MOE_ERR_INVALID_ARG;
  Prob r{};
  r.T = p->T; r.H = p->H; r.I = p->I; r.nffn = p->n_ffn; r.nzero = p->n_zero;
  r.k = p->top_k; r.lb = p->local_begin; r.le = p->local_end;
  r.act = p->act; r.wt = p->wt; r.actq = p->act_q;
  const int layout = p->wt_layout;
  if (r.T < 0 || r.H <= 0 || r.I <= 0 || r.nffn < 0 || r.nzero < 0)
    return MOE_ERR_INVALID_ARG;
  r.E = r.nffn + r.nzero;
  if (r.E < 1 || r.k < 1 || r.k > r.E) return MOE_ERR_INVALID_ARG;
  if (r.lb < 0 || r.lb >= r.le || r.le > r.E) return MOE_ERR_INVALID_ARG;
  if (r.E > kMaxE || r.k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (r.H % 32 || r.I % 32) return MOE_ERR_UNSUPPORTED;
  r.N = (long long)r.T * r.k;
  if (r.N >= (1LL << 31) || (long long)r.N * r.H >= (1LL << 40))
    return MOE_ERR_UNSUPPORTED;
  const bool f32 = r.act == MOE_F32 && r.wt == MOE_F32 && r.actq == MOE_F32;
  const bool bf16 = r.act == MOE_BF16 && r.wt == MOE_BF16 && r.actq == MOE_BF16;
  r.mx = r.act == MOE_BF16 && r.wt == MOE_MXFP4_E2M1 && r.actq == MOE_MXFP8_E4M3;
  r.i8 = r.act == MOE_BF16 && r.wt == MOE_INT8 && r.actq == MOE_INT8;
  if (!f32 && !bf16 && !r.mx && !r.i8) return MOE_ERR_UNSUPPORTED;
  // the quantised GEMMs read packed weights only, the fp32 one row-major
  // ones, the bf16 ones either (packed: whole 256-column slabs)
  if (layout != MOE_LAYOUT_ROWMAJOR && layout != MOE_LAYOUT_PACKED)
    return MOE_ERR_UNSUPPORTED;
  const bool packed = layout == MOE_LAYOUT_PACKED;
  if ((r.mx || r.i8) ? !packed : (f32 && packed)) return MOE_ERR_UNSUPPORTED;
  r.pk = bf16 && packed;
  if (r.pk && (r.I % 128 || r.H % 256)) return MOE_ERR_UNSUPPORTED;
  if (r.mx && (r.H % 128 || r.I % 128)) return MOE_ERR_UNSUPPORTED;
  // int8: K steps of 128; int32 sums of 127 * 127 * K products stay exact;
  // weight offsets (2I * H bytes per expert) fit 32 bits
  if (r.i8 && (r.H % 128 || r.I % 128 || 2LL * r.I * r.H >= (1LL << 31)))
    return MOE_ERR_UNSUPPORTED;
  r.fb = r.lb < r.nffn ? r.lb : r.nffn;
  r.fe = r.le < r.nffn ? r.le : r.nffn;
  r.El = r.fe - r.fb;
  *q = r;
  return MOE_OK;
}

size_t act_bytes(const Prob& q) { return q.act == MOE_F32 ? 4 : 2; }

// Tile height of the grouped GEMM chosen for the problem, from the expected
// rows per expert: weight-streaming tiles of 16 or 32 rows for decode-size
// batches, LDS-tiled MFMA tiles of 128 rows beyond them and of 256 rows
// (bf16 and int8) once experts average 512 rows or more. (256-row tiles are
// 6-11 % faster when most rows sit in full tiles, but slower than 128-row
// ones at 256 rows per expert under skewed routing, where the many partial
// tiles leave half of their waves without rows.) The streaming kernels read
// an expert's weights once per tile they run, the tiled ones once per 128
// rows, so the tiled kernels take over from a few rows per expert on: from
// 10 for int8 and 20 for bf16 (measured with both kinds streaming weights
// that only they read nontemporally: int8 on the 2048 x 768 expert shape
// 123.5 us streaming vs 130.6 us tiled at 8 rows, 134.8 vs 132.9 us at 10,
// 141.1 vs 134.3 us at 12; bf16 on the same shape is 2-5 % faster tiled
// from 4 rows on (201.5 vs 197.4 us at 4, 210.4 vs 200.9 us at 8), but on
// 6144 x 2048 experts streaming stays ahead (6090 vs 6340 us at 16 rows),
// so bf16 switches at 20). W4A8 always runs the tiled scaled-MFMA
// kernels, which beat weight streaming on 4096 x 1536 experts from a single
// token on (1 to 128 tokens of a 32-expert share: 15-26 % faster). Below
// the switch bf16 streams 32-row tiles from 8 rows per expert (3-6 % faster
// than 16-row ones at 8-12 rows), int8 16-row tiles throughout (32-row ones
// were 8-12 % slower at 8-10 rows).
// Expected rows per expert from which the bf16 / int8 tiled GEMMs take over
// from weight streaming, and from which they take 256-row tiles.
#ifndef MOE_TILED_FROM_BF16
#define MOE_TILED_FROM_BF16 20
#endif
#ifndef MOE_TILED_FROM_I8
#define MOE_TILED_FROM_I8 10
#endif
#ifndef MOE_TILE256_AVG
#define MOE_TILE256_AVG 512
#endif

int tile_rows(const Prob& q) {
  if (q.act == MOE_F32) return 32;
  if (q.mx) return 128;
  const long long avg = q.E ? q.N / q.E : 0;  // expected rows per expert
  if (avg >= MOE_TILE256_AVG) return 256;
  if (avg >= (q.i8 ? MOE_TILED_FROM_I8 : MOE_TILED_FROM_BF16)) return 128;
  return q.i8 || avg < 8 ? 16 : 32;
}

// moe_layer fuses the gather into GEMM1's activation loads for bf16 (the
// tiled kernel addresses x with 32-bit offsets, so x must span < 4 GB).

bool fused_gather(const Prob& q) {
  return q.act == MOE_BF16 && !q.mx && !q.i8 &&
         (unsigned long long)q.T * q.H * 2 < (1ull << 32);
}

long long max_tiles(const Prob& q, int mt) {
  if (q.El == 0 || q.N == 0) return 0;
  long long ne = q.El < q.N ? q.El : q.N;
  return ne + q.N / mt + 1;
}

// ---------------------------------------------------------------- prefetch

// Blocks of moe_prefetch_weights (256 threads each).
constexpr int kPrefetchBlocks = 1024;

// How a grouped GEMM reads one expert's weights: bytes per expert, its
// K-major regions (one for bf16 [K, N] and for packed int8 / e2m1 in 64-byte
// K chunks of all N columns; the 256-column slabs of slab-packed bf16), bytes
// per K step of a region, steps, the K split its waves start at (streaming
// kernels), and how many tiles its first round of blocks holds (the experts
// whose heads are read first).
struct Geom {
  long long ebytes = 0, step = 0, slab_bytes = 0;
  int nsteps = 0, nseg = 0, nslab = 1, round_tiles = 0;
};

Geom gemm_geom(const Prob& q, int mt, bool up) {
  Geom g;
  const int mtl = (int)max_tiles(q, mt);
  if (q.El == 0 || mtl == 0 || q.act == MOE_F32) return g;
  const int K = up ? q.H : q.I, N = up ? 2 * q.I : q.H, Nout = up ? q.I : q.H;
  const int cus = moe::device_cus();
  if (q.mx || mt >= 128) {
    // tiled kernels: 64 bytes of K of every column per step; every (tile,
    // slab) item walks K from its head, items of every expert run at once
    const int eb2 = q.mx ? 1 : (q.i8 ? 2 : 4);  // element bytes x 2
    g.ebytes = (long long)K * N * eb2 / 2;
    g.step = 64LL * N;
    g.nsteps = (int)(g.ebytes / g.step);
    g.nseg = 1;
    g.round_tiles = q.El;
  } else if (q.i8) {
    g.ebytes = (long long)K * N;
    g.step = 128LL * N;
    g.nsteps = K / 128;
    g.nseg = moe::stream_i8_ksplit(up, mtl, K, Nout, mt / 16);
    g.round_tiles = cus * (8 / g.nseg) / moe::stream_i8_slabs(up, Nout);
  } else {
    g.ebytes = (long long)K * N * 2;
    g.step = 64LL * N;
    g.nsteps = K / 32;
    g.nseg = moe::stream_bf16_ksplit(up, mtl, K, Nout, mt / 16);
    g.round_tiles = cus * (8 / g.nseg) / moe::stream_bf16_slabs(up, Nout);
  }
  if (q.pk) {
    // slab-packed bf16: N / 256 slabs of K / 32 steps of 16 KB each
    g.nslab = N / 256;
    g.step = 16384;
    g.slab_bytes = (long long)K * 512;
  }
  return g;
}

// Prefetch of `budget` bytes: bytes [skip, skip + lead) of each K segment of
// the first `nexp` selected experts (all local experts, or those `ids`
// routes to), lead = budget / (nexp * segments), within the segments.
moe::Prefetch make_prefetch(const Geom& g, const void* w, const Prob& q,
                            const int32_t* ids, int nids, long long skip,
                            long long budget, int nexp) {
  moe::Prefetch pf{};
  if (g.nseg <= 0 || nexp <= 0 || budget < 16 || !w) return pf;
  const long long segmin = (long long)(g.nsteps / g.nseg) * g.step;
  long long lead = budget / ((long long)nexp * g.nseg * g.nslab);
  if (lead > segmin - skip) lead = segmin - skip;
  lead &= ~15LL;
  if (lead < 16) return pf;
  pf.w = (const char*)w;
  pf.ebytes = g.ebytes;
  pf.step_bytes = g.step;
  pf.slab_bytes = g.slab_bytes;
  pf.nslab = g.nslab;
  pf.nsteps = g.nsteps;
  pf.nseg = g.nseg;
  pf.skip = (int)skip;
  pf.lead = (int)lead;
  pf.nexp = nexp;
  pf.El = q.El;
  pf.ids = ids;
  pf.nids = nids;
  pf.fb = q.fb;
  pf.sink = nullptr;
  return pf;
}

struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

// Every tensor pointer must be 16-byte aligned (the kernels move 16 bytes
// per lane and copy straight into LDS); NULL passes.
bool aligned16() { return true; }
template <class P, class... R>
bool aligned16(P p, R... rest) {
  return ((uintptr_t)(const void*)p & 15u) == 0 && aligned16(rest...);
}
bool ws_aligned(const void* w) { return ((uintptr_t)w & 255u) == 0; }

moe_status hip_status(hipError_t e) {
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

#define MOE_TRY(expr)                                 \
  do {                                                \
    hipError_t _e = (expr);                           \
    if (_e != hipSuccess) return MOE_ERR_HIP;         \
  } while (0)

// ---------------------------------------------------------------- FFN halves

struct FfnWs {
  Tile* tiles;
  int32_t* tile_count;
};

FfnWs carve_ffn_ws(Carve& c, const Prob& q, int mt) {
  FfnWs w;
  w.tiles = c.take<Tile>((size_t)max_tiles(q, mt) + 1);
  w.tile_count = c.take<int32_t>(1);
  return w;
}

// gidx/gbase: fused gather (bf16 only) -- activation row of sorted copy i is
// row gidx[gbase[0] + i] / top_k of xp (= x); NULL: xp holds permuted rows.
// W8A8: GEMM1 writes h in fp32 (h), quantised by run_quant_h afterwards.
moe_status run_up(const Prob& q, int mt, const Tile* tiles,
                  const int32_t* tile_count, const void* xp, const void* xs,
                  const void* w13, const void* w13s, void* h, void* hs,
                  hipStream_t s, const int32_t* gidx = nullptr,
                  const int32_t* gbase = nullptr) {
  const int mtl = (int)max_tiles(q, mt);
  if (mtl == 0) return MOE_OK;
  if (q.i8 && mt >= 128)
    MOE_TRY(moe::launch_gemm_i8_tiled(true, mt, tiles, tile_count, mtl,
                                      (const int8_t*)xp, (const float*)xs,
                                      (const int8_t*)w13, (const float*)w13s,
                                      h, q.H, 2 * q.I, q.I, gidx, gbase, q.k,
                                      s));
  else if (q.i8)
    MOE_TRY(moe::launch_gemm_i8_stream(true, mt / 16, tiles, tile_count, mtl,
                                       (const int8_t*)xp, (const float*)xs,
                                       (const int8_t*)w13, (const float*)w13s,
                                       h, q.H, 2 * q.I, q.I, gidx, gbase, q.k,
                                       s));
  else if (q.act == MOE_F32)
    MOE_TRY(moe::launch_gemm_f32(true, tiles, tile_count, mtl, (const float*)xp,
                                 (const float*)w13, (float*)h, q.H, 2 * q.I,
                                 q.I, s));
  else if (q.mx)
    MOE_TRY(moe::launch_gemm_mx_tiled(true, tiles, tile_count, mtl,
                                      (const uint8_t*)xp, (const uint8_t*)xs,
                                      (const uint8_t*)w13,
                                      (const uint8_t*)w13s, h, (uint8_t*)hs,
                                      q.H, 2 * q.I, q.I, gidx, gbase, q.k, s));
  else if (mt >= 128)
    MOE_TRY(moe::launch_gemm_bf16_tiled(
        true, mt, tiles, tile_count, mtl, (const uint16_t*)xp,
        (const uint16_t*)w13, (uint16_t*)h, q.H, 2 * q.I, q.I, gidx, gbase,
        q.k, s, q.pk));
  else
    MOE_TRY(moe::launch_gemm_bf16_stream(
        true, mt / 16, tiles, tile_count, mtl, (const uint16_t*)xp,
        (const uint16_t*)w13, (uint16_t*)h, q.H, 2 * q.I, q.I, gidx, gbase,
        q.k, s, q.pk));
  return MOE_OK;
}

// W8A8: the R rows of GEMM1's fp32 h -> int8 codes hq + fp32 row scales hs.
moe_status run_quant_h(const Prob& q, const float* h32, const int32_t* offsets,
                       void* hq, void* hs, hipStream_t s) {
  MOE_TRY(moe::launch_quant_i8_rows(true, h32, q.I, (int)q.N, nullptr, offsets,
                                    q.fb, q.fe, 1, (int8_t*)hq, (float*)hs, s));
  return MOE_OK;
}

moe_status run_down(const Prob& q, int mt, const Tile* tiles,
                    const int32_t* tile_count, const void* h,
                    const void* hs, const void* w2, const void* w2s,
                    void* y, hipStream_t s) {
  const int mtl = (int)max_tiles(q, mt);
  if (mtl == 0) return MOE_OK;
  if (q.i8 && mt >= 128)
    MOE_TRY(moe::launch_gemm_i8_tiled(false, mt, tiles, tile_count, mtl,
                                      (const int8_t*)h, (const float*)hs,
                                      (const int8_t*)w2, (const float*)w2s, y,
                                      q.I, q.H, q.H, nullptr, nullptr, q.k, s));
  else if (q.i8)
    MOE_TRY(moe::launch_gemm_i8_stream(false, mt / 16, tiles, tile_count, mtl,
                                       (const int8_t*)h, (const float*)hs,
                                       (const int8_t*)w2, (const float*)w2s, y,
                                       q.I, q.H, q.H, nullptr, nullptr, q.k,
                                       s));
  else if (q.act == MOE_F32)
    MOE_TRY(moe::launch_gemm_f32(false, tiles, tile_count, mtl,
                                 (const float*)h, (const float*)w2, (float*)y,
                                 q.I, q.H, q.H, s));
  else if (q.mx)
    MOE_TRY(moe::launch_gemm_mx_tiled(false, tiles, tile_count, mtl,
                                      (const uint8_t*)h, (const uint8_t*)hs,
                                      (const uint8_t*)w2, (const uint8_t*)w2s,
                                      y, nullptr, q.I, q.H, q.H, nullptr,
                                      nullptr, q.k, s));
  else if (mt >= 128)
    MOE_TRY(moe::launch_gemm_bf16_tiled(
        false, mt, tiles, tile_count, mtl, (const uint16_t*)h,
        (const uint16_t*)w2, (uint16_t*)y, q.I, q.H, q.H, nullptr, nullptr,
        q.k, s, q.pk));
  else
    MOE_TRY(moe::launch_gemm_bf16_stream(
        false, mt / 16, tiles, tile_count, mtl, (const uint16_t*)h,
        (const uint16_t*)w2, (uint16_t*)y, q.I, q.H, q.H, nullptr, nullptr,
        q.k, s, q.pk));
  return MOE_OK;
}

moe_status check_weights(const Prob& q, const void* w13, const void* w13s,
                         const void* w2, const void* w2s, bool need13,
                         bool need2) {
  if (q.El == 0) return MOE_OK;  // no FFN expert in range: weights unused
  if ((need13 && !w13) || (need2 && !w2)) return MOE_ERR_INVALID_ARG;
  if (q.mx || q.i8) {
    if ((need13 && !w13s) || (need2 && !w2s)) return MOE_ERR_INVALID_ARG;
  } else if (w13s || w2s) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

// The current device's copy of `scratch`: looked up once per device (with that
// device current) and kept.
moe_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside library limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch failed";
  }
  return "unknown moe_status";
}

int32_t moe_abi_version(void) { return 200; }

moe_status moe_gate_topk(const moe_problem* p, const float* logits,
                         int32_t* topk_ids, float* topk_weight, void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (q.T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weight) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits, topk_ids, topk_weight)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_gate_topk(logits, q.T, q.E, q.k, topk_ids,
                                          topk_weight, (hipStream_t)stream));
}

moe_status moe_init_routing(const moe_problem* p, const int32_t* topk_ids,
                            const void* x, int32_t* tokens_per_expert,
                            int32_t* offsets, int32_t* sorted_copy,
                            int32_t* copy_pos, void* x_perm,
                            void* x_perm_scale, void* workspace,
                            size_t* workspace_bytes, void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (!workspace_bytes) return MOE_ERR_INVALID_ARG;
  const int nch = moe::route_num_chunks((int)q.N);
  Carve c(workspace);
  int32_t* cc = c.take<int32_t>((size_t)nch * q.E + 1);
  if (!workspace) { *workspace_bytes = c.off; return MOE_OK; }
  if (*workspace_bytes < c.off) return MOE_ERR_WORKSPACE;
  if (!tokens_per_expert || !offsets) return MOE_ERR_INVALID_ARG;
  if (q.N > 0 && (!topk_ids || !sorted_copy || !copy_pos)) return MOE_ERR_INVALID_ARG;
  if (q.El > 0 && q.N > 0 && (!x || !x_perm)) return MOE_ERR_INVALID_ARG;
  if ((q.mx || q.i8) ? (q.El > 0 && q.N > 0 && !x_perm_scale)
                     : (x_perm_scale != nullptr))
    return MOE_ERR_INVALID_ARG;
  if (!ws_aligned(workspace) ||
      !aligned16(topk_ids, x, tokens_per_expert, offsets, sorted_copy,
                 copy_pos, x_perm, x_perm_scale))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (moe::route_small_ok((int)q.N, q.E)) {
    MOE_TRY(moe::launch_route_small(topk_ids, (int)q.N, q.E,
                                    tokens_per_expert, offsets, sorted_copy,
                                    copy_pos, q.fb, q.fe, 0, nullptr, 0,
                                    nullptr, s));
  } else {
    if (q.N > 0) MOE_TRY(moe::launch_route_count(topk_ids, (int)q.N, q.E, cc, s));
    MOE_TRY(moe::launch_route_scan(cc, nch, q.E, tokens_per_expert, offsets,
                                   q.fb, q.fe, 0, nullptr, 0, nullptr, s));
    if (q.N > 0)
      MOE_TRY(moe::launch_route_scatter(topk_ids, (int)q.N, q.E, cc, offsets,
                                        sorted_copy, copy_pos, s));
  }
  if (q.N > 0 && q.i8) {
    MOE_TRY(moe::launch_quant_i8_rows(false, x, q.H, (int)q.N, sorted_copy,
                                      offsets, q.fb, q.fe, q.k,
                                      (int8_t*)x_perm, (float*)x_perm_scale,
                                      s));
  } else if (q.N > 0) {
    MOE_TRY(moe::launch_route_gather(x, q.act == MOE_F32 ? 0 : 1, q.mx ? 1 : 0,
                                     q.H, q.k, sorted_copy, offsets, q.fb,
                                     q.fe, (int)q.N, x_perm,
                                     (uint8_t*)x_perm_scale, s));
  }
  return MOE_OK;
}

moe_status moe_ffn_up(const moe_problem* p, const int32_t* offsets,
                      const void* x_perm, const void* x_perm_scale,
                      const void* w13, const void* w13_scale, void* h,
                      void* h_scale, void* workspace,
                      size_t* workspace_bytes, void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (!workspace_bytes) return MOE_ERR_INVALID_ARG;
  const int mt = tile_rows(q);
  Carve c(workspace);
  FfnWs fw = carve_ffn_ws(c, q, mt);
  float* h32 = q.i8 ? c.take<float>((size_t)q.N * q.I) : nullptr;
  if (!workspace) { *workspace_bytes = c.off; return MOE_OK; }
  if (*workspace_bytes < c.off) return MOE_ERR_WORKSPACE;
  if ((st = check_weights(q, w13, w13_scale, nullptr, nullptr, true, false)) != MOE_OK)
    return st;
  if (q.El == 0 || q.N == 0) return MOE_OK;
  if (!offsets || !x_perm || !h) return MOE_ERR_INVALID_ARG;
  if ((q.mx || q.i8) ? (!x_perm_scale || !h_scale) : (x_perm_scale || h_scale))
    return MOE_ERR_INVALID_ARG;
  if (!ws_aligned(workspace) ||
      !aligned16(offsets, x_perm, x_perm_scale, w13, w13_scale, h, h_scale))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(moe::launch_build_tiles(offsets, q.fb, q.fe, mt, fw.tiles,
                                  (int)max_tiles(q, mt), fw.tile_count, s));
  if (q.i8) {
    st = run_up(q, mt, fw.tiles, fw.tile_count, x_perm, x_perm_scale, w13,
                w13_scale, h32, nullptr, s);
    if (st != MOE_OK) return st;
    return run_quant_h(q, h32, offsets, h, h_scale, s);
  }
  return run_up(q, mt, fw.tiles, fw.tile_count, x_perm, x_perm_scale, w13,
                w13_scale, h, h_scale, s);
}

moe_status moe_ffn_down(const moe_problem* p, const int32_t* offsets,
                        const void* h, const void* h_scale, const void* w2,
                        const void* w2_scale, void* y, void* workspace,
                        size_t* workspace_bytes, void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (!workspace_bytes) return MOE_ERR_INVALID_ARG;
  const int mt = tile_rows(q);
  Carve c(workspace);
  FfnWs fw = carve_ffn_ws(c, q, mt);
  if (!workspace) { *workspace_bytes = c.off; return MOE_OK; }
  if (*workspace_bytes < c.off) return MOE_ERR_WORKSPACE;
  if ((st = check_weights(q, nullptr, nullptr, w2, w2_scale, false, true)) != MOE_OK)
    return st;
  if (q.El == 0 || q.N == 0) return MOE_OK;
  if (!offsets || !h || !y) return MOE_ERR_INVALID_ARG;
  if ((q.mx || q.i8) ? !h_scale : (h_scale != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!ws_aligned(workspace) || !aligned16(offsets, h, h_scale, w2, w2_scale, y))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(moe::launch_build_tiles(offsets, q.fb, q.fe, mt, fw.tiles,
                                  (int)max_tiles(q, mt), fw.tile_count, s));
  return run_down(q, mt, fw.tiles, fw.tile_count, h, h_scale, w2, w2_scale, y,
                  s);
}

moe_status moe_grouped_ffn(const moe_problem* p, const int32_t* offsets,
                           const void* x_perm, const void* x_perm_scale,
                           const void* w13, const void* w13_scale,
                           const void* w2, const void* w2_scale, void* y,
                           void* workspace, size_t* workspace_bytes,
                           void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (!workspace_bytes) return MOE_ERR_INVALID_ARG;
  const int mt = tile_rows(q);
  Carve c(workspace);
  FfnWs fw = carve_ffn_ws(c, q, mt);
  void* h = c.take<char>((size_t)q.N * q.I * ((q.mx || q.i8) ? 1 : act_bytes(q)));
  void* hs = q.mx ? (void*)c.take<uint8_t>((size_t)q.N * (q.I / 32))
             : q.i8 ? (void*)c.take<float>((size_t)q.N) : nullptr;
  float* h32 = q.i8 ? c.take<float>((size_t)q.N * q.I) : nullptr;
  if (!workspace) { *workspace_bytes = c.off; return MOE_OK; }
  if (*workspace_bytes < c.off) return MOE_ERR_WORKSPACE;
  if ((st = check_weights(q, w13, w13_scale, w2, w2_scale, true, true)) != MOE_OK)
    return st;
  if (q.El == 0 || q.N == 0) return MOE_OK;
  if (!offsets || !x_perm || !y) return MOE_ERR_INVALID_ARG;
  if ((q.mx || q.i8) ? !x_perm_scale : (x_perm_scale != nullptr))
    return MOE_ERR_INVALID_ARG;
  if (!ws_aligned(workspace) ||
      !aligned16(offsets, x_perm, x_perm_scale, w13, w13_scale, w2, w2_scale, y))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(moe::launch_build_tiles(offsets, q.fb, q.fe, mt, fw.tiles,
                                  (int)max_tiles(q, mt), fw.tile_count, s));
  st = run_up(q, mt, fw.tiles, fw.tile_count, x_perm, x_perm_scale, w13,
              w13_scale, q.i8 ? (void*)h32 : h, hs, s);
  if (st != MOE_OK) return st;
  if (q.i8 && (st = run_quant_h(q, h32, offsets, h, hs, s)) != MOE_OK)
    return st;
  return run_down(q, mt, fw.tiles, fw.tile_count, h, hs, w2, w2_scale, y, s);
}

moe_status moe_finalize(const moe_problem* p, const int32_t* topk_ids,
                        const float* topk_weight, const int32_t* copy_pos,
                        const int32_t* offsets, const void* y, const void* x,
                        const void* residual, void* out, void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (q.T == 0) return MOE_OK;
  if (!topk_ids || !topk_weight || !copy_pos || !offsets || !x || !out)
    return MOE_ERR_INVALID_ARG;
  if (q.El > 0 && !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(topk_ids, topk_weight, copy_pos, offsets, y, x, residual, out))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_finalize(
      topk_ids, topk_weight, copy_pos, offsets, q.fb, q.nffn, q.lb, q.le, y, x,
      residual, out, q.act == MOE_F32 ? 0 : 1, q.T, q.H, q.k,
      (hipStream_t)stream));
}

moe_status moe_add_rms_norm_cast(int32_t T, int32_t H, const void* x,
                                 const void* residual, const void* norm_weight,
                                 float epsilon, float* y_f32, void* y_bf16,
                                 void* residual_out, void* stream) {
  if (T < 0 || H <= 0 || !(epsilon >= 0.f) || epsilon > 3.0e38f)
    return MOE_ERR_INVALID_ARG;
  if (H % 32 || H > kMaxNormH) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !norm_weight || (!y_f32 && !y_bf16)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x, residual, norm_weight, y_f32, y_bf16, residual_out))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_add_rms_norm(
      0, (const uint16_t*)x, (const uint16_t*)residual,
      (const uint16_t*)norm_weight, epsilon, T, H, y_f32, (uint16_t*)y_bf16,
      nullptr, nullptr, (uint16_t*)residual_out, (hipStream_t)stream));
}

moe_status moe_add_rms_norm_mx_quant(int32_t T, int32_t H, const void* x,
                                     const void* residual,
                                     const void* norm_weight, float epsilon,
                                     uint8_t* y_codes, uint8_t* y_scales,
                                     void* residual_out, void* stream) {
  if (T < 0 || H <= 0 || !(epsilon >= 0.f) || epsilon > 3.0e38f)
    return MOE_ERR_INVALID_ARG;
  if (H % 32 || H > kMaxNormH) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !norm_weight || !y_codes || !y_scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x, residual, norm_weight, y_codes, y_scales, residual_out))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_add_rms_norm(
      1, (const uint16_t*)x, (const uint16_t*)residual,
      (const uint16_t*)norm_weight, epsilon, T, H, nullptr, nullptr, y_codes,
      y_scales, (uint16_t*)residual_out, (hipStream_t)stream));
}

moe_status moe_pack_weights(int32_t E, int32_t N, int32_t K_bytes,
                            const void* src, void* dst, void* stream) {
  if (E < 0 || N <= 0 || K_bytes <= 0) return MOE_ERR_INVALID_ARG;
  if (N % 16 || K_bytes % 64 || (long long)N * K_bytes >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  if (E == 0) return MOE_OK;
  if (!src || !dst || !aligned16(src, dst)) return MOE_ERR_INVALID_ARG;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  const uintptr_t n = (uintptr_t)E * N * K_bytes;
  if (a < b + n && b < a + n) return MOE_ERR_INVALID_ARG;  // overlap
  return hip_status(moe::launch_pack_weights(E, N, K_bytes,
                                             (const uint8_t*)src,
                                             (uint8_t*)dst,
                                             (hipStream_t)stream));
}

moe_status moe_pack_bf16_weights(int32_t E, int32_t K, int32_t N,
                                 int32_t glu, const void* src, void* dst,
                                 void* stream) {
  if (E < 0 || K <= 0 || N <= 0 || (glu != 0 && glu != 1))
    return MOE_ERR_INVALID_ARG;
  if (K % 32 || N % 256 || (long long)E * K * N >= (1LL << 40))
    return MOE_ERR_UNSUPPORTED;
  if (E == 0) return MOE_OK;
  if (!src || !dst || !aligned16(src, dst)) return MOE_ERR_INVALID_ARG;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  const uintptr_t n = (uintptr_t)E * K * N * 2;
  if (a < b + n && b < a + n) return MOE_ERR_INVALID_ARG;  // overlap
  return hip_status(moe::launch_pack_bf16_weights(
      E, K, N, glu != 0, (const uint16_t*)src, (uint16_t*)dst,
      (hipStream_t)stream));
}

moe_status moe_quant_mxfp4_weights(int32_t E, int32_t K, int32_t N,
                                   const void* w, uint8_t* codes,
                                   uint8_t* scales, void* stream) {
  if (E < 0 || K <= 0 || N <= 0) return MOE_ERR_INVALID_ARG;
  if (K % 32 || (long long)E * N * K >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  if (E == 0) return MOE_OK;
  if (!w || !codes || !scales || !aligned16(w, codes, scales))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_quant_mxfp4_weights(
      E, K, N, (const uint16_t*)w, codes, scales, (hipStream_t)stream));
}

moe_status moe_router_logits(int32_t T, int32_t H, int32_t E, const float* y,
                             const float* w_router, float* logits,
                             void* stream) {
  if (T < 0 || H <= 0 || E <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 16 || E % 32 || E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y, w_router, logits)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router_logits(y, w_router, logits, T, H, E,
                                              (hipStream_t)stream));
}

moe_status moe_layer_traced(const moe_problem* p, const float* logits,
                            const void* x, const void* residual,
                            const void* w13, const void* w13_scale,
                            const void* w2, const void* w2_scale, void* out,
                            void* workspace, size_t* workspace_bytes,
                            void* stream, void* const* stage_events,
                            int32_t n_events) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if (!workspace_bytes || n_events < 0) return MOE_ERR_INVALID_ARG;
  const int mt = tile_rows(q);
  const size_t N = (size_t)q.N;
  const int nch = moe::route_num_chunks((int)q.N);
  Carve c(workspace);
  int32_t* ids = c.take<int32_t>(N);
  float* wts = c.take<float>(N);
  int32_t* counts = c.take<int32_t>(q.E);
  int32_t* offsets = c.take<int32_t>(q.E + 1);
  int32_t* cc = c.take<int32_t>((size_t)nch * q.E + 1);
  int32_t* sorted_copy = c.take<int32_t>(N);
  int32_t* copy_pos = c.take<int32_t>(N);
  FfnWs fw = carve_ffn_ws(c, q, mt);
  const size_t ab = (q.mx || q.i8) ? 1 : act_bytes(q);
  // bf16: GEMM1 reads its rows straight from x (no permuted copy)
  const bool gather = fused_gather(q);
  // MXFP8 with the tiled GEMM, and int8: x is quantised once per token and
  // GEMM1 reads the token rows of the codes (32-bit offsets)
  const bool small_x = (int64_t)q.T * q.H < (int64_t(1) << 31);
  const bool mx_tok = q.mx && small_x;
  const bool i8_tok = q.i8 && small_x;
  const size_t xrows = (mx_tok || i8_tok) ? (size_t)q.T : N;
  void* xp = c.take<char>(q.El && !gather ? xrows * q.H * ab : 0);
  void* xs = q.mx ? (void*)c.take<uint8_t>(q.El ? xrows * (q.H / 32) : 0)
             : q.i8 ? (void*)c.take<float>(q.El ? xrows : 0) : nullptr;
  void* h = c.take<char>(q.El ? N * q.I * ab : 0);
  void* hs = q.mx ? (void*)c.take<uint8_t>(q.El ? N * (q.I / 32) : 0)
             : q.i8 ? (void*)c.take<float>(q.El ? N : 0) : nullptr;
  float* h32 = q.i8 ? c.take<float>(q.El ? N * q.I : 0) : nullptr;
  void* y = c.take<char>(q.El ? N * q.H * act_bytes(q) : 0);
  if (!workspace) { *workspace_bytes = c.off; return MOE_OK; }
  if (*workspace_bytes < c.off) return MOE_ERR_WORKSPACE;
  if ((st = check_weights(q, w13, w13_scale, w2, w2_scale, true, true)) != MOE_OK)
    return st;
  if (q.T == 0) return MOE_OK;
  if (!logits || !x || !out) return MOE_ERR_INVALID_ARG;
  if (!ws_aligned(workspace) ||
      !aligned16(logits, x, residual, w13, w13_scale, w2, w2_scale, out))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) -> hipError_t {
    if (stage_events && i < n_events && stage_events[i])
      return hipEventRecord((hipEvent_t)stage_events[i], s);
    return hipSuccess;
  };
  // small problems route in one block
  const bool small = moe::route_small_ok((int)q.N, q.E);
  const int mtl = (int)max_tiles(q, mt);
  // the per-token quantisation of x (W4A8 tiled, W8A8) rides along with the
  // gate when the fused kernel covers the shape, else, on the multi-block
  // routing path, with the scan (one latency-bound block, the rest of the
  // chip free); a separate launch otherwise. Beside the gate measured ahead
  // of beside the scan once the scan had become short: W4A8 rank layer
  // 248.8 -> 246.4 us, W8A8 skewed prefill 336.0 -> 333.0 us.
  const bool tok_q = q.El > 0 && (mx_tok || i8_tok);
  const bool fused_q = tok_q && moe::gate_quant_ok(q.E, q.H, q.mx);
  const bool scan_q = tok_q && !fused_q && !small;
  MOE_TRY(mark(0));
  if (fused_q)
    MOE_TRY(moe::launch_gate_topk_quant(logits, q.T, q.E, q.k, ids, wts,
                                        (const uint16_t*)x, q.H, q.mx, xp, xs,
                                        s));
  else
    MOE_TRY(moe::launch_gate_topk(logits, q.T, q.E, q.k, ids, wts, s));
  MOE_TRY(mark(1));
  if (small) {
    MOE_TRY(moe::launch_route_small(ids, (int)q.N, q.E, counts, offsets,
                                    sorted_copy, copy_pos, q.fb, q.fe, mt,
                                    mtl ? fw.tiles : nullptr, mtl,
                                    fw.tile_count, s));
  } else {
    MOE_TRY(moe::launch_route_count(ids, (int)q.N, q.E, cc, s));
  }
  MOE_TRY(mark(2));
  if (!small)
    MOE_TRY(moe::launch_route_scan(cc, nch, q.E, counts, offsets, q.fb, q.fe,
                                   mt, mtl ? fw.tiles : nullptr, mtl,
                                   fw.tile_count, s, (const uint16_t*)x, q.H,
                                   scan_q ? q.T : 0, scan_q ? (q.mx ? 1 : 2) : 0,
                                   xp, xs));
  MOE_TRY(mark(3));
  if (!small)
    MOE_TRY(moe::launch_route_scatter(ids, (int)q.N, q.E, cc, offsets,
                                      sorted_copy, copy_pos, s));
  MOE_TRY(mark(4));
  if (fused_q || scan_q)
    ;  // x was quantised with the gate or with the scan
  else if (q.El > 0 && mx_tok)
    MOE_TRY(moe::launch_quantize_mx(x, (int)q.T, q.H, (uint8_t*)xp,
                                    (uint8_t*)xs, s));
  else if (q.El > 0 && i8_tok)
    MOE_TRY(moe::launch_quant_i8_rows(false, x, q.H, (int)q.T, nullptr,
                                      nullptr, 0, 0, 1, (int8_t*)xp,
                                      (float*)xs, s));
  else if (q.El > 0 && q.i8)
    MOE_TRY(moe::launch_quant_i8_rows(false, x, q.H, (int)q.N, sorted_copy,
                                      offsets, q.fb, q.fe, q.k, (int8_t*)xp,
                                      (float*)xs, s));
  else if (q.El > 0 && !gather)
    MOE_TRY(moe::launch_route_gather(x, q.act == MOE_F32 ? 0 : 1, q.mx ? 1 : 0,
                                     q.H, q.k, sorted_copy, offsets, q.fb,
                                     q.fe, (int)q.N, xp, (uint8_t*)xs, s));
  MOE_TRY(mark(5));
  void* h_up = q.i8 ? (void*)h32 : h;  // W8A8: fp32 h, quantised below
  if (q.El > 0) {
    if (gather)
      st = run_up(q, mt, fw.tiles, fw.tile_count, x, nullptr, w13, w13_scale,
                  h_up, hs, s, sorted_copy, offsets + q.fb);
    else if (mx_tok || i8_tok)
      st = run_up(q, mt, fw.tiles, fw.tile_count, xp, xs, w13, w13_scale,
                  h_up, hs, s, sorted_copy, offsets + q.fb);
    else
      st = run_up(q, mt, fw.tiles, fw.tile_count, xp, xs, w13, w13_scale,
                  h_up, hs, s);
    if (st != MOE_OK) return st;
  }
  MOE_TRY(mark(6));
  if (q.El > 0) {
    if (q.i8 && (st = run_quant_h(q, h32, offsets, h, hs, s)) != MOE_OK)
      return st;
    st = run_down(q, mt, fw.tiles, fw.tile_count, h, hs, w2, w2_scale, y, s);
    if (st != MOE_OK) return st;
  }
  MOE_TRY(mark(7));
  MOE_TRY(moe::launch_finalize(ids, wts, copy_pos, offsets, q.fb, q.nffn, q.lb,
                               q.le, y, x, residual, out,
                               q.act == MOE_F32 ? 0 : 1, q.T, q.H, q.k, s));
  MOE_TRY(mark(8));
  return MOE_OK;
}

moe_status moe_layer(const moe_problem* p, const float* logits, const void* x,
                     const void* residual, const void* w13,
                     const void* w13_scale, const void* w2,
                     const void* w2_scale, void* out, void* workspace,
                     size_t* workspace_bytes, void* stream) {
  return moe_layer_traced(p, logits, x, residual, w13, w13_scale, w2, w2_scale,
                          out, workspace, workspace_bytes, stream, nullptr, 0);
}

moe_status moe_prefetch_weights(const moe_problem* p, const int32_t* topk_ids,
                                const void* w13, const void* w2, int32_t which,
                                int64_t max_bytes, void* stream) {
  Prob q;
  moe_status st = check(p, &q);
  if (st != MOE_OK) return st;
  if ((which & ~3) || max_bytes < 0) return MOE_ERR_INVALID_ARG;
  if (q.act == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (q.El == 0 || q.N == 0 || which == 0 || max_bytes < 16) return MOE_OK;
  if (((which & 1) && !w13) || ((which & 2) && !w2)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(topk_ids, w13, w2)) return MOE_ERR_INVALID_ARG;
  const int mt = tile_rows(q);
  // w13 and w2 share the budget in proportion to their sizes (w13 holds
  // H x 2I elements, w2 I x H: two thirds and one third)
  long long b13 = 0, b2 = 0;
  if (which == 3) {
    b13 = max_bytes / 3 * 2;
    b2 = max_bytes - b13;
  } else if (which == 1) {
    b13 = max_bytes;
  } else {
    b2 = max_bytes;
  }
  hipStream_t s = (hipStream_t)stream;
  const int nids = topk_ids ? (int)q.N : 0;
  for (int up = 1; up >= 0; --up) {
    const long long b = up ? b13 : b2;
    if (b < 16) continue;
    const Geom g = gemm_geom(q, mt, up != 0);
    int nexp = g.round_tiles < q.El ? g.round_tiles : q.El;
    if (topk_ids && (long long)nexp > q.N) nexp = (int)q.N;
    const moe::Prefetch pf =
        make_prefetch(g, up ? w13 : w2, q, topk_ids, nids, 0, b, nexp);
    MOE_TRY(moe::launch_prefetch(pf, kPrefetchBlocks, s));
  }
  return MOE_OK;
}

moe_status moe_layer_noalloc(const moe_problem* p, const float* logits,
                             const void* x, const void* residual,
                             const void* w13, const void* w13_scale,
                             const void* w2, const void* w2_scale, void* out,
                             void* stream) {
  // host-side size query first: a problem past the scratch is refused
  // before anything is looked up or launched
  size_t need = 0;
  moe_status st = moe_layer_traced(p, logits, x, residual, w13, w13_scale, w2,
                                   w2_scale, out, nullptr, &need, stream,
                                   nullptr, 0);
  if (st != MOE_OK) return st;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != MOE_OK) return st;
  size_t have = MOE_NOALLOC_SCRATCH_BYTES;
  return moe_layer_traced(p, logits, x, residual, w13, w13_scale, w2, w2_scale,
                          out, ws, &have, stream, nullptr, 0);
}

}  // extern "C"
