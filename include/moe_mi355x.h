/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) MoE expert-layer library.
 *
 * The layer: router logits -> gating top-k softmax -> routing (expert
 * histogram, stable permutation of token copies, gather) -> grouped GEMM over
 * the merged gate/up weights w13 with a fused SwiGLU -> grouped GEMM over the
 * down weights w2 -> finalize (weighted un-permute and sum, identity experts,
 * optional residual).
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters"
 *   [P2] "LongCat-Flash inference on Atlas A3 clusters"
 *   [P3] "NPU Qwen3-Next inference practice" (quantisation strategy only)
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers to memory the caller allocated
 *     and owns. The library never allocates, frees, copies to the host or
 *     synchronises; it only enqueues kernels on `stream` (a hipStream_t; NULL
 *     is the null stream). Outputs are overwritten, never accumulated into.
 *   - Every array is row-major and contiguous. Sizes are element counts.
 *   - Argument checks run on the host before any launch. A failed check
 *     returns an error and enqueues nothing. A launch failure returns
 *     MOE_ERR_HIP. Faults inside kernels surface at the caller's next
 *     synchronisation. Nothing is printed; no call aborts.
 *   - Calls keep no mutable global state and may run concurrently on
 *     different streams with different buffers (moe_layer_noalloc excepted:
 *     its scratch is one array per GPU).
 *   - Workspace (hipcub style): when `workspace` is NULL the call stores the
 *     bytes it needs in *workspace_bytes, returns MOE_OK and launches nothing.
 *     Otherwise *workspace_bytes is the size of `workspace`; a buffer that is
 *     too small gives MOE_ERR_WORKSPACE.
 *   - Alignment: every array pointer must be 16-byte aligned and the
 *     workspace 256-byte aligned (allocations from hipMalloc or the torch
 *     allocator are); a misaligned one gives MOE_ERR_INVALID_ARG.
 *
 * Expert ids: FFN experts are [0, n_ffn); identity ("zero-compute") experts
 * are [n_ffn, n_ffn + n_zero) and return their input, MoE(x) = x ([P2]
 * "MoE模块 / Decode阶段优化"). E_tot = n_ffn + n_zero. A call handles the ids
 * in [local_begin, local_end) -- one expert-parallel rank's share ([P1] "MoE
 * EP优化 / AllGather方案": routing keeps only the copies of this rank's
 * experts and finalize yields a partial sum). Copies of experts outside the
 * range contribute 0. The FFN experts of the range, [fb, fe) with
 * fb = min(local_begin, n_ffn) and fe = min(local_end, n_ffn), are the ones
 * whose weights the call receives, indexed by e - fb (E_loc = fe - fb).
 *
 * Limits: 1 <= top_k <= min(E_tot, 64); E_tot <= 2048; H and I multiples of
 * 32; T*top_k < 2^31. Status MOE_ERR_UNSUPPORTED otherwise.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad range            */
  MOE_ERR_UNSUPPORTED = 2, /* valid problem outside this library's limits  */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than required              */
  MOE_ERR_HIP = 4          /* a HIP launch failed                           */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_MXFP8_E4M3 = 2, /* e4m3fn codes + one e8m0 scale per 32 along K      */
  MOE_MXFP4_E2M1 = 3, /* e2m1 codes, 2 per byte (low nibble = even k),
                         + one e8m0 scale per 32 along K                    */
  MOE_INT8 = 4        /* symmetric int8 codes in [-127, 127] + one fp32
                         scale per output channel (weights, static) or per
                         row (activations, dynamic: amax / 127)             */
} moe_dtype;

/* Layout of the expert weights handed to a call (moe_problem.wt_layout). */
typedef enum moe_layout {
  MOE_LAYOUT_ROWMAJOR = 0, /* as in "Weight layouts" below, unpacked        */
  MOE_LAYOUT_PACKED = 1    /* the packed order of moe_pack_weights (MXFP4,
                              INT8) or moe_pack_bf16_weights (BF16)          */
} moe_layout;

typedef struct moe_problem {
  int32_t T;           /* tokens                                            */
  int32_t H;           /* hidden size                                       */
  int32_t I;           /* per-expert intermediate size                      */
  int32_t n_ffn;       /* FFN experts                                       */
  int32_t n_zero;      /* identity experts                                  */
  int32_t top_k;       /* experts per token                                 */
  int32_t local_begin; /* expert-id range handled by the call              */
  int32_t local_end;
  int32_t act;   /* MOE_F32 | MOE_BF16: x, residual, y, out, h (unquantised) */
  int32_t wt;    /* MOE_F32 | MOE_BF16 | MOE_MXFP4_E2M1 | MOE_INT8          */
  int32_t act_q; /* == act (no quantisation) | MOE_MXFP8_E4M3 | MOE_INT8
                    (dynamic)                                               */
  int32_t wt_layout; /* moe_layout of w13 / w2: MOE_LAYOUT_PACKED for
                        MXFP4_E2M1 and INT8 weights, MOE_LAYOUT_ROWMAJOR for
                        F32, either for BF16 (packed: the slab order of
                        moe_pack_bf16_weights, I % 128 == 0 and
                        H % 256 == 0); any other pairing is refused with
                        MOE_ERR_UNSUPPORTED before anything is launched (the
                        quantised GEMMs read only the packed order: pack
                        row-major MXFP4 / int8 weights once with
                        moe_pack_weights)                                    */
} moe_problem;

/* Supported combinations: (act, wt, act_q) = (F32, F32, F32),
 * (BF16, BF16, BF16), (BF16, MXFP4_E2M1, MXFP8_E4M3) and W8A8
 * (BF16, INT8, INT8) -- [P3] "量化策略": routed experts with int8 weights
 * (static per-channel scales) and int8 activations (dynamic per-token
 * scales). MX and INT8 need H and I multiples of 128; INT8 also
 * 2 * I * H < 2^31.
 *
 * Dynamic int8 quantisation of a row v (x per token before routing, h per
 * row between the GEMMs, after h is formed in fp32): scale = amax|v| / 127
 * rounded to fp32, code = rint(v / scale) with the quotient rounded to fp32
 * and ties to even, clipped to [-127, 127]; an all-zero row has scale 0 and
 * codes 0. int8 products are summed exactly in int32 and dequantised as
 * acc * row scale * channel scale in fp32.
 *
 * Scale pointers (x_perm_scale, h_scale, w13_scale, w2_scale) point to
 * uint8 e8m0 codes for MX and to fp32 values for INT8.
 *
 * Weight layouts (E_loc experts, weights of expert e at index e - fb):
 *   F32 / BF16:  w13 [E_loc, H, 2I]   columns [0, I) = gate, [I, 2I) = up
 *                w2  [E_loc, I, H]
 *                (the merged gate/up matrix of [P1] "MoE TP优化 / 计算分解")
 *   MXFP4_E2M1:  w13 = W13 [E_loc, 2I, H/2] bytes (K = H per output
 *                column, two codes per byte; columns [0, I) gate, [I, 2I)
 *                up) and w2 = W2 [E_loc, H, I/2] bytes, each in the packed
 *                order below (same byte count);
 *                w13_scale [E_loc, 2I, H/32] e8m0 (not packed)
 *                w2_scale [E_loc, H, I/32] e8m0 (not packed)
 *   INT8:        w13 = W13 [E_loc, 2I, H] int8 (K = H per output column;
 *                columns [0, I) gate, [I, 2I) up) and w2 = W2 [E_loc, H, I]
 *                int8, each in the packed order below (same byte count);
 *                w13_scale fp32 [E_loc, 2I] (one per output column),
 *                w2_scale fp32 [E_loc, H]
 * Scale pointers must be NULL unless wt is MXFP4_E2M1 or INT8.
 * The quantised byte matrices W13 / W2 arrive row-major (K contiguous, as
 * moe_quant_mxfp4_weights writes them) from a checkpoint; the calls below
 * take them only in the packed order, made once by moe_pack_weights, and the
 * problem states which it holds (wt_layout): a row-major quantised buffer is
 * refused with MOE_ERR_UNSUPPORTED, never misread.
 *
 * Packed weights (MXFP4_E2M1 and INT8): a static weight matrix W [E, N, Kb]
 * of bytes (Kb = K for int8, K/2 for e2m1; K contiguous per output column
 * n) is stored as fragments of 1 KB in the order [E][Kb/64][N/16];
 * fragment (e, c, n16) holds, at byte 16 * l (l = 0..63), the 16 bytes
 * W[e, 16 * n16 + l % 16, 64 * c + 16 * (l / 16) .. + 15]: exactly what
 * lane l of a wave feeds as the B operand of a v_mfma_i32_16x16x64_i8 (K
 * bytes [64 c, + 64)) or of a scaled v_mfma_*_16x16x128_f8f6f4 (e2m1, K
 * [128 c, + 128)), and one LDS copy instruction's worth for the tiled
 * kernels. Every weight load of the quantised GEMMs then reads 1 KB
 * contiguous (K-contiguous rows read 64 bytes per column per load
 * otherwise, ~30 % below the streaming rate). moe_pack_weights converts
 * once, e.g. when the weights are loaded.
 *
 * Slab-packed weights (BF16 with MOE_LAYOUT_PACKED): the bf16 GEMMs read an
 * expert's matrix W [K, N] in slabs of 256 columns -- for w13 (N = 2I) slab
 * j holds the gate columns [128 j, 128 j + 128) and the matching up columns
 * [I + 128 j, I + 128 j + 128), for w2 (N = H) the columns [256 j, 256 j +
 * 256) -- and each slab in K steps of 32 rows. Packed, the 32 x 256 block of
 * step s of slab j is one contiguous 16 KB, in the order [E][N/256][K/32]
 * [32][256]: element (e, j, s, r, c) = W[e][32 s + r][col_j(c)], col_j(c) =
 * 128 j + c for c < 128 and I + 128 j + c - 128 otherwise (w13), 256 j + c
 * (w2). Same element count as row-major, same results bit for bit. Which
 * layout streams faster depends on the experts (measured on MI355X): row-
 * major, the blocks reading the slabs of one expert share DRAM rows, which
 * pays while they run in step (2048 x 768 experts at decode batch sizes:
 * row-major layer 3-4 % faster); blocks that stream long slabs over several
 * rounds drift apart, and then contiguous slabs pay (6144 x 2048 experts at
 * 16 rows each: slab order 4 % faster). Prefill-size batches are neutral.
 */

/* Gating: [P1] "GMM使能和Routing优化 / 快速选择专家" (fused top-k + softmax
 * replacing topk-then-softmax); [P2] "MoE模块 / Router" (sort router output,
 * take the top-k experts).
 *   logits      fp32 [T, E_tot]
 *   topk_ids    int32 [T, top_k]  the k largest logits per token, descending,
 *                                 ties to the lower expert id
 *   topk_weight fp32  [T, top_k]  softmax over the k selected logits (the
 *                                 full softmax renormalised over the top-k)
 * Uses all E_tot experts regardless of the local range. */
MOE_API moe_status moe_gate_topk(const moe_problem* p, const float* logits,
                         int32_t* topk_ids, float* topk_weight, void* stream);

/* Routing: [P1] "高效排序和token路由" (init_routing sorts the token copies by
 * expert, compute_expert_tokens counts each expert's tokens); [P1] "MoE
 * EP优化 / AllGather方案" (MXFP8 quantisation of the hidden states and
 * routing restricted to the local expert range).
 * Copies are numbered c = t * top_k + j.
 *   topk_ids          int32 [T, top_k]; ids outside [0, E_tot) are ignored
 *                     (not counted; their copy_pos is -1)
 *   x                 act [T, H]
 *   tokens_per_expert int32 [E_tot]   copies routed to each expert
 *   offsets           int32 [E_tot+1] exclusive prefix sum; offsets[E_tot]
 *                     is the number of valid copies
 *   sorted_copy       int32 [T*top_k] copies sorted by (expert id, c)
 *   copy_pos          int32 [T*top_k] inverse: sorted position of copy c
 *   x_perm            rows r = 0 .. R-1, R = offsets[fe] - offsets[fb]:
 *                     x_perm[r] = x[sorted_copy[offsets[fb] + r] / top_k];
 *                     act [T*top_k, H] or, when act_q is MXFP8_E4M3, e4m3
 *                     codes uint8 [T*top_k, H], or when act_q is INT8 the
 *                     token's int8 codes [T*top_k, H]. Rows >= R are not
 *                     written.
 *   x_perm_scale      e8m0 uint8 [T*top_k, H/32] when act_q is MXFP8_E4M3,
 *                     the token's fp32 scale [T*top_k] when act_q is INT8,
 *                     else must be NULL.
 *   workspace         scratch (see conventions). */
MOE_API moe_status moe_init_routing(const moe_problem* p, const int32_t* topk_ids,
                            const void* x, int32_t* tokens_per_expert,
                            int32_t* offsets, int32_t* sorted_copy,
                            int32_t* copy_pos, void* x_perm,
                            void* x_perm_scale, void* workspace,
                            size_t* workspace_bytes, void* stream);

/* Grouped expert FFN: [P1] "MoE TP优化 / 计算分解" (expert =
 * down(SiLU(gate(x)) * up(x)); npu_swiglu halves the last axis and returns
 * SiLU(first) * second) and "高性能专家计算" (all experts' matmuls in one
 * grouped operator). For every FFN expert e in [fb, fe) with rows
 * [offsets[e] - offsets[fb], offsets[e+1] - offsets[fb]) of x_perm:
 *   h = SwiGLU(x_perm_rows @ w13[e])   fp32 accumulation (int32 for INT8);
 *                                      stored in act dtype, or MXFP8 (one
 *                                      e8m0 per 32 along I) when act_q is
 *                                      MXFP8_E4M3, or int8 with one fp32
 *                                      scale per row when act_q is INT8
 *   y = h @ w2[e]                      fp32 (int32) accumulation, stored in act
 * Experts with no rows never read their weights.
 *   offsets  int32 [E_tot+1] as produced by moe_init_routing
 *   y        act [T*top_k, H]; rows >= R are not written
 * moe_ffn_up and moe_ffn_down are the two halves (h buffer explicit):
 *   h        act [T*top_k, I], or e4m3 codes uint8 [T*top_k, I], or int8
 *            codes [T*top_k, I]
 *   h_scale  e8m0 uint8 [T*top_k, I/32] when act_q is MXFP8_E4M3, fp32
 *            [T*top_k] when act_q is INT8, else NULL */
MOE_API moe_status moe_grouped_ffn(const moe_problem* p, const int32_t* offsets,
                           const void* x_perm, const void* x_perm_scale,
                           const void* w13, const void* w13_scale,
                           const void* w2, const void* w2_scale, void* y,
                           void* workspace, size_t* workspace_bytes,
                           void* stream);

MOE_API moe_status moe_ffn_up(const moe_problem* p, const int32_t* offsets,
                      const void* x_perm, const void* x_perm_scale,
                      const void* w13, const void* w13_scale, void* h,
                      void* h_scale, void* workspace,
                      size_t* workspace_bytes, void* stream);

MOE_API moe_status moe_ffn_down(const moe_problem* p, const int32_t* offsets,
                        const void* h, const void* h_scale, const void* w2,
                        const void* w2_scale, void* y, void* workspace,
                        size_t* workspace_bytes, void* stream);

/* Finalize: [P1] "高效排序和token路由" (finalize_routing restores token order
 * and takes the weighted sum) and [P2] "Decode阶段优化" (identity experts).
 *   out[t] = residual[t] + sum_{j=0..k-1} topk_weight[t,j] * v(t,j)
 *   v = y[copy_pos[t*k+j] - offsets[fb]]  FFN expert in the range
 *     = x[t]                              identity expert in the range
 *     = 0                                 expert outside the range
 * Summed in fp32 in the order j = 0..k-1 starting from the residual,
 * rounded once to act.
 *   residual act [T, H] or NULL; x act [T, H]; y as from moe_grouped_ffn;
 *   out act [T, H]. */
MOE_API moe_status moe_finalize(const moe_problem* p, const int32_t* topk_ids,
                        const float* topk_weight, const int32_t* copy_pos,
                        const int32_t* offsets, const void* y, const void* x,
                        const void* residual, void* out, void* stream);

/* The whole layer in one call: gate, routing, grouped FFN, finalize. All
 * intermediates live in `workspace`. Same result as the five calls above in
 * sequence. */
MOE_API moe_status moe_layer(const moe_problem* p, const float* logits, const void* x,
                     const void* residual, const void* w13,
                     const void* w13_scale, const void* w2,
                     const void* w2_scale, void* out, void* workspace,
                     size_t* workspace_bytes, void* stream);

/* moe_layer with stage timing: when stage_events is non-NULL, entry i (a
 * hipEvent_t or NULL) is recorded on `stream` right before stage i is
 * enqueued, for i < n_events, with stages 0 gate, 1 expert histogram,
 * 2 scan (+ GEMM tile list), 3 permutation, 4 gather (+ MXFP8 or int8
 * quantisation of x), 5 GEMM1 + SwiGLU, 6 GEMM2, 7 finalize, and entry 8
 * after the last. Each of stages 0-7 is at most one kernel launch (a stage
 * with nothing to do launches nothing), except stage 6 for INT8, which
 * quantises h and then runs GEMM2. Where x is quantised once per token
 * (INT8, and MXFP8 with 128-row GEMM tiles), the gate launch of stage 0
 * quantises it for E_tot <= 256 (int8: only for H = 2048 or 4096), else
 * the scan launch of stage 2 when routing takes the multi-block path (more
 * than 4096 copies or 1024 experts); stage 4 is then empty, and otherwise
 * holds the quantisation. For performance tooling; results are identical
 * to moe_layer. */
MOE_API moe_status moe_layer_traced(const moe_problem* p, const float* logits,
                                    const void* x, const void* residual,
                                    const void* w13, const void* w13_scale,
                                    const void* w2, const void* w2_scale,
                                    void* out, void* workspace,
                                    size_t* workspace_bytes, void* stream,
                                    void* const* stage_events, int32_t n_events);

/* Weight prefetch ([P2] "LongCat-Flash inference on Atlas A3 clusters",
 * section 权重预取: the weights of a memory-bound matmul are fetched ahead
 * while an earlier, latency-bound operator runs, about HBM bandwidth x that
 * operator's duration of them; its AFD section does the same for the FFN
 * side's grouped matmuls in communication gaps). Reads up to max_bytes of the
 * expert weights the layer's grouped GEMMs will read first -- the heads of
 * the K ranges their waves start at, for the experts of their first round of
 * blocks -- so that those lines are in the GPU's caches (the memory-side
 * cache in front of HBM) when moe_layer / moe_grouped_ffn runs next with the
 * same problem and weights. For a caller to enqueue on a second stream while
 * the operators in front of the MoE layer (attention, the fused norm) run.
 * It writes nothing and changes no result.
 *   topk_ids  int32 [T, top_k] (the gate's output) or NULL: only the experts
 *             it routes to are read (ids outside the local range are
 *             ignored); NULL reads every local expert.
 *   w13, w2   the layer's weight arguments (as for moe_layer); which: bit 0
 *             reads w13 (GEMM1), bit 1 w2 (GEMM2), the budget split 2 : 1.
 *             w2's heads help only when GEMM1 leaves them cached, i.e. when
 *             the layer's weights are small against the 256 MB cache.
 *   max_bytes upper bound of the bytes read (>= 0; below 16 reads nothing).
 * The layer itself does not prefetch: spare blocks of its gate and routing
 * launches reading ahead were measured to lengthen those latency-bound
 * kernels by more than the GEMM gained. Checks as for moe_layer (which
 * outside 0..3 or max_bytes < 0: MOE_ERR_INVALID_ARG; fp32 problems:
 * MOE_ERR_UNSUPPORTED). */
MOE_API moe_status moe_prefetch_weights(const moe_problem* p,
                                        const int32_t* topk_ids,
                                        const void* w13, const void* w2,
                                        int32_t which, int64_t max_bytes,
                                        void* stream);

/* moe_layer without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The layer's intermediates live in a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * nothing itself. Same arguments as moe_layer minus the workspace pair, and
 * the same result bit for bit. A problem whose moe_layer workspace would be
 * larger than the array (about 1,400 tokens of the Qwen3-30B-A3B shapes) is
 * refused with MOE_ERR_WORKSPACE before anything is launched. The array of
 * the current device is used (the stream must belong to it); it is looked up
 * on the first call on each device. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (different streams, or
 * threads) race and must be serialised by the caller. Nothing in the array
 * needs to start at zero (every call writes what it reads first), so what a
 * previous call left there is harmless. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
MOE_API moe_status moe_layer_noalloc(const moe_problem* p, const float* logits,
                                     const void* x, const void* residual,
                                     const void* w13, const void* w13_scale,
                                     const void* w2, const void* w2_scale,
                                     void* out, void* stream);

/* ---------------------------------------------------------------------
 * Upstream fused norm ([P1] "融合算子优化"): the residual add, the RMSNorm in
 * front of the MoE block and the conversion of its output in one pass, so
 * that neither the sum nor the normalised rows are written and read back
 * between operators.
 *
 *   s[t]            = x[t] + residual[t]  (fp32 add of the bf16 inputs;
 *                                           s = x when residual is NULL, the
 *                                           first layer)
 *   residual_out[t] = bf16(s[t])            (the new residual stream)
 *   y[t]            = s[t] / sqrt(mean(s[t]^2) + epsilon) * norm_weight
 *                     ([P1] "RmsNorm算子优化": LayerNorm without the mean)
 *
 * x, residual, residual_out: bf16 [T, H]; norm_weight: bf16 [H]. residual
 * and residual_out may be NULL (residual_out is then not written). T >= 0
 * (T == 0 launches nothing), H % 32 == 0 and H <= 8192 (else
 * MOE_ERR_UNSUPPORTED), epsilon finite and >= 0 (else MOE_ERR_INVALID_ARG).
 * The mean of squares is accumulated in fp32.
 */

/* "融合RMSNorm Cast": y in fp32 [T, H] (for the router) and in bf16 [T, H]
 * (for the experts), each rounded to nearest even from the fp32 value. Either
 * output may be NULL (not written), not both. */
MOE_API moe_status moe_add_rms_norm_cast(int32_t T, int32_t H, const void* x,
                                         const void* residual,
                                         const void* norm_weight, float epsilon,
                                         float* y_f32, void* y_bf16,
                                         void* residual_out, void* stream);

/* "融合RMSNorm MX量化": y as MXFP8 -- e4m3fn codes [T, H], rounded to nearest
 * even ("rint") and saturating at 448, with one e8m0 scale per 32 consecutive
 * columns [T, H/32] (OCP MX v1.0: floor(log2(amax)) - 8, clamped; an
 * all-zero block gets code 0): the layout of moe_init_routing's MXFP8
 * x_perm. */
MOE_API moe_status moe_add_rms_norm_mx_quant(int32_t T, int32_t H,
                                             const void* x,
                                             const void* residual,
                                             const void* norm_weight,
                                             float epsilon, uint8_t* y_codes,
                                             uint8_t* y_scales,
                                             void* residual_out, void* stream);

/* Packs static quantised expert weights -- the W8A8 int8 experts ([P3]
 * "量化策略": int8 weights with fixed per-channel scales) and the MXFP4
 * experts of W4A8 ([P1] "MoE EP优化 / AllGather方案(W4A8量化)"), both prepared
 * once -- into the packed order described above: src = W [E, N, K_bytes]
 * row-major bytes, dst = the same E * N * K_bytes bytes packed; dst must not
 * overlap src. E >= 0 (E == 0 launches nothing), N > 0, K_bytes > 0 (else
 * MOE_ERR_INVALID_ARG); N % 16 == 0, K_bytes % 64 == 0,
 * N * K_bytes < 2^31 (else MOE_ERR_UNSUPPORTED); pointers 16-byte aligned.
 * Stream-ordered; the caller owns both buffers. */
MOE_API moe_status moe_pack_weights(int32_t E, int32_t N, int32_t K_bytes,
                                    const void* src, void* dst, void* stream);

/* Packs static bf16 expert weights into the slab order described above
 * (moe_problem.wt_layout = MOE_LAYOUT_PACKED with BF16 weights); [P2]
 * "LongCat-Flash inference on Atlas A3 clusters": the decode grouped matmuls
 * are bound by streaming the expert weights, which the slab order makes
 * contiguous.
 *   src  bf16 [E, K, N] row-major (w13 [E_loc, H, 2I] with glu = 1, w2
 *        [E_loc, I, H] with glu = 0)
 *   dst  the same E * K * N bf16 values in the slab order; must not overlap
 *        src
 * glu = 1 pairs gate column 128 j + c with up column N/2 + 128 j + c in slab
 * j; glu = 0 takes 256 consecutive columns per slab. E >= 0 (E == 0
 * launches nothing), K > 0, N > 0, glu 0 or 1 (else MOE_ERR_INVALID_ARG);
 * K % 32 == 0, N % 256 == 0 and E * K * N < 2^40 (else
 * MOE_ERR_UNSUPPORTED); pointers 16-byte aligned. Stream-ordered; the
 * caller owns both buffers. */
MOE_API moe_status moe_pack_bf16_weights(int32_t E, int32_t K, int32_t N,
                                         int32_t glu, const void* src,
                                         void* dst, void* stream);

/* MXFP4 quantisation of bf16 expert weights, the form the W4A8 experts hold
 * ([P1] "MoE EP优化 / AllGather方案(W4A8量化)": MXFP4 weights), for a caller
 * that has bf16 weights; done once, e.g. when the weights are loaded. The
 * encoding is OCP MX v1.0 (the pages name MXFP4 without defining it): each
 * block of 32 consecutive K of one output column shares an e8m0 scale 2^s,
 * s = floor(log2(amax of the block)) - 2 clamped to [-127, 127] (an all-zero
 * block gets scale code 0); each element is the e2m1 code of v / 2^s rounded
 * to nearest, ties to even, saturating at 6, sign kept.
 *   w      bf16 [E, K, N], N contiguous (w13 [E, H, 2I] with K = H, N = 2I;
 *          w2 [E, I, H] with K = I, N = H)
 *   codes  uint8 [E, N, K/2]: K contiguous per output column, two codes per
 *          byte, the low nibble holds the even k -- the row-major MXFP4
 *          layout; moe_pack_weights turns it into the packed order
 *   scales uint8 [E, N, K/32] e8m0 (the w13_scale / w2_scale of moe_layer)
 * E >= 0 (E == 0 launches nothing), K > 0, N > 0 (else MOE_ERR_INVALID_ARG);
 * K % 32 == 0 and E * N * K < 2^40 (else MOE_ERR_UNSUPPORTED); pointers
 * 16-byte aligned. Stream-ordered; the caller owns all buffers. */
MOE_API moe_status moe_quant_mxfp4_weights(int32_t E, int32_t K, int32_t N,
                                           const void* w, uint8_t* codes,
                                           uint8_t* scales, void* stream);

/* Router linear ([P1] "融合算子优化 / 融合RMSNorm Cast": the fp32 output of
 * the norm is the input of the gate computation): the logits of
 * moe_gate_topk,
 *   logits[t, e] = sum_h y[t, h] * w_router[e, h]   (fp32 accumulation)
 * y: fp32 [T, H] (the y_f32 output of moe_add_rms_norm_cast); w_router: fp32
 * [E, H] (one row per expert, the layout of a linear layer's weight, no
 * bias); logits: fp32 [T, E]. T >= 0 (T == 0 launches nothing), H > 0,
 * E > 0 (else MOE_ERR_INVALID_ARG); H % 16 == 0, E % 32 == 0, E <= 2048
 * (else MOE_ERR_UNSUPPORTED). */
MOE_API moe_status moe_router_logits(int32_t T, int32_t H, int32_t E,
                                     const float* y, const float* w_router,
                                     float* logits, void* stream);

/* Static strings; never NULL. */
MOE_API const char* moe_status_string(moe_status s);
/* Library ABI version (major * 100 + minor). */
MOE_API int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
