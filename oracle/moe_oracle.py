"""Float64 CPU oracle of the MoE expert layer (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this module. It is deliberately plain: numpy float64, one expert at a time,
library primitives (stable argsort, bincount, matmul, exp) as single steps and
no blocking, fusion or reordering beyond what the definitions state.

Sources (web pages; cited by title and section):
  [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters"
       (cann-recipes-infer practice article)
  [P2] "LongCat-Flash inference on Atlas A3 clusters"
  [P3] "NPU Qwen3-Next inference practice" (cann-recipes-infer practice
       article; only its quantisation strategy section is used)
  OCP Microscaling Formats (MX) v1.0 specification for the MX element/scale
  encodings, which the pages use by name (MXFP8 / MXFP4) without defining.

What each function follows:
  gate_topk        [P1] "GMM使能和Routing优化 / 快速选择专家": fused top-k + softmax
                   router scores; [P2] "MoE模块 / Router": sort router output and
                   take the top-k experts.
  init_routing     [P1] "高效排序和token路由": sort token copies by expert
                   (init_routing) and count tokens per expert
                   (compute_expert_tokens).
  swiglu, expert_ffn
                   [P1] "MoE TP优化 / 计算分解": expert = down(SiLU(gate(x)) * up(x));
                   gate and up merged into one w13 matmul; swiglu splits the last
                   axis in two halves and returns SiLU(first) * second.
  finalize         [P1] "高效排序和token路由" (finalize_routing: restore token order
                   and take the weighted sum); [P2] "MoE模块 / Decode阶段优化":
                   zero-compute experts return their input, MoE(x) = x.
  mx_quant_*       [P1] "MoE EP优化 / AllGather方案(W4A8量化)": dynamic MX quant of
                   hidden states before routing; [P1] "融合算子优化 / 融合RMSNorm MX
                   量化": round_mode "rint", dst float8_e4m3fn; OCP MX v1.0 for
                   block size 32, e8m0 scale = floor(log2(amax)) - emax_elem.
  router_logits    [P1] "融合算子优化 / 融合RMSNorm Cast": the fp32 output of the
                   norm feeds the gate (router) computation; the router is a
                   linear map without bias to one logit per expert.
  int8_quant_rows, int8_dequant_rows
                   [P3] "量化策略": routed experts in W8A8 -- weights int8 with a
                   static scale per output channel, activations int8 with a
                   dynamic scale per token (per row).
  rms_norm, add_rms_norm_cast, add_rms_norm_mx_quant
                   [P1] "融合算子优化": the residual add, RMSNorm and the output
                   conversion fused into one operator -- dual output (fp32 for
                   the router, bf16 for the experts, "融合RMSNorm Cast") or
                   dynamic MXFP8 with round mode "rint" to float8_e4m3fn
                   ("融合RMSNorm MX量化"; without a residual on the first layer);
                   [P1] "RmsNorm算子优化": RMSNorm is LayerNorm without the mean
                   subtraction, i.e. s / sqrt(mean(s^2) + eps) * weight.
  local expert range
                   [P1] "MoE EP优化 / AllGather方案": routing keeps only the copies
                   whose expert lies in this rank's range; finalize of a rank gives
                   a partial sum that a later reduce-scatter adds up.

Readings taken where the pages are silent:
  * top-k order: descending logit, ties to the lower expert id; weights are the
    softmax over the k selected logits (equal in exact arithmetic to a softmax
    over all experts followed by renormalising the k selected).
  * stable permutation key: (expert id, flat copy index t*k + j).
  * identity experts have ids [n_ffn, n_ffn + n_zero); a call's range
    [local_begin, local_end) is over all E_tot ids; copies outside it add 0.
  * fused norm: the residual add is an fp32 add of the two bf16 inputs; the
    RMSNorm is taken of that fp32 sum (not of its bf16 rounding), exactly; the
    new residual is the sum rounded to bf16; the outputs are the fp32 rounding
    of the exact y, and the bf16 rounding and MXFP8 quantisation of that fp32
    value.
  * intermediates are stored in the activation dtype (bf16 or fp32) between
    the two GEMMs, or as MXFP8 / int8 when activations are quantised (the
    fp32-rounded h is quantised); y is stored in the activation dtype;
    finalize sums in high precision and rounds once.
  * W8A8: symmetric int8 codes in [-127, 127]; a row's scale is its amax / 127
    in fp32 and its codes are rint(v / scale) in fp32 (ties to even); an
    all-zero row has scale 0 and codes 0. Weights arrive already quantised
    (codes + one fp32 scale per output channel). x is quantised once per
    token before routing and gathered; h per row (token copy).

Parity status: every function here is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "round_bf16", "round_f32", "round_to",
    "gate_topk", "init_routing",
    "e4m3_decode", "e4m3_encode", "e2m1_decode", "e2m1_encode",
    "e8m0_decode", "mx_scale_code", "mx_quant", "mx_dequant",
    "mxfp4_unpack", "mxfp4_dequant_rows",
    "int8_quant_rows", "int8_dequant_rows",
    "silu", "swiglu", "expert_ffn", "moe_layer", "moe_tokens", "moe_dense",
    "rms_norm", "add_rms_norm", "add_rms_norm_cast", "add_rms_norm_mx_quant",
    "router_logits",
]

# --------------------------------------------------------------------------
# Rounding of fp64 values to storage formats (round to nearest, ties to even)
# --------------------------------------------------------------------------


def _round_to_precision(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round to a binary float with `mant_bits` stored mantissa bits and minimum
    normal exponent `min_exp` (no overflow handling), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                         # |x| = m * 2^e, m in [0.5, 1)
    exp = np.maximum(e - 1, min_exp)           # floor(log2|x|), clamped
    ulp = np.ldexp(1.0, exp - mant_bits)
    return np.round(x / ulp) * ulp             # np.round: half to even; 0 -> 0


def round_bf16(x) -> np.ndarray:
    """fp64 -> nearest bfloat16 value (8-bit exponent, 7 stored mantissa bits)."""
    return _round_to_precision(x, 7, -126)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Gate: top-k over router logits, softmax over the selected logits
# --------------------------------------------------------------------------


def gate_topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per token, the k experts with the largest logits (ties -> lower id), in
    descending order, and their renormalised softmax weights.

    [P1] "快速选择专家": the fused gating op replaces "topk then softmax".
    Selection compares the given fp32 logits exactly; weights are
    exp(l_j - l_max) / sum_j exp(l_j - l_max) over the k selected, in fp64.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must be in [1, E]")
    # stable sort on -logit keeps equal logits in ascending expert order
    order = np.argsort(-L, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    p = np.exp(sel - sel[:, :1])
    w = p / p.sum(axis=1, keepdims=True)
    return ids, w


# --------------------------------------------------------------------------
# Routing: expert histogram, offsets, stable permutation and its inverse
# --------------------------------------------------------------------------


def init_routing(topk_ids: np.ndarray, n_experts: int):
    """[P1] "高效排序和token路由".

    Copies are numbered c = t*k + j. Returns
      counts[e]      = number of copies routed to expert e
      offsets        = exclusive prefix sum of counts, offsets[E] = T*k
      sorted_copy[i] = copy at sorted position i, sorted by (expert, c)
      copy_pos[c]    = sorted position of copy c (inverse permutation)
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= n_experts):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_copy = np.argsort(flat, kind="stable").astype(np.int64)
    copy_pos = np.empty_like(sorted_copy)
    copy_pos[sorted_copy] = np.arange(flat.size)
    return counts, offsets, sorted_copy, copy_pos


# --------------------------------------------------------------------------
# MX formats (OCP MX v1.0): e4m3fn and e2m1 elements, e8m0 block scales
# --------------------------------------------------------------------------

_FMT = {
    # name: (stored mantissa bits, exponent bias, max finite, emax of element)
    "e4m3": (3, 7, 448.0, 8),
    "e2m1": (1, 1, 6.0, 2),
}


def _elem_decode(codes, fmt):
    m_bits, bias, _, _ = _FMT[fmt]
    e_bits = {"e4m3": 4, "e2m1": 2}[fmt]
    codes = np.asarray(codes, dtype=np.int64)
    sign = (codes >> (m_bits + e_bits)) & 1
    ex = (codes >> m_bits) & ((1 << e_bits) - 1)
    man = codes & ((1 << m_bits) - 1)
    mag = np.where(ex == 0,
                   np.ldexp(man / (1 << m_bits), 1 - bias),
                   np.ldexp(1.0 + man / (1 << m_bits), ex - bias))
    val = np.where(sign == 1, -mag, mag)
    if fmt == "e4m3":  # e4m3fn: exponent and mantissa all ones is NaN
        val = np.where((ex == 15) & (man == 7), np.nan, val)
    return val


def _elem_encode(v, fmt):
    """Round fp64 values to the element format: nearest, ties to even,
    saturating at the largest finite magnitude; the sign is kept, so values
    that round to zero encode as +0 or -0."""
    m_bits, bias, vmax, _ = _FMT[fmt]
    e_bits = {"e4m3": 4, "e2m1": 2}[fmt]
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    min_normal_exp = 1 - bias
    r = np.minimum(_round_to_precision(a, m_bits, min_normal_exp), vmax)
    # normal values: biased exponent and the stored mantissa bits
    _, e = np.frexp(r)
    ex = np.maximum(e - 1, min_normal_exp)
    man = np.round((r / np.ldexp(1.0, ex) - 1.0) * (1 << m_bits)).astype(np.int64)
    normal_code = ((ex + bias) << m_bits) | man
    # subnormal values (and zero): multiples of the smallest subnormal step
    sub_code = np.round(r / np.ldexp(1.0, min_normal_exp - m_bits)).astype(np.int64)
    code = np.where(r >= np.ldexp(1.0, min_normal_exp), normal_code, sub_code)
    code |= sign << (m_bits + e_bits)
    return code.astype(np.uint8)


def e4m3_decode(codes):
    return _elem_decode(codes, "e4m3")


def e4m3_encode(v):
    return _elem_encode(v, "e4m3")


def e2m1_decode(codes):
    return _elem_decode(np.asarray(codes) & 0xF, "e2m1")


def e2m1_encode(v):
    return _elem_encode(v, "e2m1")


def e8m0_decode(codes):
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mx_scale_code(amax, fmt: str):
    """e8m0 code of the shared block scale: floor(log2(amax)) - emax_elem,
    clamped to [-127, 127], biased by 127. An all-zero block gets code 0."""
    emax = _FMT[fmt][3]
    amax = np.asarray(amax, dtype=np.float64)
    code = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, e = np.frexp(amax[nz])
    s = np.clip((e - 1) - emax, -127, 127)
    code[nz] = s + 127
    return code.astype(np.uint8)


def mx_quant(v: np.ndarray, fmt: str = "e4m3", block: int = 32):
    """Blockwise MX quantisation along the last axis.

    Returns (element codes uint8 [..., K], scale codes uint8 [..., K/block]).
    Element = encode(v / 2^s) with s the block's shared exponent."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % block:
        raise ValueError("last axis must be a multiple of the block size")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.abs(vb).max(axis=-1)
    sc = mx_scale_code(amax, fmt)
    scaled = vb / np.ldexp(1.0, sc.astype(np.int64) - 127)[..., None]
    codes = _elem_encode(scaled, fmt).reshape(v.shape)
    return codes, sc


def mx_dequant(codes: np.ndarray, scales: np.ndarray, fmt: str = "e4m3",
               block: int = 32) -> np.ndarray:
    codes = np.asarray(codes)
    K = codes.shape[-1]
    vals = _elem_decode(codes, fmt).reshape(codes.shape[:-1] + (K // block, block))
    out = vals * e8m0_decode(scales)[..., None]
    return out.reshape(codes.shape)


def mxfp4_unpack(packed: np.ndarray) -> np.ndarray:
    """Two e2m1 codes per byte along the last axis; the low nibble holds the
    even element. [..., K/2] bytes -> [..., K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_dequant_rows(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 weight matrix [N, K/2] + scales [N, K/32] -> fp64 [N, K]."""
    return mx_dequant(mxfp4_unpack(packed), scales, "e2m1")


# --------------------------------------------------------------------------
# W8A8: symmetric int8 with one fp32 scale per row ([P3] "量化策略")
# --------------------------------------------------------------------------


def int8_quant_rows(v):
    """Dynamic per-row (per-token) int8 quantisation along the last axis.

    The values must be fp32 numbers (bf16 x, or h after its fp32 rounding).
    Per row: amax = max |v|; scale = amax / 127 rounded to fp32; code =
    rint(v / scale) with the division rounded to fp32 and rint taking ties to
    even, clipped to [-127, 127]. An all-zero row gets scale 0 and codes 0.
    Returns (codes int8 [..., K], scales float32 [...])."""
    v64 = np.asarray(v, dtype=np.float64)
    v32 = v64.astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), v64):
        raise ValueError("int8_quant_rows takes fp32 values")
    amax = np.abs(v32).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    nz = scale > 0
    div = np.where(nz, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(v32 / div[..., None])            # fp32 quotient, half to even
    q = np.clip(q, -127, 127)
    q = np.where(nz[..., None], q, 0.0)
    return q.astype(np.int8), scale


def int8_dequant_rows(codes, scales) -> np.ndarray:
    """codes [..., K] * scales[...] per row, exact in fp64. For weights the
    rows are output channels ([N, K] codes, [N] scales)."""
    return (np.asarray(codes, dtype=np.float64)
            * np.asarray(scales, dtype=np.float64)[..., None])


# --------------------------------------------------------------------------
# Expert FFN: down(SiLU(gate(x)) * up(x)) with merged w13
# --------------------------------------------------------------------------


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gu: np.ndarray) -> np.ndarray:
    """Split the last axis into two halves; SiLU(first half) * second half."""
    n = gu.shape[-1]
    if n % 2:
        raise ValueError("last axis must be even")
    g, u = gu[..., : n // 2], gu[..., n // 2:]
    return silu(g) * u


def _act_rows(xrows: np.ndarray, act_q: str):
    """Activation values entering GEMM1 (and their MX codes when quantised)."""
    if act_q == "mxfp8":
        codes, sc = mx_quant(xrows, "e4m3")
        return mx_dequant(codes, sc, "e4m3"), (codes, sc)
    if act_q == "int8":
        codes, sc = int8_quant_rows(xrows)
        return int8_dequant_rows(codes, sc), (codes, sc)
    return np.asarray(xrows, dtype=np.float64), None


def expert_ffn(a: np.ndarray, w13: np.ndarray, w2: np.ndarray, *,
               act: str, act_q: str = "none", exact: bool = False):
    """One expert on activation rows a [n, H] (already the GEMM1 input values).

    w13: fp64 [H, 2I] (columns [0, I) gate, [I, 2I) up); w2: fp64 [I, H].
    Storage roundings (bf16 / fp32) between the steps follow the activation
    format unless `exact`; quantisation of h (act_q "mxfp8" or "int8") is part
    of the computed function and is applied either way, to the fp32-rounded h
    (int8 takes fp32 values, so it rounds even when `exact`).
    Returns (h, h_codes, y)."""
    gu = a @ w13
    h = swiglu(gu)
    h_codes = None
    if act_q == "mxfp8":
        codes, sc = mx_quant(h if exact else round_f32(h), "e4m3")
        h_codes = (codes, sc)
        h = mx_dequant(codes, sc, "e4m3")
    elif act_q == "int8":
        codes, sc = int8_quant_rows(round_f32(h))
        h_codes = (codes, sc)
        h = int8_dequant_rows(codes, sc)
    elif not exact:
        h = round_to(h, act)
    y = h @ w2
    if not exact:
        y = round_to(y, act)
    return h, h_codes, y


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------


def _check_problem(T, H, I, n_ffn, n_zero, top_k, local_begin, local_end):
    E = n_ffn + n_zero
    if min(T, H, I) < 0 or n_ffn < 0 or n_zero < 0 or E < 1:
        raise ValueError("bad sizes")
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E_tot]")
    if not 0 <= local_begin < local_end <= E:
        raise ValueError("bad local range")


WeightFn = Callable[[int], Tuple[np.ndarray, np.ndarray]]


def moe_layer(*, logits, x, get_weights: WeightFn, T, H, I, n_ffn, n_zero,
              top_k, local_begin, local_end, act, act_q="none",
              residual=None, exact=False) -> Dict[str, np.ndarray]:
    """Routed evaluation: gate -> routing -> per-expert FFN -> finalize.

    get_weights(e) returns the fp64 (w13 [H,2I], w2 [I,H]) of FFN expert e.
    Returns every intermediate: topk ids/weights, counts, offsets,
    sorted_copy, copy_pos, x_perm (values, and codes when quantised), h, y,
    out (rounded to the activation dtype unless exact)."""
    _check_problem(T, H, I, n_ffn, n_zero, top_k, local_begin, local_end)
    E = n_ffn + n_zero
    x = np.asarray(x, dtype=np.float64)
    ids, w = gate_topk(logits, top_k)
    counts, offsets, sorted_copy, copy_pos = init_routing(ids, E)
    fb, fe = min(local_begin, n_ffn), min(local_end, n_ffn)
    r0, r1 = int(offsets[fb]), int(offsets[fe])
    R = r1 - r0
    tok_of_row = sorted_copy[r0:r1] // top_k
    xrows = x[tok_of_row] if R else np.zeros((0, H))
    a, a_codes = _act_rows(xrows, act_q)
    h = np.zeros((R, I))
    y = np.zeros((R, H))
    if act_q == "int8":
        h_codes = (np.zeros((R, I), np.int8), np.zeros(R, np.float32))
    else:
        h_codes = (np.zeros((R, I), np.uint8),
                   np.zeros((R, I // 32 if I % 32 == 0 else 0), np.uint8))
    for e in range(fb, fe):
        lo, hi = int(offsets[e]) - r0, int(offsets[e + 1]) - r0
        if hi == lo:
            continue  # an expert with no rows is never evaluated
        w13, w2 = get_weights(e)
        he, hc, ye = expert_ffn(a[lo:hi], w13, w2, act=act, act_q=act_q, exact=exact)
        h[lo:hi], y[lo:hi] = he, ye
        if hc is not None:
            h_codes[0][lo:hi], h_codes[1][lo:hi] = hc
    out = finalize(ids=ids, w=w, copy_pos=copy_pos, row0=r0, y=y, x=x,
                   n_ffn=n_ffn, local_begin=local_begin, local_end=local_end,
                   residual=residual)
    if not exact:
        out = round_to(out, act)
    res = dict(topk_ids=ids, topk_weight=w, counts=counts, offsets=offsets,
               sorted_copy=sorted_copy, copy_pos=copy_pos, row0=r0, R=R,
               x_perm=a, h=h, y=y, out=out)
    if a_codes is not None:
        res["x_perm_codes"], res["x_perm_scale"] = a_codes
        res["h_codes"], res["h_scale"] = h_codes
    return res


def finalize(*, ids, w, copy_pos, row0, y, x, n_ffn, local_begin, local_end,
             residual=None) -> np.ndarray:
    """out[t] = residual[t] + sum_j w[t,j] * v(t,j), with
    v = y[copy_pos[t*k+j] - row0] for an FFN expert in the call's range,
    x[t] for an identity expert in the range, 0 for a copy outside the range.
    fp64 sum (no rounding here)."""
    T, k = ids.shape
    H = x.shape[1]
    out = np.zeros((T, H)) if residual is None else np.array(residual, dtype=np.float64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not local_begin <= e < local_end:
                continue
            if e >= n_ffn:
                out[t] += w[t, j] * x[t]
            else:
                out[t] += w[t, j] * y[int(copy_pos[t * k + j]) - row0]
    return out


def moe_tokens(tokens: Sequence[int], *, logits, x, get_weights: WeightFn, T, H,
               I, n_ffn, n_zero, top_k, local_begin, local_end, act,
               act_q="none", residual=None, exact=False,
               cache_weights=True) -> np.ndarray:
    """Brute-force per-token evaluation (no routing structures): for each token
    t in `tokens`, out[t] = residual[t] + sum_j w_j * FFN_{e_j}(x[t]) with the
    same storage roundings as moe_layer. Every step of the layer is row-local,
    so this equals the routed result row by row. Returns [len(tokens), H].
    cache_weights=False fetches an expert's weights anew for every use (for
    workloads whose fp64 weights do not fit in host memory)."""
    _check_problem(T, H, I, n_ffn, n_zero, top_k, local_begin, local_end)
    x = np.asarray(x, dtype=np.float64)
    L = np.asarray(logits)
    outs = []
    cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
    for t in tokens:
        ids, w = gate_topk(L[t:t + 1], top_k)
        acc = (np.zeros(H) if residual is None
               else np.array(residual[t], dtype=np.float64))
        for j in range(top_k):
            e = int(ids[0, j])
            if not local_begin <= e < local_end:
                continue
            if e >= n_ffn:
                acc = acc + w[0, j] * x[t]
                continue
            if e in cache:
                we = cache[e]
            else:
                we = get_weights(e)
                if cache_weights:
                    cache[e] = we
            a, _ = _act_rows(x[t:t + 1], act_q)
            _, _, ye = expert_ffn(a, *we, act=act, act_q=act_q, exact=exact)
            acc = acc + w[0, j] * ye[0]
        outs.append(acc if exact else round_to(acc, act))
    return np.stack(outs) if outs else np.zeros((0, H))


def moe_dense(*, logits, x, get_weights: WeightFn, T, H, I, n_ffn, n_zero,
              top_k, local_begin, local_end, residual=None) -> np.ndarray:
    """Dense masked form, exact fp64 (no storage roundings, no quantisation):
    out = residual + sum_e G[t,e] * F_e(x[t]) over all experts e in range, with
    G the top-k renormalised softmax scattered into a dense [T, E] matrix and
    F_e = identity for e >= n_ffn. For tiny problems only."""
    _check_problem(T, H, I, n_ffn, n_zero, top_k, local_begin, local_end)
    x = np.asarray(x, dtype=np.float64)
    E = n_ffn + n_zero
    ids, w = gate_topk(logits, top_k)
    G = np.zeros((T, E))
    np.put_along_axis(G, ids.astype(np.int64), w, axis=1)
    out = np.zeros((T, H)) if residual is None else np.array(residual, dtype=np.float64)
    for e in range(local_begin, local_end):
        if e >= n_ffn:
            out += G[:, e:e + 1] * x
        else:
            w13, w2 = get_weights(e)
            out += G[:, e:e + 1] * (swiglu(x @ w13) @ w2)
    return out


# --------------------------------------------------------------------------
# Upstream fused norm: residual add + RMSNorm + dual cast / dynamic MXFP8
# --------------------------------------------------------------------------


def rms_norm(s, weight, eps: float) -> np.ndarray:
    """RMSNorm along the last axis in fp64: s / sqrt(mean(s^2) + eps) * weight
    ([P1] "RmsNorm算子优化": LayerNorm without subtracting the mean)."""
    s = np.asarray(s, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(s * s, axis=-1, keepdims=True)
    return s / np.sqrt(ms + eps) * w


def add_rms_norm(x, residual, weight, eps: float):
    """Residual add then RMSNorm ([P1] "融合算子优化").

    x, residual: bf16 values (as fp64) [T, H]; residual may be None (first
    layer: the norm of x alone). The add is the fp32 sum of the two inputs;
    the norm is exact (fp64) from that sum. Returns (y fp64 [T, H],
    residual_out = the sum rounded to bf16)."""
    x = np.asarray(x, dtype=np.float64)
    if residual is None:
        s = x
    else:
        s = round_f32(x + np.asarray(residual, dtype=np.float64))
    return rms_norm(s, weight, eps), round_bf16(s)


def add_rms_norm_cast(x, residual, weight, eps: float):
    """[P1] "融合RMSNorm Cast": the normalised hidden states in fp32 (for the
    router) and in bf16 (for the experts), plus the new residual. The fp32
    output is the exact y rounded to fp32; the bf16 output is that fp32 value
    rounded to bf16 (the cast of the fp32 output, not of the exact y).
    Returns (y_f32, y_bf16, residual_out) as fp64 arrays of those values."""
    y, r = add_rms_norm(x, residual, weight, eps)
    y32 = round_f32(y)
    return y32, round_bf16(y32), r


def add_rms_norm_mx_quant(x, residual, weight, eps: float):
    """[P1] "融合RMSNorm MX量化": the normalised hidden states as MXFP8
    (e4m3 codes rounded to nearest even, e8m0 scale per 32 along H), plus the
    new residual. The codes quantise the fp32 value of y (the exact y rounded
    to fp32), as the dual-output form casts it. Returns (codes uint8 [T, H],
    scales uint8 [T, H/32], residual_out fp64, y_f32 the quantised values)."""
    y, r = add_rms_norm(x, residual, weight, eps)
    y32 = round_f32(y)
    codes, scales = mx_quant(y32, "e4m3")
    return codes, scales, r, y32


def router_logits(y, w_router) -> np.ndarray:
    """Router logits of the normalised hidden states, exact in fp64:
    logits[t, e] = sum_h y[t, h] * w_router[e, h].

    y: fp32 values [T, H] (the fp32 output of the fused norm); w_router: fp32
    values [E, H] (one row per expert, the layout of a linear layer's weight,
    no bias)."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    if y.ndim != 2 or w.ndim != 2 or y.shape[1] != w.shape[1]:
        raise ValueError("y [T, H] and w_router [E, H] expected")
    return y @ w.T
