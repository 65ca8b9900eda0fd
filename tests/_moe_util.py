"""Shared helpers of the tests: oracle calls on the exact tensors the GPU path
consumes, and the parity tolerances."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs
import oracle as O


def generate(shape, *args, **kwargs):
    """The seeded inputs of moe_inputs.generate, in the form the library
    takes on a GPU: int8 expert weights packed by the library's own pack
    call; W4A8 expert weights (drawn in bf16) quantised to MXFP4 by the
    library's weight-quantisation call and then packed. The originals stay
    for the oracle under "w13_rowmajor" / "w2_rowmajor" (int8 codes) or
    "w13_bf16" / "w2_bf16" (W4A8: the oracle quantises them itself)."""
    inp = moe_inputs.generate(shape, *args, **kwargs)
    w13 = inp.get("w13")
    if w13 is None or not w13.is_cuda:
        return inp
    if shape.wt in ("int8", "mxfp4"):
        import moe_expert_layer_gate_amd as m
        for k in ("w13", "w2"):
            if shape.wt == "mxfp4":
                inp[k + "_bf16"] = inp[k]
                codes, scales = m.quant_mxfp4_weights(inp[k])
                inp[k + "_scale"] = scales
                inp[k] = m.pack_weights(codes)
            else:
                inp[k + "_rowmajor"] = inp[k]
                inp[k] = m.pack_weights(inp[k])
    return inp


def to64(t):
    return None if t is None else t.detach().double().cpu().numpy()


class _MxWeightCache:
    """The oracle's MXFP4 quantisation of bf16 expert weights, dequantised to
    fp64 and kept per (tensor, expert): W4A8 checks on full-size experts
    would otherwise quantise the same weights once per test."""

    def __init__(self, cap=40):
        self.cap, self.d = cap, {}

    def get(self, w13b, w2b, i):
        key = (id(w13b), id(w2b), i)
        hit = self.d.get(key)
        if hit is not None:
            return hit[2]
        if len(self.d) >= self.cap:
            self.d.pop(next(iter(self.d)))
        # [H, 2I] -> quantise the K = H blocks of each output column
        a = to64(w13b[i]).T
        c, sc = O.mx_quant(a, "e2m1")
        A = O.mx_dequant(c, sc, "e2m1").T.copy()
        b = to64(w2b[i]).T
        c, sc = O.mx_quant(b, "e2m1")
        B = O.mx_dequant(c, sc, "e2m1").T.copy()
        self.d[key] = (w13b, w2b, (A, B))   # the tensors pin the ids
        return A, B


MX_WEIGHTS = _MxWeightCache()


def weight_getter(shape, inp):
    """Lazy per-expert fp64 weights from (possibly device-resident) tensors."""
    fb = shape.ffn_begin
    if shape.wt == "mxfp4":
        w13b = inp.get("w13_bf16", inp["w13"])
        w2b = inp.get("w2_bf16", inp["w2"])

        def get(e):
            return MX_WEIGHTS.get(w13b, w2b, e - fb)
        return get
    if shape.wt == "int8":
        w13, w2 = inp.get("w13_rowmajor", inp["w13"]), inp.get("w2_rowmajor", inp["w2"])
        s13, s2 = inp["w13_scale"], inp["w2_scale"]

        def get(e):
            i = e - fb
            a = O.int8_dequant_rows(w13[i].cpu().numpy(), s13[i].cpu().numpy())
            b = O.int8_dequant_rows(w2[i].cpu().numpy(), s2[i].cpu().numpy())
            return a.T.copy(), b.T.copy()   # [H, 2I], [I, H]
        return get
    w13, w2 = inp["w13"], inp["w2"]

    def get(e):
        i = e - fb
        return to64(w13[i]), to64(w2[i])
    return get


def oracle_kwargs(shape, inp):
    return dict(logits=inp["logits"].cpu().numpy(), x=to64(inp["x"]),
                residual=to64(inp["residual"]),
                get_weights=weight_getter(shape, inp), T=shape.T, H=shape.H,
                I=shape.I, n_ffn=shape.n_ffn, n_zero=shape.n_zero,
                top_k=shape.top_k, local_begin=shape.local_begin,
                local_end=shape.local_end, act=shape.act, act_q=shape.act_q)


def layer_ref(m, shape, inp, toks=None, residual=True):
    """The oracle's layer output for all tokens (toks=None) or for the tokens
    `toks` (the routed oracle on that subset: every step is row-local), and
    the allowance of assert_close: None unless h is quantised; then the GPU's
    h codes are taken through the library's split calls on the full problem
    (gate, routing, GEMM1: the kernels moe_layer runs, bit for bit), checked
    for validity row by row against the oracle's, and their effect on y is
    carried through the weighted sum of finalize."""
    kw = oracle_kwargs(shape, inp)
    if not residual:
        kw["residual"] = None
    idx = np.arange(shape.T) if toks is None else np.asarray(toks)
    if toks is not None:
        kw["logits"] = kw["logits"][idx]
        kw["x"] = kw["x"][idx]
        if kw["residual"] is not None:
            kw["residual"] = kw["residual"][idx]
        kw["T"] = len(idx)
    ref = O.moe_layer(**kw)
    if shape.act_q not in ("mxfp8", "int8") or ref["R"] == 0:
        return ref["out"], None
    p = m.problem(shape)
    ids, _ = m.gate_topk(p, inp["logits"])
    r = m.init_routing(p, ids, inp["x"])
    h, hs = m.ffn_up(p, r["offsets"], r["x_perm"], r["x_perm_scale"], inp["w13"],
                     inp["w13_scale"])
    torch.cuda.synchronize()
    fb, fe, k = shape.ffn_begin, shape.ffn_end, shape.top_k
    cp_g = r["copy_pos"].cpu().numpy().astype(np.int64)
    r0_g = int(r["offsets"][fb])
    ids_s, cp_s, r0_s = ref["topk_ids"], ref["copy_pos"], ref["row0"]
    gpu_row = np.zeros(ref["R"], dtype=np.int64)
    for ts, t in enumerate(idx):
        for j in range(k):
            if fb <= ids_s[ts, j] < fe:
                gpu_row[cp_s[ts * k + j] - r0_s] = cp_g[t * k + j] - r0_g
    sel = torch.from_numpy(gpu_row).to(h.device)
    gh, ghs = h[sel].cpu().numpy(), hs[sel].cpu().numpy()
    A_y = quant_h_allowance(shape, ref["x_perm"], gh, ghs, ref["h_codes"],
                            ref["h_scale"], ref["offsets"], r0_s,
                            np.arange(ref["R"]), kw["get_weights"])
    A = np.zeros((len(idx), shape.H))
    w = ref["topk_weight"]
    for ts in range(len(idx)):
        for j in range(k):
            if fb <= ids_s[ts, j] < fe:
                A[ts] += abs(w[ts, j]) * A_y[cp_s[ts * k + j] - r0_s]
    return ref["out"], A


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (d if d > 0 else 1.0)


def bf16_ulp(v):
    """Unit in the last place of bf16 at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, np.finfo(np.float64).tiny)))
    return np.exp2(np.maximum(e, -126.0) - 7.0)


def assert_close(got, ref, shape, what="", allow=None):
    """Tolerances of the layer, as stated: fp32 rel-L2 <= 1e-5; bf16 and
    quantised outputs rel-L2 <= 1e-2 and max|got - ref| <= 5e-2 * RMS(ref).

    allow (same shape, or None): extra room per element for outputs that
    depend on an intermediate quantisation decision (the MXFP8 / int8 codes
    of h) which the GPU, summing in another order, took the other valid way;
    it comes from quant_h_allowance, which checks first that every such code
    is a valid rounding. Returns the statistics (rel-L2, max-abs / RMS, how
    many elements sit exactly one bf16 ulp from the reference -- two correct
    sums that straddle a rounding boundary -- and how many needed `allow`)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    if shape.act == "f32" and shape.wt == "f32":
        assert r <= 1e-5, f"{what}: rel_l2 {r:.3e} > 1e-5"
        return dict(rel_l2=r)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.abs(got - ref)
    mx = float(np.max(err)) if ref.size else 0.0
    one_ulp = int(np.count_nonzero(err == bf16_ulp(ref))) if ref.size else 0
    over = err > 5e-2 * rms
    stats = dict(rel_l2=r, max_abs_over_rms=mx / rms if rms else 0.0,
                 one_ulp=one_ulp, n=int(ref.size), allowed=int(over.sum()))
    print(f"  {what}: rel_l2 {r:.2e}, max_abs/rms {stats['max_abs_over_rms']:.3e}, "
          f"one-ulp straddles {one_ulp} of {ref.size}, beyond the bound by a "
          f"differing h code: {stats['allowed']}", flush=True)
    assert r <= 1e-2, f"{what}: rel_l2 {r:.3e} > 1e-2"
    if allow is None:
        assert mx <= 5e-2 * rms, f"{what}: max_abs {mx:.3e} > 5e-2*rms {rms:.3e}"
    else:
        allow = np.asarray(allow, dtype=np.float64)
        bad = err > 5e-2 * rms + allow
        assert not bad.any(), (
            f"{what}: {int(bad.sum())} elements beyond 5e-2*rms {rms:.3e} plus "
            f"the h-code allowance; worst {float(np.max(err - allow)):.3e}")
    return stats


def h_error_bound(shape, a, w13):
    """The exact fp32-rounded h of rows `a` (GEMM1 input values) and a bound
    on how far an fp32 evaluation of it may land from that: the standard
    bound of a K-term fp32 dot product, |fl(sum) - sum| <= K 2^-24 sum |a w|
    (int8: the integer sums are exact, only the two scale products round),
    carried through SwiGLU to first order, plus 16 fp32 ulps of h for the
    activation's exp, reciprocal and products."""
    a = np.asarray(a, dtype=np.float64)
    I = w13.shape[1] // 2
    gu = a @ w13
    ga = np.abs(a) @ np.abs(w13)
    g, u = gu[:, :I], gu[:, I:]
    if shape.act_q == "int8":
        dg, du = 2.0 ** -22 * np.abs(g), 2.0 ** -22 * np.abs(u)
    else:
        eps = w13.shape[0] * 2.0 ** -24
        dg, du = eps * ga[:, :I], eps * ga[:, I:]
    sig = 1.0 / (1.0 + np.exp(-g))
    h = g * sig * u
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    tol = dsilu * dg * np.abs(u) + np.abs(g * sig) * du + dg * du + 2.0 ** -20 * np.abs(h)
    return O.round_f32(h), tol


def check_quant_h(shape, v32, tol, gc, gs, rc, rs):
    """The GPU's codes of h against the oracle's, for rows whose fp32 h the
    oracle gives as v32, with tol the error bound of an fp32 evaluation of
    h (h_error_bound): every GPU code must decode to within half a
    quantisation step plus tol of v32 -- the correct rounding of some value
    the GPU's fp32 arithmetic may have reached -- MX scales may differ by one
    only where the block maximum lies within tol of a power of two, int8 row
    scales only by what tol allows at the row maximum, and differing codes
    must be rare (the caller counts them over all rows: assert_rare_codes).
    Returns (GPU dequantised h, oracle dequantised h, differing codes)."""
    v32 = np.asarray(v32, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    if shape.act_q == "mxfp8":
        gd, rd = O.mx_dequant(gc, gs, "e4m3"), O.mx_dequant(rc, rs, "e4m3")
        ds = gs.astype(np.int64) - rs.astype(np.int64)
        assert np.all(np.abs(ds) <= 1)
        n, I = v32.shape
        vb, tb = np.abs(v32).reshape(n, I // 32, 32), tol.reshape(n, I // 32, 32)
        amax = vb.max(axis=2)
        amax_tol = np.take_along_axis(tb, vb.argmax(axis=2)[..., None], 2)[..., 0]
        p2 = np.exp2(np.round(np.log2(np.maximum(amax, 1e-300))))
        near2 = np.abs(amax - p2) <= amax_tol + 2.0 ** -23 * amax
        assert np.all(near2[ds != 0]), "an MX scale differs away from a power of two"
        same = np.repeat(ds == 0, 32, axis=1)
        sc = np.repeat(np.ldexp(1.0, gs.astype(np.int64) - 127), 32, axis=1)
        a = np.maximum(np.abs(v32), np.abs(gd)) / sc
        step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(a, 1e-300))), -6) - 3) * sc
        sat = (np.abs(v32) + tol) / sc > 448
        ok = (np.abs(gd - v32) <= 0.5 * step + tol) | sat | ~same
        assert ok.all(), f"{int((~ok).sum())} MXFP8 h codes are no valid rounding"
        frac = float(np.mean(gc != rc))
    else:
        gd = gc.astype(np.float64) * gs.astype(np.float64)[:, None]
        rd = rc.astype(np.float64) * rs.astype(np.float64)[:, None]
        amax_tol = np.take_along_axis(tol, np.abs(v32).argmax(axis=1)[:, None], 1)[:, 0]
        ds = np.abs(gs.astype(np.float64) - rs.astype(np.float64))
        assert np.all(ds <= amax_tol / 127 + 2.0 ** -22 * np.abs(rs)), "int8 row scales"
        step = gs.astype(np.float64)[:, None]
        ok = np.abs(gd - v32) <= 0.5 * step * (1 + 2.0 ** -20) + tol + 1e-30
        assert ok.all(), f"{int((~ok).sum())} int8 h codes are no valid rounding"
        frac = float(np.mean(gc != rc))
    return gd, rd, int(round(frac * gd.size))


def assert_rare_codes(ndiff, n):
    """Differing h codes come from values within fp32 noise of a rounding
    midpoint: a handful, not a share of the codes."""
    print(f"  h codes: {ndiff} of {n} differ from the oracle's (each a valid "
          f"rounding)", flush=True)
    assert ndiff <= 1e-3 * n + 4, f"{ndiff} of {n} h codes differ"


def quant_h_allowance(shape, a_rows, gh, ghs, ref_h_codes, ref_h_scale,
                      offsets, r0, rows, get_weights):
    """The y allowance of the rows `rows` (indices into the R local rows,
    expert-sorted) from differing h codes: |h_gpu - h_oracle| @ |W2_e| per
    expert, after check_quant_h has shown every GPU code valid. a_rows are
    the oracle's GEMM1 input values of those rows; gh / ghs the GPU's codes
    and scales of the same rows; ref_h_* the oracle's."""
    rows = np.asarray(rows)
    A = np.zeros((len(rows), shape.H))
    if not len(rows):
        return A
    # expert of each row
    fb, fe = shape.ffn_begin, shape.ffn_end
    bounds = np.asarray(offsets[fb:fe + 1], dtype=np.int64) - r0
    ex = np.searchsorted(bounds, rows, side="right") - 1 + fb
    ndiff = 0
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        w13, w2 = get_weights(int(e))
        v32, tol = h_error_bound(shape, a_rows[sel], w13)
        gd, rd, nd = check_quant_h(shape, v32, tol, gh[sel], ghs[sel],
                                   ref_h_codes[sel], ref_h_scale[sel])
        ndiff += nd
        dh = np.abs(gd - rd)
        hit = dh.any(axis=1)
        if hit.any():
            A[sel[hit]] = dh[hit] @ np.abs(w2)
    assert_rare_codes(ndiff, len(rows) * shape.I)
    return A


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a tensor (for bit-exact comparisons)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def np_to_act_bits(v: np.ndarray, act: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v))
    return bits(t.to(torch.float32 if act == "f32" else torch.bfloat16))
