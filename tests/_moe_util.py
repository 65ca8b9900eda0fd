"""Shared helpers of the tests: oracle calls on the exact tensors the GPU path
consumes, and the parity tolerances."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs
import oracle as O


def generate(shape, *args, **kwargs):
    """The seeded inputs of moe_inputs.generate; quantised (int8, MXFP4)
    expert weights on a GPU are handed to the library packed (the form its
    int8 and MX GEMMs take, made by the library's own pack call), and the
    row-major originals stay under "w13_rowmajor" / "w2_rowmajor" for the
    oracle."""
    inp = moe_inputs.generate(shape, *args, **kwargs)
    w13 = inp.get("w13")
    if shape.wt in ("int8", "mxfp4") and w13 is not None and w13.is_cuda:
        import moe_expert_layer_gate_amd as m
        for k in ("w13", "w2"):
            inp[k + "_rowmajor"] = inp[k]
            inp[k] = m.pack_weights(inp[k])
    return inp


def to64(t):
    return None if t is None else t.detach().double().cpu().numpy()


def weight_getter(shape, inp):
    """Lazy per-expert fp64 weights from (possibly device-resident) tensors."""
    fb = shape.ffn_begin
    if shape.wt == "mxfp4":
        w13, w2 = inp.get("w13_rowmajor", inp["w13"]), inp.get("w2_rowmajor", inp["w2"])
        s13, s2 = inp["w13_scale"], inp["w2_scale"]

        def get(e):
            i = e - fb
            a = O.mxfp4_dequant_rows(w13[i].cpu().numpy(), s13[i].cpu().numpy())
            b = O.mxfp4_dequant_rows(w2[i].cpu().numpy(), s2[i].cpu().numpy())
            return a.T.copy(), b.T.copy()   # [H, 2I], [I, H]
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


def assert_close(got, ref, shape, what=""):
    """Tolerances of the layer: fp32 rel-L2 <= 1e-5; bf16 and quantised
    rel-L2 <= 1e-2 and max-abs <= 5e-2 * RMS(ref).

    A bf16 output is the rounding of an fp32 (GPU) or fp64 (oracle) sum; two
    correct sums that straddle a rounding boundary land one bf16 ulp apart,
    which for a rare large output (heavy-tailed MXFP4 weights give outputs
    past 20x the RMS) exceeds 5e-2 * RMS by itself. The max-abs bound is
    therefore applied to the part of each element's error beyond one bf16
    ulp of the reference value; rel-L2 sees the whole error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    if shape.act == "f32" and shape.wt == "f32":
        assert r <= 1e-5, f"{what}: rel_l2 {r:.3e} > 1e-5"
        return r
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    excess = np.maximum(np.abs(got - ref) - bf16_ulp(ref), 0.0)
    mx = np.max(excess) if ref.size else 0.0
    assert r <= 1e-2, f"{what}: rel_l2 {r:.3e} > 1e-2"
    assert mx <= 5e-2 * rms + 1e-30, (
        f"{what}: max_abs beyond one bf16 ulp {mx:.3e} > 5e-2*rms {rms:.3e}")
    return r


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
