"""GPU parity of the fused residual add + RMSNorm (dual cast / MXFP8) against
the CPU oracle, through the C ABI.

Bars: the new residual is bit-exact (an fp32 add of two bf16 values rounded
to bf16 is the same on both sides); y in fp32 within rel 1e-5 per element
(fp32 sum of squares, one division, one square root); y in bf16 within one
bf16 ulp of the exact value; MXFP8: every code decodes to within the MX
rounding bound of the exact y (half an e4m3 step at the block scale, or the
saturation error past 448), scale codes equal unless the block maximum sits
within fp32 noise of a power of two, and codes equal the oracle's own for all
but a sliver of elements that sit on a rounding midpoint."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import NORM_EPS, generate_norm
from _moe_util import bf16_ulp

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SHAPES = [(1, 32), (7, 96), (33, 384), (64, 2048), (5, 6144), (3, 8192), (130, 512)]
FULL = [(4096, 2048), (4096, 4096), (1024, 6144)]


def _m():
    import moe_expert_layer_gate_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    return m


def _host(t):
    return None if t is None else t.double().cpu().numpy()


def _check_cast(inp, eps, y32, y16, res):
    ry32, ry16, rres = O.add_rms_norm_cast(_host(inp["x"]), _host(inp["residual"]),
                                           _host(inp["weight"]), eps)
    y, _ = O.add_rms_norm(_host(inp["x"]), _host(inp["residual"]),
                          _host(inp["weight"]), eps)
    assert np.array_equal(res.view(torch.int16).cpu().numpy(),
                          torch.from_numpy(rres).to(torch.bfloat16).view(torch.int16).numpy())
    g32 = y32.double().cpu().numpy()
    assert np.all(np.abs(g32 - y) <= 1e-5 * np.abs(y) + 1e-30)
    g16 = y16.double().cpu().numpy()
    assert np.all(np.abs(g16 - y) <= bf16_ulp(y))


def _check_mx(inp, eps, codes, scales, res):
    rc, rs, rres, y = O.add_rms_norm_mx_quant(_host(inp["x"]), _host(inp["residual"]),
                                              _host(inp["weight"]), eps)
    assert np.array_equal(res.view(torch.int16).cpu().numpy(),
                          torch.from_numpy(rres).to(torch.bfloat16).view(torch.int16).numpy())
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    T, H = y.shape
    # scale codes: equal unless the block max is within fp32 noise of 2^n
    amax = np.abs(y).reshape(T, H // 32, 32).max(axis=2)
    frac = np.log2(np.maximum(amax, 1e-300))
    near = np.abs(frac - np.round(frac)) < 1e-5
    ds = gs.astype(np.int64) - rs.astype(np.int64)
    assert np.all(ds[~near] == 0) and np.all(np.abs(ds[near]) <= 1)
    # every decoded value within the MX rounding bound of the exact y
    sc = np.repeat(np.ldexp(1.0, gs.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(y) / sc
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)
    bound = np.where(a > 448, a - 448, 0.5 * ulp) * sc
    deq = O.mx_dequant(gc, gs, "e4m3")
    assert np.all(np.abs(deq - y) <= bound * (1 + 1e-5) + 1e-6 * np.abs(y))
    # and the codes are the oracle's own nearly everywhere
    same = gc == rc
    assert same.mean() >= 0.999, f"{(~same).sum()} of {same.size} codes differ"


@pytest.mark.parametrize("with_res", [True, False])
@pytest.mark.parametrize("T,H", SHAPES)
def test_add_rms_norm_cast(T, H, with_res):
    m = _m()
    inp = generate_norm(T, H, seed=T + H, device=DEV, residual=with_res)
    y32, y16, res = m.add_rms_norm_cast(inp["x"], inp["residual"], inp["weight"], NORM_EPS)
    torch.cuda.synchronize()
    _check_cast(inp, NORM_EPS, y32, y16, res)


@pytest.mark.parametrize("with_res", [True, False])
@pytest.mark.parametrize("T,H", SHAPES)
def test_add_rms_norm_mx_quant(T, H, with_res):
    m = _m()
    inp = generate_norm(T, H, seed=T * H, device=DEV, residual=with_res)
    codes, scales, res = m.add_rms_norm_mx_quant(inp["x"], inp["residual"],
                                                 inp["weight"], NORM_EPS)
    torch.cuda.synchronize()
    _check_mx(inp, NORM_EPS, codes, scales, res)


@pytest.mark.parametrize("T,H", FULL)
def test_add_rms_norm_full_size(T, H):
    m = _m()
    print("norm full", T, H, flush=True)
    inp = generate_norm(T, H, seed=1, device=DEV)
    y32, y16, res = m.add_rms_norm_cast(inp["x"], inp["residual"], inp["weight"], NORM_EPS)
    codes, scales, res2 = m.add_rms_norm_mx_quant(inp["x"], inp["residual"],
                                                  inp["weight"], NORM_EPS)
    torch.cuda.synchronize()
    _check_cast(inp, NORM_EPS, y32, y16, res)
    _check_mx(inp, NORM_EPS, codes, scales, res2)


def test_add_rms_norm_edges():
    m = _m()
    # zero rows (y = +-0 with the weight's sign; MX block all zero -> code 0),
    # a tiny and a huge row, a negative weight, large epsilon
    T, H = 6, 256
    inp = generate_norm(T, H, seed=9, device=DEV)
    inp["x"][0] = 0
    inp["residual"][0] = 0
    inp["x"][1] *= 1e-30
    inp["residual"][1] *= 1e-30
    inp["x"][2] *= 1e15
    inp["weight"][::7] *= -1
    for eps in (NORM_EPS, 0.5):
        y32, y16, res = m.add_rms_norm_cast(inp["x"], inp["residual"], inp["weight"], eps)
        codes, scales, res2 = m.add_rms_norm_mx_quant(inp["x"], inp["residual"],
                                                      inp["weight"], eps)
        torch.cuda.synchronize()
        _check_cast(inp, eps, y32, y16, res)
        _check_mx(inp, eps, codes, scales, res2)
        assert int(scales[0].abs().sum()) == 0
    # only one of the dual outputs; no residual output
    y32, y16, res = m.add_rms_norm_cast(inp["x"], inp["residual"], inp["weight"],
                                        NORM_EPS, want_bf16=False, want_residual=False)
    torch.cuda.synchronize()
    assert y16 is None and res is None
    ref32, _, _ = O.add_rms_norm_cast(_host(inp["x"]), _host(inp["residual"]),
                                      _host(inp["weight"]), NORM_EPS)
    assert np.all(np.abs(y32.double().cpu().numpy() - ref32) <= 1e-5 * np.abs(ref32) + 1e-30)
    # no rows
    e = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    y32, y16, res = m.add_rms_norm_cast(e, None, inp["weight"], NORM_EPS)
    torch.cuda.synchronize()
    assert y32.shape == (0, H)
