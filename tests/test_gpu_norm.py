"""GPU parity of the fused residual add + RMSNorm (dual cast / MXFP8) against
the CPU oracle, through the C ABI.

Bars: the new residual is bit-exact (an fp32 add of two bf16 values rounded
to bf16 is the same on both sides); y in fp32 within rel 1e-5 per element of
the exact y (fp32 sum of squares, one division, one square root). The bf16
and MXFP8 outputs are taken of the fp32 y on both sides, so wherever the
GPU's fp32 y (from the dual-output call on the same inputs; both calls form
y with the same code) equals the oracle's fp32 rounding of the exact y, the
bf16 values and, block by block, the MX codes and scales must be bit-exact.
Elsewhere -- elements or blocks whose fp32 y differs by rounding, reported
as a count -- the bf16 value is the rounding of the GPU's own fp32 y, and the
MX codes decode to within the MX rounding bound of the exact y (half an e4m3
step at the block scale, or the saturation error past 448) with scales
within one."""
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


def _bits16(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).view(torch.int16).numpy()


def _check_cast(inp, eps, y32, y16, res):
    ry32, ry16, rres = O.add_rms_norm_cast(_host(inp["x"]), _host(inp["residual"]),
                                           _host(inp["weight"]), eps)
    y, _ = O.add_rms_norm(_host(inp["x"]), _host(inp["residual"]),
                          _host(inp["weight"]), eps)
    assert np.array_equal(res.view(torch.int16).cpu().numpy(), _bits16(rres))
    g32 = y32.double().cpu().numpy()
    assert np.all(np.abs(g32 - y) <= 1e-5 * np.abs(y) + 1e-30)
    g16 = y16.view(torch.int16).cpu().numpy()
    same = g32 == ry32
    assert np.array_equal(g16[same], _bits16(ry16)[same])
    # where the fp32 values differ, bf16 is the rounding of the GPU's own y
    assert np.array_equal(g16, y32.cpu().to(torch.bfloat16).view(torch.int16).numpy())
    print(f"  cast: fp32 y equal to the oracle's in {same.mean():.6f} of "
          f"{same.size} elements", flush=True)


def _check_mx(inp, eps, codes, scales, res, y32):
    rc, rs, rres, ry32 = O.add_rms_norm_mx_quant(_host(inp["x"]), _host(inp["residual"]),
                                                 _host(inp["weight"]), eps)
    y, _ = O.add_rms_norm(_host(inp["x"]), _host(inp["residual"]),
                          _host(inp["weight"]), eps)
    assert np.array_equal(res.view(torch.int16).cpu().numpy(), _bits16(rres))
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    T, H = y.shape
    g32 = y32.double().cpu().numpy()
    blk_same = (g32 == ry32).reshape(T, H // 32, 32).all(axis=2)
    # bit-exact codes and scales in every block whose fp32 y agrees
    el_same = np.repeat(blk_same, 32, axis=1)
    assert np.array_equal(gs[blk_same], rs[blk_same])
    assert np.array_equal(gc[el_same], rc[el_same])
    # the other blocks: scales within one, codes within the MX rounding bound
    ds = gs.astype(np.int64) - rs.astype(np.int64)
    assert np.all(np.abs(ds) <= 1)
    sc = np.repeat(np.ldexp(1.0, gs.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(y) / sc
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)
    bound = np.where(a > 448, a - 448, 0.5 * ulp) * sc
    deq = O.mx_dequant(gc, gs, "e4m3")
    assert np.all(np.abs(deq - y) <= bound * (1 + 1e-5) + 1e-6 * np.abs(y))
    print(f"  mx: {int((~blk_same).sum())} of {blk_same.size} blocks with an fp32 "
          f"y differing from the oracle's; {int((gc != rc).sum())} codes differ there",
          flush=True)


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
    y32, _, _ = m.add_rms_norm_cast(inp["x"], inp["residual"], inp["weight"],
                                    NORM_EPS, want_bf16=False, want_residual=False)
    torch.cuda.synchronize()
    _check_mx(inp, NORM_EPS, codes, scales, res, y32)


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
    _check_mx(inp, NORM_EPS, codes, scales, res2, y32)


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
        _check_mx(inp, eps, codes, scales, res2, y32)
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
