"""GPU parity of the fp32 router linear (logits = y @ w_router^T) against the
CPU oracle, through the C ABI.

Bar: fp32 accumulation of H products. Every logit is within 1e-5 of the sum
of the magnitudes of its products (an fp32 dot product of length H <= 8192
errs by far less), and the whole output within rel-L2 1e-5 (the fp32
tolerance of the layer)."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import generate_router
from _moe_util import rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (T, H, E): ragged token counts, the Qwen3-MoE (2048 x 128) and LongCat
# (6144 x 768) router shapes, short and long rows
SHAPES = [(1, 64, 32), (37, 2048, 128), (16, 16, 32), (100, 512, 64),
          (33, 6144, 768), (5, 8192, 2048)]
FULL = [(4096, 2048, 128), (32, 2048, 128), (1024, 6144, 768)]


def _m():
    import moe_expert_layer_gate_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    return m


def _check(y, w, got):
    yh, wh = y.double().cpu().numpy(), w.double().cpu().numpy()
    ref = O.router_logits(yh, wh)
    bound = np.abs(yh) @ np.abs(wh).T
    g = got.double().cpu().numpy()
    assert g.shape == ref.shape
    assert np.all(np.abs(g - ref) <= 1e-5 * bound + 1e-30)
    assert rel_l2(g, ref) <= 1e-5


@pytest.mark.parametrize("T,H,E", SHAPES)
def test_router_logits_shapes(T, H, E):
    m = _m()
    inp = generate_router(T, H, E, seed=1, device=DEV)
    out = m.router_logits(inp["y"], inp["w"])
    torch.cuda.synchronize()
    _check(inp["y"], inp["w"], out)


@pytest.mark.parametrize("T,H,E", FULL)
def test_router_logits_full_size(T, H, E):
    m = _m()
    print("router", T, H, E, flush=True)
    inp = generate_router(T, H, E, seed=0, device=DEV)
    out = m.router_logits(inp["y"], inp["w"])
    torch.cuda.synchronize()
    _check(inp["y"], inp["w"], out)


def test_router_one_hot_rows_pick_columns():
    # expert rows that are one-hot copy a column of y exactly
    m = _m()
    T, H, E = 40, 256, 32
    y = generate_router(T, H, E, seed=2, device=DEV)["y"]
    w = torch.zeros((E, H), dtype=torch.float32)
    cols = (np.arange(E) * 7) % H
    w[np.arange(E), cols] = 1.0
    out = m.router_logits(y, w.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), y.cpu()[:, torch.from_numpy(cols)])


def test_router_zero_tokens_launch_nothing():
    m = _m()
    y = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    w = torch.ones((32, 64), dtype=torch.float32, device=DEV)
    out = m.router_logits(y, w)
    torch.cuda.synchronize()
    assert out.shape == (0, 32)


def test_norm_router_gate_chain():
    # fused norm (fp32 output) -> router -> gate on the device, against the
    # oracle chain
    from moe_inputs import NORM_EPS, generate_norm
    m = _m()
    T, H, E, k = 64, 2048, 128, 8
    nin = generate_norm(T, H, seed=3, device=DEV)
    w = generate_router(T, H, E, seed=3, device=DEV)["w"]
    y32, _, _ = m.add_rms_norm_cast(nin["x"], nin["residual"], nin["weight"],
                                    NORM_EPS, want_bf16=False, want_residual=False)
    logits = m.router_logits(y32, w)
    p = m.problem(T=T, H=H, I=32, n_ffn=E, n_zero=0, top_k=k, local_begin=0,
                  local_end=E, act="bf16", wt="bf16", act_q="none")
    ids, wts = m.gate_topk(p, logits)
    torch.cuda.synchronize()
    ry32, _, _ = O.add_rms_norm_cast(nin["x"].double().cpu().numpy(),
                                     nin["residual"].double().cpu().numpy(),
                                     nin["weight"].double().cpu().numpy(), NORM_EPS)
    rl = O.router_logits(ry32, w.double().cpu().numpy())
    rid, _ = O.gate_topk(rl.astype(np.float32), k)
    # tokens whose k+1 largest logits are all more than 1e-4 apart (the
    # selection and the order of the k slots cannot flip on fp32 rounding)
    srt = np.sort(rl, axis=1)[:, ::-1]
    clear = np.min(srt[:, :k] - srt[:, 1:k + 1], axis=1) > 1e-4
    assert clear.mean() > 0.9
    assert np.array_equal(ids.cpu().numpy()[clear], rid[clear])
    assert np.allclose(wts.sum(1).cpu().numpy(), 1.0, atol=1e-6)
