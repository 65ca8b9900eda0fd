"""Seeded random layer shapes on the GPU against the oracle.

The parity cases of test_gpu_parity.py are chosen by hand, one per kernel
path. Here each case draws its configuration (dtype, batch regime, H, I,
FFN and identity expert counts, top-k, expert range, residual, skewed
logits) from a seeded generator within the library's documented limits, so
the switches between kernels (weight-streaming 16- and 32-row tiles,
128- and 256-row LDS tiles, single- and multi-block routing, the gate-fused
quantisation) are crossed at sizes nobody picked. Every case must meet the
layer tolerances of the hand-picked ones."""
import numpy as np
import pytest
import torch

from moe_inputs import get_workload
from _moe_util import assert_close, generate, layer_ref, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 60

# base workload of each kind (dtypes), and the multiples H and I must keep
_KINDS = {
    "f32": ("tiny_fp32", 32, 32),
    "bf16": ("qwen3_30b_a3b_prefill_skewed_bf16", 32, 32),
    "bf16_packed": ("qwen3_30b_a3b_prefill_skewed_bf16", 256, 128),
    "w4a8": ("qwen3_235b_a22b_ep_rank_w4a8", 128, 128),
    "w8a8": ("qwen3_30b_a3b_prefill_skewed_w8a8", 128, 128),
}


def _case(i):
    """(shape, packed bf16 weights?) of case i."""
    rng = np.random.default_rng(7000 + i)
    kind = list(_KINDS)[i % len(_KINDS)]
    base, hq, iq = _KINDS[kind]
    H = hq * int(rng.integers(1, 768 // hq + 1))
    I = iq * int(rng.integers(1, 384 // iq + 1))
    # decode-, mid- and prefill-size batches (rows per expert ~ T k / E),
    # and long prefills on a few experts (256-row LDS tiles from an average
    # of 512 rows per expert)
    regime = int(rng.integers(0, 4))
    if regime < 3:
        n_ffn = int(rng.integers(1, 33))
        n_zero = int(rng.integers(1, 9)) if rng.random() < 0.3 else 0
        T = int(rng.integers(*((1, 17), (17, 160), (160, 700))[regime]))
    else:
        n_ffn, n_zero = int(rng.integers(1, 5)), 0
        T = int(rng.integers(600, 1300))
    E = n_ffn + n_zero
    k = int(rng.integers(1, min(E, 8) + 1))
    if rng.random() < 0.5:
        lb, le = 0, E
    else:
        lb = int(rng.integers(0, E))
        le = int(rng.integers(lb + 1, E + 1))
    shape = get_workload(base).replace(
        name=f"random_shape_{i}", T=T, H=H, I=I, n_ffn=n_ffn, n_zero=n_zero,
        top_k=k, local_begin=lb, local_end=le,
        residual=bool(rng.random() < 0.5),
        logit_bias_std=1.5 if rng.random() < 0.5 else 0.0)
    return shape, kind == "bf16_packed"


@pytest.mark.parametrize("i", range(N_CASES))
def test_layer_random_shape(i):
    import moe_expert_layer_gate_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    shape, packed = _case(i)
    print(f"case {i}: {shape} packed={packed}", flush=True)
    inp = generate(shape, seed=i, device=DEV)
    w13, w2, kw = inp["w13"], inp["w2"], {}
    if packed:
        # the layer reads the slab order; the oracle keeps the row-major
        # tensors in inp
        w13 = m.pack_bf16_weights(w13, glu=True)
        w2 = m.pack_bf16_weights(w2, glu=False)
        kw["wt_layout"] = "packed"
    out = m.layer(m.problem(shape, **kw), inp["logits"], inp["x"], w13, w2,
                  inp["w13_scale"], inp["w2_scale"], residual=inp["residual"])
    torch.cuda.synchronize()
    ref, allow = layer_ref(m, shape, inp)
    assert_close(to64(out), ref, shape, f"random case {i}", allow=allow)
