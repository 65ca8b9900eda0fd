"""moe_layer_noalloc through the C ABI: the layer with the library's static
per-GPU scratch as its workspace. On two calls in a row -- the second with a
smaller input, over what the first left in the scratch -- its output must be
moe_layer's bit for bit (same kernels, same launch sequence), and a problem
whose workspace exceeds the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from moe_inputs import get_workload, scaled
from _moe_util import bits, generate

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = {
    # (shape of the first call, tokens of the second, smaller call)
    "decode_bf16_full": (get_workload("qwen3_30b_a3b_decode_bf16"), 8),
    "decode_bf16": (scaled(get_workload("qwen3_30b_a3b_decode_bf16"), T=64,
                           H=512, I=384, n_ffn=16, local_end=16, top_k=4), 16),
    "prefill_bf16": (scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                            T=600, H=384, I=160, n_ffn=8, local_end=8,
                            top_k=4), 150),
    "ep_w4a8": (scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"), T=512,
                       H=1024, I=512, n_ffn=8, local_begin=2, local_end=6,
                       top_k=4), 100),
    "decode_w8a8": (scaled(get_workload("qwen3_30b_a3b_decode_w8a8"), T=32,
                           H=512, I=384, n_ffn=16, local_end=16, top_k=4), 8),
    "zero_experts": (scaled(get_workload("longcat_flash_zero_experts_bf16"),
                            T=64, H=512, I=256, n_ffn=24, n_zero=12,
                            local_end=36, top_k=6), 20),
    "tiny_fp32": (get_workload("tiny_fp32"), 5),
}


def _m():
    import moe_expert_layer_gate_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    return m


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_layer_on_two_calls(name):
    m = _m()
    shape, t2 = CASES[name]
    print("noalloc", name, flush=True)
    for T in (shape.T, t2):
        sh = shape.replace(T=T)
        inp = generate(sh, seed=T, device=DEV)
        p = m.problem(sh)
        assert m.layer_workspace_bytes(p) <= m.NOALLOC_SCRATCH_BYTES
        want = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                       inp["w13_scale"], inp["w2_scale"], residual=inp["residual"])
        got = m.layer_noalloc(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                              inp["w13_scale"], inp["w2_scale"],
                              residual=inp["residual"])
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(want)), (name, T)


def test_noalloc_packed_bf16_weights():
    """The slab-packed bf16 layout through the static scratch: equal to
    moe_layer on row-major weights, on two calls in a row (the second
    smaller)."""
    m = _m()
    shape = scaled(get_workload("longcat_flash_zero_experts_bf16"), T=64,
                   H=512, I=256, n_ffn=24, n_zero=12, local_end=36, top_k=6)
    print("noalloc packed bf16", flush=True)
    for T in (shape.T, 20):
        sh = shape.replace(T=T)
        inp = generate(sh, seed=T + 1, device=DEV)
        want = m.layer(m.problem(sh), inp["logits"], inp["x"], inp["w13"],
                       inp["w2"], residual=inp["residual"])
        w13p = m.pack_bf16_weights(inp["w13"], glu=True)
        w2p = m.pack_bf16_weights(inp["w2"], glu=False)
        got = m.layer_noalloc(m.problem(sh, wt_layout="packed"), inp["logits"],
                              inp["x"], w13p, w2p, residual=inp["residual"])
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(want)), T


def test_noalloc_refuses_problems_past_the_scratch():
    m = _m()
    shape = get_workload("qwen3_30b_a3b_prefill_skewed_bf16")  # T = 4096
    p = m.problem(shape)
    assert m.layer_workspace_bytes(p) > m.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: refused on the host
    st = m.lib().moe_layer_noalloc(ctypes.byref(p), fake, fake, fake, fake, None,
                                   fake, None, fake, None)
    assert st == 3
    # the scratch still serves the next call
    small = shape.replace(T=16)
    inp = generate(small, seed=3, device=DEV)
    ps = m.problem(small)
    want = m.layer(ps, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                   residual=inp["residual"])
    got = m.layer_noalloc(ps, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                          residual=inp["residual"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(want))
