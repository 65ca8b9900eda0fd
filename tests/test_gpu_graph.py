"""The layer under HIP graph capture: the library enqueues kernels only (no
allocation, no memset, no host synchronisation), so one captured moe_layer
call replays as the whole layer. Each replay runs on new inputs copied into
the captured buffers, with eager work and synchronisations in between, and
must give exactly the eager result on those inputs."""
import numpy as np
import pytest
import torch

from moe_inputs import get_workload, scaled
from _moe_util import generate
from _moe_util import bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = {
    "decode_bf16": scaled(get_workload("qwen3_30b_a3b_decode_bf16"), T=32,
                          H=512, I=384, n_ffn=16, local_end=16, top_k=4),
    "prefill_bf16": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                           T=600, H=384, I=160, n_ffn=8, local_end=8, top_k=4),
    "ep_w4a8": scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"), T=512,
                      H=1024, I=512, n_ffn=8, local_begin=2, local_end=6,
                      top_k=4),
    "decode_w8a8": scaled(get_workload("qwen3_30b_a3b_decode_w8a8"), T=32,
                          H=512, I=384, n_ffn=16, local_end=16, top_k=4),
}


def _m():
    import moe_expert_layer_gate_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    return m


@pytest.mark.parametrize("name", list(CASES))
def test_layer_graph_replays_match_eager(name):
    m = _m()
    shape = CASES[name]
    print("graph", name, flush=True)
    p = m.problem(shape)
    inp = generate(shape, seed=0, device=DEV)
    ws = torch.empty(max(m.layer_workspace_bytes(p), 1), dtype=torch.uint8, device=DEV)
    dt = torch.bfloat16
    out = torch.empty((shape.T, shape.H), dtype=dt, device=DEV)
    # captured buffers for the per-step inputs
    logits = inp["logits"].clone()
    x = inp["x"].clone()
    res = None if inp["residual"] is None else inp["residual"].clone()

    def call():
        m.layer(p, logits, x, inp["w13"], inp["w2"], inp["w13_scale"],
                inp["w2_scale"], residual=res, out=out, workspace=ws)

    call()  # warm the library and the allocator outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        new = generate(shape, seed=seed, device=DEV, weights=False)
        logits.copy_(new["logits"])
        x.copy_(new["x"])
        if res is not None:
            res.copy_(new["residual"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        # eager on the same inputs (fresh output and workspace)
        want = m.layer(p, logits, x, inp["w13"], inp["w2"], inp["w13_scale"],
                       inp["w2_scale"], residual=res)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(want)), (name, seed)
