"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Integer outputs (ids, counts, offsets, permutation, gathered rows and MX codes)
must be bit-exact; floating outputs meet the layer tolerances (fp32 rel-L2
<= 1e-5; bf16 / W4A8 rel-L2 <= 1e-2 and max-abs <= 5e-2 * RMS(ref)); router
weights within 1e-6."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import WORKLOADS, get_workload, scaled
from _moe_util import (assert_close, assert_rare_codes, bits, check_quant_h,
                       generate, h_error_bound,
                       layer_ref,
                       np_to_act_bits, oracle_kwargs, quant_h_allowance, to64,
                       weight_getter)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _m():
    import moe_expert_layer_gate_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    return m


def _say(*a):
    print(*a, flush=True)


# Small shapes of each workload: several tiles and ragged tails, fast oracle.
SMALL = {
    "tiny_fp32": get_workload("tiny_fp32"),
    "tiny_fp32_ragged": scaled(get_workload("tiny_fp32"), T=37, H=96, I=64,
                               n_ffn=5, local_end=5, top_k=3),
    "decode_bf16_small": scaled(get_workload("qwen3_30b_a3b_decode_bf16"), T=32,
                                H=512, I=384, n_ffn=16, local_end=16, top_k=4),
    "prefill_skewed_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                                   T=300, H=256, I=160, n_ffn=12, local_end=12,
                                   top_k=4),
    # many rows per expert: H = 384 leaves a ragged GEMM2 slab, I = 160 a
    # ragged GEMM1 slab
    "prefill_wide_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                                 T=600, H=384, I=160, n_ffn=8, local_end=8,
                                 top_k=4),
    "zero_experts_small": scaled(get_workload("longcat_flash_zero_experts_bf16"),
                                 T=64, H=512, I=256, n_ffn=24, n_zero=12,
                                 local_end=36, top_k=6),
    "ep_w4a8_small": scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"), T=200,
                            H=512, I=256, n_ffn=16, local_begin=4, local_end=8,
                            top_k=4),
    # enough rows per expert for the 128-row LDS-tiled scaled-MFMA kernel;
    # H = 384 leaves a ragged 256-column slab in GEMM2
    # K/32 a multiple of 16: scales copied four K steps at a time (GEMM1:
    # 8 steps = 2 batches, GEMM2: 4 steps = 1 batch)
    "ep_w4a8_wide_small": scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"),
                                 T=512, H=1024, I=512, n_ffn=8, local_begin=2,
                                 local_end=6, top_k=4),
    "ep_w4a8_prefill_small": scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"),
                                    T=384, H=384, I=256, n_ffn=16, local_begin=4,
                                    local_end=12, top_k=4),
    # W8A8: decode-size (weight-streaming kernel, 16-row tiles)
    "decode_w8a8_small": scaled(get_workload("qwen3_30b_a3b_decode_w8a8"), T=32,
                                H=512, I=384, n_ffn=16, local_end=16, top_k=4),
    # W8A8 prefill-size (128-row tiles): I = 384 gives three GEMM1 slabs,
    # H = 384 a ragged GEMM2 slab
    "prefill_w8a8_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_w8a8"),
                                 T=600, H=384, I=384, n_ffn=8, local_end=8,
                                 top_k=4),
    # W8A8 with about 100 rows per expert
    "prefill_w8a8_mid_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_w8a8"),
                                     T=300, H=256, I=256, n_ffn=12,
                                     local_end=12, top_k=4),
    # about 600 rows per expert: 256-row tiles, ragged last tiles, ragged
    # GEMM1 (I = 160) and GEMM2 (H = 384) slabs
    "prefill_long_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                                 T=1200, H=384, I=160, n_ffn=8, local_end=8,
                                 top_k=4),
    "prefill_w8a8_long_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_w8a8"),
                                      T=1200, H=384, I=384, n_ffn=8,
                                      local_end=8, top_k=4),
    # W8A8 with H = 2048: x quantised per token inside the gate kernel; 8
    # rows per expert (streaming GEMMs)
    "decode_w8a8_h2048_small": scaled(get_workload("qwen3_30b_a3b_decode_w8a8"),
                                      T=32, H=2048, I=256, n_ffn=16,
                                      local_end=16, top_k=4),
    # W4A8 with 320 experts (the gate launch takes no quantising blocks
    # above 256) and more than 4096 copies: x quantised beside the scan
    "ep_w4a8_320e_small": scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"),
                                 T=640, H=256, I=256, n_ffn=320, top_k=8,
                                 local_begin=64, local_end=96),
    # the same for W8A8 with 2048-wide rows (each lane keeps its 4 chunks of
    # 512 in registers)
    "ep_w8a8_320e_small": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_w8a8"),
                                 T=640, H=2048, I=256, n_ffn=320, top_k=8,
                                 local_begin=64, local_end=96),
    # W8A8 on an expert range, about 24 rows per expert: 128-row tiles
    "range_w8a8_small": scaled(get_workload("qwen3_30b_a3b_decode_w8a8"), T=96,
                               H=256, I=256, n_ffn=16, local_begin=4,
                               local_end=10, top_k=4),
    # W8A8 on an expert range, 8 rows per expert: 16-row streaming tiles
    "range_w8a8_stream_small": scaled(get_workload("qwen3_30b_a3b_decode_w8a8"),
                                      T=32, H=256, I=256, n_ffn=16,
                                      local_begin=4, local_end=10, top_k=4),
    # bf16 with 16 rows per expert: 32-row streaming tiles
    "decode_bf16_32row_small": scaled(get_workload("qwen3_30b_a3b_decode_bf16"),
                                      T=64, H=512, I=384, n_ffn=16,
                                      local_end=16, top_k=4),
    # W4A8 decode-size on an expert range, 6 rows per expert: mostly empty
    # 128-row scaled-MFMA tiles
    "ep_w4a8_decode_small": scaled(get_workload("qwen3_235b_a22b_ep_rank_w4a8"),
                                   T=24, H=512, I=256, n_ffn=16, local_begin=4,
                                   local_end=8, top_k=4),
}


def _oracle_layer(shape, inp, **kw):
    return O.moe_layer(**oracle_kwargs(shape, inp), **kw)


# ------------------------------------------------------------------ gate


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_gate_topk_full_size(name):
    m = _m()
    shape = get_workload(name)
    _say("gate", name)
    inp = generate(shape, seed=1, device=DEV, weights=False)
    ids, w = m.gate_topk(m.problem(shape), inp["logits"])
    torch.cuda.synchronize()
    rid, rw = O.gate_topk(inp["logits"].cpu().numpy(), shape.top_k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.max(np.abs(w.cpu().double().numpy() - rw)) <= 1e-6
    assert np.max(np.abs(w.cpu().double().numpy().sum(1) - 1.0)) <= 1e-6


@pytest.mark.parametrize("E,k", [(8, 2), (64, 64), (128, 8), (768, 12), (100, 7),
                                 (2048, 16), (1, 1)])
def test_gate_topk_ties(E, k):
    m = _m()
    g = torch.Generator().manual_seed(E * 7 + k)
    T = 203
    L = torch.randint(-2, 3, (T, E), generator=g).float()  # many ties
    L[0] = 0.0                                               # all tied
    L[1, ::2] = -0.0
    logits = L.to(DEV)
    p = m.problem(T=T, H=32, I=32, n_ffn=E, n_zero=0, top_k=k, local_begin=0,
                  local_end=E, act="bf16", wt="bf16", act_q="none")
    ids, w = m.gate_topk(p, logits)
    torch.cuda.synchronize()
    rid, rw = O.gate_topk(L.numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.max(np.abs(w.cpu().double().numpy() - rw)) <= 1e-6


# ------------------------------------------------------------------ routing


def _routing_case(shape, seed):
    m = _m()
    inp = generate(shape, seed=seed, device=DEV, weights=False)
    rid, _ = O.gate_topk(inp["logits"].cpu().numpy(), shape.top_k)
    ids = torch.from_numpy(rid).to(DEV)
    r = m.init_routing(m.problem(shape), ids, inp["x"])
    torch.cuda.synchronize()
    counts, offsets, sc, cp = O.init_routing(rid, shape.E_tot)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted_copy"].cpu().numpy(), sc)
    assert np.array_equal(r["copy_pos"].cpu().numpy(), cp)
    fb, fe = shape.ffn_begin, shape.ffn_end
    r0, r1 = int(offsets[fb]), int(offsets[fe])
    tok = sc[r0:r1] // shape.top_k
    x = inp["x"].cpu()
    if shape.act_q == "mxfp8":
        codes, scl = O.mx_quant(x.double().numpy()[tok], "e4m3")
        assert np.array_equal(r["x_perm"][: r1 - r0].cpu().numpy(), codes)
        assert np.array_equal(r["x_perm_scale"][: r1 - r0].cpu().numpy(), scl)
    elif shape.act_q == "int8":
        codes, scl = O.int8_quant_rows(x.double().numpy()[tok])
        assert np.array_equal(r["x_perm"][: r1 - r0].cpu().numpy(), codes)
        assert np.array_equal(bits(r["x_perm_scale"][: r1 - r0]), scl.view(np.int32))
    else:
        assert np.array_equal(bits(r["x_perm"][: r1 - r0]), bits(x[torch.from_numpy(tok)]))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_init_routing_full_size(name):
    _say("routing", name)
    _routing_case(get_workload(name), seed=2)


@pytest.mark.parametrize("name", list(SMALL))
def test_init_routing_small(name):
    _say("routing small", name)
    _routing_case(SMALL[name], seed=3)


def _mxfp8_edge_rows(T, H):
    """bf16 rows whose 32-value blocks sit on the edges of the MXFP8 (e4m3)
    encoding: with a block maximum of 1 the scale is 2^-8, so values below
    2^-14 land among the e4m3 subnormals (step 2^-17 before scaling) and the
    odd multiples of 2^-18 are exact ties between two of them; a maximum of
    1.96875 scales to 504 and saturates at 448, 1.0625 scales to 272, a tie
    between the normal codes 256 and 288; negative values and -0; an
    all-zero block."""
    tiny = [k * 2.0 ** -18 for k in range(1, 32, 2)]            # ties
    small = [k * 2.0 ** -17 for k in range(1, 9)]               # subnormals
    patterns = [
        [1.0] + tiny + [-v for v in tiny[:15]],
        [1.0] + small + [-v for v in small] + [2.0 ** -14, -2.0 ** -14] +
        [2.0 ** -15] * 5 + [-0.0] * 8,
        [1.96875, -1.96875, 1.875, 1.75] + [0.5, -0.25, 0.125] * 9 + [1.0],
        [1.0625, -1.0625, 1.0, 1.125] + [0.0] * 28,
        [0.0] * 32,
        [-0.0] * 31 + [2.0 ** -126],
    ]
    blocks = [np.array(b[:32] + [0.0] * (32 - len(b[:32])), dtype=np.float64)
              for b in patterns]
    rows = []
    for t in range(T):
        row = np.concatenate([blocks[(t + j) % len(blocks)] * (2.0 ** ((t % 5) - 2))
                              for j in range(H // 32)])
        rows.append(row)
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    assert np.array_equal(x.double().numpy(), np.stack(rows)), "edge values must be bf16"
    return x


def test_mxfp8_quant_edge_values():
    """MXFP8 codes and scales of x (the per-copy quantisation of the routing
    gather, the same row routine the gate-side and scan-side quantisers run)
    bit-exact against the oracle on values chosen at the encoding's edges:
    subnormal codes, ties to even, saturation, signed zeros, zero blocks."""
    m = _m()
    T, H, E, k = 40, 512, 16, 4
    g = torch.Generator().manual_seed(77)
    rid, _ = O.gate_topk(torch.randn(T, E, generator=g).numpy(), k)
    x = _mxfp8_edge_rows(T, H)
    p = m.problem(T=T, H=H, I=128, n_ffn=E, n_zero=0, top_k=k, local_begin=0,
                  local_end=E, act="bf16", wt="mxfp4", act_q="mxfp8")
    r = m.init_routing(p, torch.from_numpy(rid).to(DEV), x.to(DEV))
    torch.cuda.synchronize()
    counts, offsets, sc, cp = O.init_routing(rid, E)
    tok = sc // k
    codes, scl = O.mx_quant(x.double().numpy()[tok], "e4m3")
    got_c = r["x_perm"][: T * k].cpu().numpy()
    got_s = r["x_perm_scale"][: T * k].cpu().numpy()
    print("edge rows: code mismatches", int((got_c != codes).sum()),
          "scale mismatches", int((got_s != scl).sum()), flush=True)
    assert np.array_equal(got_c, codes)
    assert np.array_equal(got_s, scl)


@pytest.mark.parametrize("T,E,k", [(50, 2048, 2), (600, 2048, 64), (64, 1024, 64),
                                   (65, 1024, 64), (4096, 1, 1), (1000, 300, 7),
                                   (4096, 512, 32), (5000, 96, 1)])
def test_init_routing_max_sizes(T, E, k):
    """The largest expert count and top-k the library takes (2048 experts
    route through the count / scan / scatter kernels), both sides of the
    single-block routing limit of 4096 copies and 1024 experts (64 x 64
    copies is the last on the single-block side, 65 x 64 the first past it),
    and multi-block routing with a ragged last chunk and 300 experts, 512
    chunks with 512 experts, and one copy per token."""
    m = _m()
    g = torch.Generator().manual_seed(T * 31 + E + k)
    L = torch.randn(T, E, generator=g)
    rid, _ = O.gate_topk(L.numpy(), k)
    x = torch.randn(T, 64, generator=g).to(torch.bfloat16)
    p = m.problem(T=T, H=64, I=32, n_ffn=E, n_zero=0, top_k=k, local_begin=0,
                  local_end=E, act="bf16", wt="bf16", act_q="none")
    r = m.init_routing(p, torch.from_numpy(rid).to(DEV), x.to(DEV))
    torch.cuda.synchronize()
    counts, offsets, sc, cp = O.init_routing(rid, E)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["sorted_copy"].cpu().numpy(), sc)
    assert np.array_equal(r["copy_pos"].cpu().numpy(), cp)
    assert np.array_equal(bits(r["x_perm"][: T * k]),
                          bits(x[torch.from_numpy(sc // k)]))


def test_init_routing_invalid_ids_are_ignored():
    m = _m()
    shape = SMALL["decode_bf16_small"]
    inp = generate(shape, seed=0, device=DEV, weights=False)
    rid, _ = O.gate_topk(inp["logits"].cpu().numpy(), shape.top_k)
    rid = rid.copy()
    rid[3, 1] = -5
    rid[7, 0] = shape.E_tot + 3
    r = m.init_routing(m.problem(shape), torch.from_numpy(rid).to(DEV), inp["x"])
    torch.cuda.synchronize()
    cp = r["copy_pos"].cpu().numpy()
    assert cp[3 * shape.top_k + 1] == -1 and cp[7 * shape.top_k] == -1
    assert int(r["offsets"][-1]) == rid.size - 2


# ------------------------------------------------------------------ FFN, finalize


@pytest.mark.parametrize("name", list(SMALL))
def test_grouped_ffn_on_oracle_routing(name):
    """moe_grouped_ffn fed the oracle's routing and x_perm; y vs oracle y."""
    m = _m()
    shape = SMALL[name]
    _say("ffn", name)
    inp = generate(shape, seed=4, device=DEV)
    ref = _oracle_layer(shape, inp)
    R = ref["R"]
    p = m.problem(shape)
    offsets = torch.from_numpy(ref["offsets"].astype(np.int32)).to(DEV)
    N = shape.T * shape.top_k
    if shape.act_q in ("mxfp8", "int8"):
        i8 = shape.act_q == "int8"
        xp = torch.zeros((N, shape.H), dtype=torch.int8 if i8 else torch.uint8)
        xs = (torch.zeros(N, dtype=torch.float32) if i8 else
              torch.zeros((N, shape.H // 32), dtype=torch.uint8))
        xp[:R] = torch.from_numpy(ref["x_perm_codes"])
        xs[:R] = torch.from_numpy(ref["x_perm_scale"])
        xp, xs = xp.to(DEV), xs.to(DEV)
    else:
        dt = torch.float32 if shape.act == "f32" else torch.bfloat16
        xp = torch.zeros((N, shape.H), dtype=dt)
        xp[:R] = torch.from_numpy(ref["x_perm"]).to(dt)
        xp, xs = xp.to(DEV), None
    y = m.grouped_ffn(p, offsets, xp, xs, inp["w13"], inp["w2"],
                      inp["w13_scale"], inp["w2_scale"])
    torch.cuda.synchronize()
    allow = None
    if shape.act_q in ("mxfp8", "int8") and R:
        # the same GEMM1 through moe_ffn_up gives the GPU's codes of h
        h, hs = m.ffn_up(p, offsets, xp, xs, inp["w13"], inp["w13_scale"])
        torch.cuda.synchronize()
        allow = quant_h_allowance(shape, ref["x_perm"], h[:R].cpu().numpy(),
                                  hs[:R].cpu().numpy(), ref["h_codes"],
                                  ref["h_scale"], ref["offsets"], ref["row0"],
                                  np.arange(R), weight_getter(shape, inp))
    assert_close(to64(y[:R]), ref["y"], shape, "y", allow=allow)


@pytest.mark.parametrize("E,K,N", [(1, 32, 16), (3, 128, 48), (2, 512, 160),
                                   (1, 4096, 3072)])
def test_quant_mxfp4_weights_bit_exact(E, K, N):
    """The library's MXFP4 weight quantisation against the oracle's MX
    quantiser, codes and scales bit for bit, on N(0, 0.02) bf16 weights with
    planted edge blocks: all zero, exact e2m1 midpoints at scale 2^0 (ties to
    even), saturating values, negative values rounding to -0, tiny blocks
    whose scale clamps, huge values."""
    m = _m()
    g = torch.Generator().manual_seed(E * 7919 + K + N)
    w = (torch.randn(E, K, N, generator=g) * 0.02).to(torch.bfloat16)
    w[0, :32, 0] = 0.0
    if N > 1:
        mids = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                             -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -0.2,
                             0.1, 4.9, 5.5, -5.5, 2.25, 1.1, 0.3, -0.3,
                             3.0, -3.0, 0.5, -0.5, 1.0, 1.5, 2.0, 4.0])
        w[0, :32, 1] = mids.to(torch.bfloat16)
    if N > 2:
        w[0, :32, 2] = (torch.randn(32, generator=g) * 1e-38).to(torch.bfloat16)
    if N > 3:
        w[0, :32, 3] = (torch.randn(32, generator=g) * 1e37).to(torch.bfloat16)
    if E > 1 and N > 4:
        w[1, :, 4] = -1e-3  # rounds to -0 next to the block maximum below
        w[1, 0, 4] = 7.0    # amax 7: s = 0, and 7 saturates to 6
    codes, scales = m.quant_mxfp4_weights(w.to(DEV))
    torch.cuda.synchronize()
    wt = w.double().numpy().transpose(0, 2, 1)          # [E, N, K]
    rc, rs = O.mx_quant(wt, "e2m1")
    packed = (rc[..., 0::2] | (rc[..., 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), packed)


@pytest.mark.parametrize("name", list(SMALL))
def test_finalize_on_oracle_inputs(name):
    m = _m()
    shape = SMALL[name]
    inp = generate(shape, seed=5, device=DEV)
    ref = _oracle_layer(shape, inp)
    p = m.problem(shape)
    N = shape.T * shape.top_k
    dt = torch.float32 if shape.act == "f32" else torch.bfloat16
    y = torch.zeros((N, shape.H), dtype=dt)
    y[:ref["R"]] = torch.from_numpy(ref["y"]).to(dt)
    out = m.finalize(p, torch.from_numpy(ref["topk_ids"]).to(DEV),
                     torch.from_numpy(ref["topk_weight"].astype(np.float32)).to(DEV),
                     torch.from_numpy(ref["copy_pos"].astype(np.int32)).to(DEV),
                     torch.from_numpy(ref["offsets"].astype(np.int32)).to(DEV),
                     y.to(DEV), inp["x"], inp["residual"])
    torch.cuda.synchronize()
    assert_close(to64(out), ref["out"], shape, "out")


# ------------------------------------------------------------------ whole layer


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name, seed):
    m = _m()
    shape = SMALL[name]
    _say("layer", name, seed)
    inp = generate(shape, seed=seed, device=DEV)
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                  inp["w2"], inp["w13_scale"], inp["w2_scale"],
                  residual=inp["residual"])
    torch.cuda.synchronize()
    ref, allow = layer_ref(m, shape, inp)
    assert_close(to64(out), ref, shape, f"{name} seed {seed}", allow=allow)


def test_layer_split_calls_equal_fused():
    """The five calls in sequence give the same bits as moe_layer."""
    m = _m()
    for name in ("prefill_skewed_small", "prefill_wide_small", "ep_w4a8_small",
                 "ep_w4a8_prefill_small", "ep_w4a8_wide_small",
                 "tiny_fp32", "decode_bf16_small", "decode_w8a8_small",
                 "prefill_w8a8_small", "prefill_w8a8_mid_small",
                 "prefill_long_small", "prefill_w8a8_long_small",
                 "decode_w8a8_h2048_small", "range_w8a8_small",
                 "decode_bf16_32row_small", "range_w8a8_stream_small",
                 "zero_experts_small"):
        shape = SMALL[name]
        inp = generate(shape, seed=6, device=DEV)
        p = m.problem(shape)
        fused = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                        inp["w13_scale"], inp["w2_scale"], residual=inp["residual"])
        ids, w = m.gate_topk(p, inp["logits"])
        r = m.init_routing(p, ids, inp["x"])
        h, hs = m.ffn_up(p, r["offsets"], r["x_perm"], r["x_perm_scale"],
                         inp["w13"], inp["w13_scale"])
        y = m.ffn_down(p, r["offsets"], h, hs, inp["w2"], inp["w2_scale"])
        out = m.finalize(p, ids, w, r["copy_pos"], r["offsets"], y, inp["x"],
                         inp["residual"])
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(fused)), name


@pytest.mark.parametrize("name", ["decode_bf16_small", "decode_w8a8_small",
                                  "ep_w4a8_small", "prefill_wide_small",
                                  "zero_experts_small", "decode_bf16_32row_small",
                                  "range_w8a8_stream_small"])
def test_prefetch_weights_changes_nothing(name):
    """moe_prefetch_weights only reads: the layer gives the same bits after
    it as before, whatever the budget (none, small, past every weight byte),
    with and without routing ids (ids outside the range among them), for
    w13, w2 or both."""
    m = _m()
    shape = SMALL[name]
    inp = generate(shape, seed=9, device=DEV)
    p = m.problem(shape)
    args = (p, inp["logits"], inp["x"], inp["w13"], inp["w2"], inp["w13_scale"],
            inp["w2_scale"])
    want = m.layer(*args, residual=inp["residual"])
    ids, _ = m.gate_topk(p, inp["logits"])
    bad = ids.clone()
    bad[0, 0] = -3
    bad[-1, -1] = shape.E_tot + 5
    for topk in (None, ids, bad):
        for which in (1, 2, 3):
            for nbytes in (0, 4096, 1 << 20, 1 << 40):
                m.prefetch_weights(p, inp["w13"], inp["w2"], topk_ids=topk,
                                   max_bytes=nbytes, which=which)
    got = m.layer(*args, residual=inp["residual"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(want))


def test_prefetch_weights_full_size_decode():
    """The decode workload at full size: prefetch of every expert's w13 heads
    with the gate's ids, then the layer, equal to the layer alone."""
    m = _m()
    shape = get_workload("qwen3_30b_a3b_decode_bf16")
    inp = generate(shape, seed=3, device=DEV)
    p = m.problem(shape)
    want = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"])
    ids, _ = m.gate_topk(p, inp["logits"])
    m.prefetch_weights(p, inp["w13"], topk_ids=ids, max_bytes=96 << 20)
    got = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(want))


def test_layer_deterministic():
    m = _m()
    shape = SMALL["prefill_skewed_small"]
    inp = generate(shape, seed=7, device=DEV)
    p = m.problem(shape)
    a = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                residual=inp["residual"])
    b = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                residual=inp["residual"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("name", ["ep_w4a8_small", "qwen3_235b_a22b_ep_rank_w4a8"])
def test_expert_range_partials_add_up(name):
    """One call per expert-parallel share; the partial sums add up to the
    full-range layer (the single-GPU stand-in for the reduce-scatter), on a
    small W4A8 shape and on the W4A8 rank's full shape (four ranks of 32 of
    the 128 experts)."""
    m = _m()
    _say("EP additivity", name)
    base = SMALL[name] if name in SMALL else get_workload(name)
    full = base.replace(local_begin=0, local_end=base.n_ffn)
    inp = generate(full, seed=8, device=DEV)
    p = m.problem(full)
    ref = m.layer(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                  inp["w13_scale"], inp["w2_scale"]).double()
    total = torch.zeros_like(ref)
    q = full.n_ffn // 4
    for i in range(4):
        sh = full.replace(local_begin=i * q, local_end=(i + 1) * q)
        sl = slice(i * q, (i + 1) * q)
        part = m.layer(m.problem(sh), inp["logits"], inp["x"],
                       inp["w13"][sl].contiguous(), inp["w2"][sl].contiguous(),
                       inp["w13_scale"][sl].contiguous(),
                       inp["w2_scale"][sl].contiguous())
        total += part.double()
    torch.cuda.synchronize()
    assert_close(total.cpu().numpy(), ref.cpu().numpy(), full, "partials")


# ------------------------------------------------------------------ edge cases


def _layer_vs_oracle(shape, seed=0, logit_fn=None):
    m = _m()
    inp = generate(shape, seed=seed, device=DEV)
    if logit_fn is not None:
        inp["logits"] = logit_fn(inp["logits"]).contiguous()
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                  inp["w2"], inp["w13_scale"], inp["w2_scale"],
                  residual=inp["residual"])
    torch.cuda.synchronize()
    if shape.T:
        ref, allow = layer_ref(m, shape, inp)
        assert_close(to64(out), ref, shape, shape.name, allow=allow)
    return out


def test_edge_single_token_and_k_equals_E():
    b = SMALL["decode_bf16_small"]
    _layer_vs_oracle(b.replace(T=1))
    _layer_vs_oracle(b.replace(T=5, top_k=b.n_ffn))
    _layer_vs_oracle(SMALL["tiny_fp32"].replace(top_k=1))


def test_edge_max_experts_and_top_k():
    """2048 experts with top-64 routing (the library's limits): about two
    rows per expert through the streaming GEMMs, checked on the whole layer."""
    b = SMALL["decode_bf16_small"].replace(T=64, H=64, I=32, n_ffn=2048,
                                            local_end=2048, top_k=64)
    _layer_vs_oracle(b)


def test_edge_zero_tokens():
    m = _m()
    shape = SMALL["decode_bf16_small"].replace(T=0)
    inp = generate(shape, seed=0, device=DEV)
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"], inp["w2"])
    torch.cuda.synchronize()
    assert out.shape == (0, shape.H)


def test_edge_identity_experts_only():
    b = SMALL["zero_experts_small"]
    # every token routes only to identity experts: out = x (weights sum to 1)
    _layer_vs_oracle(b, logit_fn=lambda L: torch.cat(
        [L[:, : b.n_ffn] - 100.0, L[:, b.n_ffn:]], 1))
    # a range holding only identity experts: no FFN expert in range at all
    _layer_vs_oracle(b.replace(local_begin=b.n_ffn, local_end=b.E_tot))


def test_edge_hot_expert_many_tiles():
    # one expert takes every token: one expert with T rows, many tiles
    b = SMALL["prefill_skewed_small"].replace(T=700)
    _layer_vs_oracle(b, logit_fn=lambda L: L + torch.nn.functional.one_hot(
        torch.full((L.shape[0],), 3, device=L.device), L.shape[1]).float() * 50)


@pytest.mark.parametrize("I", [32, 64, 96])
def test_edge_short_k_tiled(I):
    # GEMM2 with K = I of 1..3 steps of 32: no longer than the LDS ring
    _layer_vs_oracle(SMALL["prefill_wide_small"].replace(I=I))


@pytest.mark.parametrize("name", ["prefill_w8a8_small", "decode_w8a8_small"])
def test_edge_short_k_w8a8(name):
    # GEMM2 with K = I = 128: two int8 steps of the tiled kernel, one of the
    # streaming kernel
    _layer_vs_oracle(SMALL[name].replace(I=128))


def test_edge_w8a8_zero_rows_of_x():
    # all-zero tokens quantise to scale 0 and codes 0: their expert outputs
    # are exactly 0 and the layer returns the residual for them
    def zero_some(inp):
        inp["x"][::3] = 0
        return inp
    b = SMALL["prefill_w8a8_small"]
    m = _m()
    inp = zero_some(generate(b, seed=1, device=DEV))
    out = m.layer(m.problem(b), inp["logits"], inp["x"], inp["w13"], inp["w2"],
                  inp["w13_scale"], inp["w2_scale"], residual=inp["residual"])
    torch.cuda.synchronize()
    ref, allow = layer_ref(m, b, inp)
    assert_close(to64(out), ref, b, "zero rows", allow=allow)
    assert np.array_equal(bits(out[::3]), bits(inp["residual"][::3]))


def test_edge_range_drops_everything():
    b = SMALL["ep_w4a8_small"]
    # logits steer every token away from the local range: partial sum is 0
    out = _layer_vs_oracle(b, logit_fn=lambda L: torch.cat(
        [L[:, : b.local_begin], L[:, b.local_begin: b.local_end] - 100.0,
         L[:, b.local_end:]], 1))
    assert float(out.abs().max()) == 0.0


# ------------------------------------------------------------------ full size


FFN_FULL = ["qwen3_30b_a3b_prefill_skewed_bf16", "longcat_flash_zero_experts_bf16",
            "qwen3_235b_a22b_ep_rank_w4a8", "qwen3_30b_a3b_prefill_skewed_w8a8"]


@pytest.mark.parametrize("name", FFN_FULL)
def test_grouped_ffn_full_size_sampled_experts(name):
    """moe_grouped_ffn at the full workload size (the launch configuration of
    the layer), fed the oracle's routing and permuted activations; y of the
    rows of sampled experts -- the hottest, the coldest non-empty one, the
    median and five at random -- against the oracle's expert FFN, element by
    element."""
    m = _m()
    shape = get_workload(name)
    _say("ffn full", name)
    inp = generate(shape, seed=0, device=DEV)
    ids, _ = O.gate_topk(inp["logits"].cpu().numpy(), shape.top_k)
    counts, offsets, sc, _ = O.init_routing(ids, shape.E_tot)
    fb, fe = shape.ffn_begin, shape.ffn_end
    r0, R = int(offsets[fb]), int(offsets[fe] - offsets[fb])
    tok = sc[r0:r0 + R] // shape.top_k
    x64 = to64(inp["x"])
    N = shape.T * shape.top_k
    if shape.act_q == "mxfp8":
        qc, qs = O.mx_quant(x64, "e4m3")            # per token, then gathered
        xp = torch.zeros((N, shape.H), dtype=torch.uint8)
        xs = torch.zeros((N, shape.H // 32), dtype=torch.uint8)
        xp[:R], xs[:R] = torch.from_numpy(qc[tok]), torch.from_numpy(qs[tok])
        a_all = O.mx_dequant(qc, qs, "e4m3")
    elif shape.act_q == "int8":
        qc, qs = O.int8_quant_rows(x64)
        xp = torch.zeros((N, shape.H), dtype=torch.int8)
        xs = torch.zeros(N, dtype=torch.float32)
        xp[:R], xs[:R] = torch.from_numpy(qc[tok]), torch.from_numpy(qs[tok])
        a_all = O.int8_dequant_rows(qc, qs)
    else:
        xp = torch.zeros((N, shape.H), dtype=torch.bfloat16)
        xp[:R] = inp["x"].cpu()[torch.from_numpy(tok)]
        xs, a_all = None, x64
    xp = xp.to(DEV)
    xs = None if xs is None else xs.to(DEV)
    p = m.problem(shape)
    y = m.grouped_ffn(p, torch.from_numpy(offsets.astype(np.int32)).to(DEV), xp, xs,
                      inp["w13"], inp["w2"], inp["w13_scale"], inp["w2_scale"])
    torch.cuda.synchronize()
    loc = counts[fb:fe]
    nz = np.nonzero(loc)[0]
    order = nz[np.argsort(loc[nz], kind="stable")]
    rng = np.random.default_rng(0)
    pick = {int(order[-1]), int(order[0]), int(order[len(order) // 2])}
    pick |= set(int(v) for v in rng.choice(nz, size=min(5, len(nz)), replace=False))
    get = weight_getter(shape, inp)
    quant = shape.act_q in ("mxfp8", "int8")
    ndiff = nrows = 0
    if quant:
        h, hs = m.ffn_up(p, torch.from_numpy(offsets.astype(np.int32)).to(DEV), xp,
                         xs, inp["w13"], inp["w13_scale"])
        torch.cuda.synchronize()
    for i in sorted(pick):
        e = fb + i
        lo, hi = int(offsets[e]) - r0, int(offsets[e + 1]) - r0
        a = a_all[tok[lo:hi]]
        _, hc, ye = O.expert_ffn(a, *get(e), act=shape.act, act_q=shape.act_q)
        allow = None
        if quant:
            allow, nd = _expert_allowance(shape, e, a, h[lo:hi], hs[lo:hi], hc, get)
            ndiff, nrows = ndiff + nd, nrows + hi - lo
        assert_close(to64(y[lo:hi]), ye, shape, f"{name} expert {e} ({hi - lo} rows)",
                     allow=allow)
    if quant:
        assert_rare_codes(ndiff, nrows * shape.I)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_prefill_skewed_bf16",
                                  "qwen3_30b_a3b_prefill_skewed_w8a8"])
def test_layer_full_size_without_residual(name):
    """The residual workloads at full size with residual = None: the sampled
    outputs are the expert sums alone, so the tolerance is not diluted by the
    N(0, 1) residual."""
    m = _m()
    shape = get_workload(name)
    _say("full no residual", name)
    inp = generate(shape, seed=2, device=DEV)
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                  inp["w2"], inp["w13_scale"], inp["w2_scale"], residual=None)
    torch.cuda.synchronize()
    toks = _sample_tokens(shape.T, 48, seed=2)
    ref, allow = layer_ref(m, shape, inp, toks, residual=False)
    assert_close(to64(out)[toks], ref, shape, name, allow=allow)


def _expert_allowance(shape, e, a, gh, ghs, ref_codes, get):
    """assert_close's allowance for the rows of one expert: the GPU's codes
    of h (gh, ghs) checked against the oracle's (ref_codes) and their effect
    |h_gpu - h_oracle| @ |w2| on y."""
    w13, w2 = get(e)
    v32, tol = h_error_bound(shape, a, w13)
    gd, rd, nd = check_quant_h(shape, v32, tol, gh.cpu().numpy(), ghs.cpu().numpy(),
                               ref_codes[0], ref_codes[1])
    return np.abs(gd - rd) @ np.abs(w2), nd


def _sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=min(n, T), replace=False))


FULL_SAMPLES = {"tiny_fp32": 16, "qwen3_30b_a3b_decode_bf16": 32,
                "qwen3_30b_a3b_prefill_skewed_bf16": 48,
                "longcat_flash_zero_experts_bf16": 32,
                "qwen3_235b_a22b_ep_rank_w4a8": 48,
                "qwen3_30b_a3b_decode_w8a8": 32,
                "qwen3_30b_a3b_prefill_skewed_w8a8": 48}


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_prefill_skewed_bf16",
                                  "qwen3_30b_a3b_prefill_skewed_w8a8"])
def test_layer_long_prefill_sampled(name):
    """The skewed prefill workloads at T = 16384 (1024 rows per expert on
    average: the 256-row LDS tiles); sampled tokens against the oracle."""
    m = _m()
    shape = get_workload(name).replace(T=16384)
    _say("long prefill", name)
    inp = generate(shape, seed=1, device=DEV)
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                  inp["w2"], inp["w13_scale"], inp["w2_scale"],
                  residual=inp["residual"])
    torch.cuda.synchronize()
    toks = _sample_tokens(shape.T, 32, seed=1)
    ref, allow = layer_ref(m, shape, inp, toks)
    assert_close(to64(out)[toks], ref, shape, name, allow=allow)
    assert torch.isfinite(out.float()).all()
    # the expert part alone (no residual to dilute the tolerance)
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                  inp["w2"], inp["w13_scale"], inp["w2_scale"], residual=None)
    torch.cuda.synchronize()
    ref, allow = layer_ref(m, shape, inp, toks, residual=False)
    assert_close(to64(out)[toks], ref, shape, name + " without residual",
                 allow=allow)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layer_full_size_sampled(name):
    """Full-size workload through moe_layer (the benchmark's call); sampled
    tokens checked against the oracle's per-token evaluation."""
    m = _m()
    shape = get_workload(name)
    _say("full", name)
    inp = generate(shape, seed=0, device=DEV)
    out = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                  inp["w2"], inp["w13_scale"], inp["w2_scale"],
                  residual=inp["residual"])
    torch.cuda.synchronize()
    toks = _sample_tokens(shape.T, FULL_SAMPLES[name])
    ref, allow = layer_ref(m, shape, inp, toks)
    got = to64(out)[toks]
    assert_close(got, ref, shape, name, allow=allow)
    # every output row is finite
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("E,N,Kb,dt", [(3, 48, 256, torch.int8),
                                       (1, 16, 64, torch.uint8),
                                       (2, 1536, 2048, torch.int8),
                                       (2, 3072, 2048, torch.uint8)])
def test_pack_weights(E, N, Kb, dt):
    """The packed weight order, byte for byte: fragments in the order
    [e][c][n16]; lane l of fragment (e, c, n16) holds
    W[e, 16 n16 + l % 16, 64 c + 16 (l / 16) .. + 15]."""
    m = _m()
    g = torch.Generator().manual_seed(E * 1000 + N + Kb)
    w = torch.randint(-128, 128, (E, N, Kb), generator=g, dtype=torch.int16).to(dt)
    got = m.pack_weights(w.to(DEV))
    torch.cuda.synchronize()
    W = w.numpy().reshape(E, N // 16, 16, Kb // 64, 4, 16)
    # [e][n16][col][c][q][16 bytes] -> [e][c][n16][q][col][16]; lane = 16 q + col
    want = W.transpose(0, 3, 1, 4, 2, 5).reshape(E, N, Kb)
    assert np.array_equal(got.cpu().numpy(), want)


# bf16 shapes with whole 256-column slabs (I % 128 == 0, H % 256 == 0), one
# per bf16 GEMM schedule: 16- and 32-row weight-streaming tiles (K split 3
# and 1), 128- and 256-row LDS-tiled tiles, identity experts, an expert range
PACKED_BF16 = {
    "decode_16row": scaled(get_workload("qwen3_30b_a3b_decode_bf16"), T=16,
                           H=512, I=384, n_ffn=16, local_end=16, top_k=4),
    "decode_32row": scaled(get_workload("qwen3_30b_a3b_decode_bf16"), T=32,
                           H=512, I=384, n_ffn=16, local_end=16, top_k=4),
    # 8 rows per expert on the decode expert shape: 32-row tiles, no K split
    "decode_32row_wide": scaled(get_workload("qwen3_30b_a3b_decode_bf16"),
                                T=128),
    "prefill_128": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                          T=300, H=256, I=256, n_ffn=12, local_end=12, top_k=4),
    "prefill_256": scaled(get_workload("qwen3_30b_a3b_prefill_skewed_bf16"),
                          T=1200, H=512, I=256, n_ffn=8, local_end=8, top_k=4),
    "zero_experts": scaled(get_workload("longcat_flash_zero_experts_bf16"),
                           T=64, H=512, I=256, n_ffn=24, n_zero=12,
                           local_end=36, top_k=6),
    "range": scaled(get_workload("qwen3_30b_a3b_decode_bf16"), T=48, H=768,
                    I=512, n_ffn=16, local_begin=3, local_end=11, top_k=4),
}


def _packed_inputs(m, inp):
    """The workload's bf16 weights in the slab order (w13 gate/up paired)."""
    return (m.pack_bf16_weights(inp["w13"], glu=True),
            m.pack_bf16_weights(inp["w2"], glu=False))


@pytest.mark.parametrize("E,K,N,glu", [(1, 32, 256, True), (3, 96, 512, True),
                                       (2, 64, 768, False), (2, 2048, 1536, True),
                                       (2, 768, 2048, False)])
def test_pack_bf16_weights(E, K, N, glu):
    """The slab order, element for element: [e][j][s][r][c] holds
    W[e, 32 s + r, col_j(c)] with col_j(c) = 128 j + c / N/2 + 128 j + c - 128
    (gate/up pairs) or 256 j + c."""
    m = _m()
    _say("pack_bf16", E, K, N, glu)
    g = torch.Generator().manual_seed(E * 7919 + K + N)
    w = torch.randint(-32768, 32768, (E, K, N), generator=g,
                      dtype=torch.int32).to(torch.int16)
    got = m.pack_bf16_weights(w.view(torch.bfloat16).to(DEV), glu=glu)
    torch.cuda.synchronize()
    W = w.numpy()
    nsl, nst = N // 256, K // 32
    if glu:
        gate = W[:, :, : N // 2].reshape(E, nst, 32, nsl, 128)
        up = W[:, :, N // 2:].reshape(E, nst, 32, nsl, 128)
        slabs = np.concatenate([gate, up], axis=4)  # [e][s][r][j][256]
    else:
        slabs = W.reshape(E, nst, 32, nsl, 256)
    want = slabs.transpose(0, 3, 1, 2, 4).reshape(E, K, N)
    assert np.array_equal(got.cpu().view(torch.int16).numpy(), want)


@pytest.mark.parametrize("name", list(PACKED_BF16))
def test_layer_bf16_packed(name):
    """Slab-packed bf16 weights feed the MFMAs the same operands as row-major
    ones: the layer's output is bit-identical, and within tolerance of the
    oracle."""
    m = _m()
    shape = PACKED_BF16[name]
    _say("layer packed bf16", name)
    inp = generate(shape, seed=4, device=DEV)
    w13p, w2p = _packed_inputs(m, inp)
    want = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                   inp["w2"], residual=inp["residual"])
    got = m.layer(m.problem(shape, wt_layout="packed"), inp["logits"], inp["x"],
                  w13p, w2p, residual=inp["residual"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(want)), name
    ref, allow = layer_ref(m, shape, inp)
    assert_close(to64(got), ref, shape, f"{name} packed", allow=allow)


def test_layer_bf16_packed_split_calls_and_prefetch():
    """The per-stage calls and the weight prefetch take the packed layout
    too: same bits as the fused layer on row-major weights."""
    m = _m()
    for name in ("decode_32row", "prefill_128", "decode_16row"):
        shape = PACKED_BF16[name]
        _say("packed split/prefetch", name)
        inp = generate(shape, seed=5, device=DEV)
        w13p, w2p = _packed_inputs(m, inp)
        want = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                       inp["w2"], residual=inp["residual"])
        p = m.problem(shape, wt_layout="packed")
        ids, w = m.gate_topk(p, inp["logits"])
        for which in (1, 2, 3):
            for nbytes in (4096, 1 << 20, 1 << 40):
                m.prefetch_weights(p, w13p, w2p, topk_ids=ids,
                                   max_bytes=nbytes, which=which)
        r = m.init_routing(p, ids, inp["x"])
        h, hs = m.ffn_up(p, r["offsets"], r["x_perm"], r["x_perm_scale"], w13p)
        y = m.ffn_down(p, r["offsets"], h, hs, w2p)
        out = m.finalize(p, ids, w, r["copy_pos"], r["offsets"], y, inp["x"],
                         inp["residual"])
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(want)), name


@pytest.mark.parametrize("name", ["longcat_flash_zero_experts_bf16",
                                  "qwen3_30b_a3b_decode_bf16",
                                  "qwen3_30b_a3b_prefill_skewed_bf16"])
def test_layer_full_size_bf16_packed(name):
    """At the workloads' full sizes, in the configuration bench.py times:
    the packed layer equals the row-major one bit for bit."""
    m = _m()
    shape = get_workload(name)
    _say("full-size packed", name)
    inp = generate(shape, seed=0, device=DEV)
    want = m.layer(m.problem(shape), inp["logits"], inp["x"], inp["w13"],
                   inp["w2"], residual=inp["residual"])
    w13p, w2p = _packed_inputs(m, inp)
    del inp["w13"], inp["w2"]
    got = m.layer(m.problem(shape, wt_layout="packed"), inp["logits"], inp["x"],
                  w13p, w2p, residual=inp["residual"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(want)), name
