"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked fixtures (tests/golden), closed forms, library routines (scipy
softmax, torch float8 conversion, torch SiLU / chunk), invariants, and brute
force on tiny inputs. No GPU needed."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- gate


def test_gate_golden_cases():
    for c in _load("gate_cases.json")["cases"]:
        L = np.array([c["logits"]], dtype=np.float32)
        ids, w = O.gate_topk(L, c["k"])
        assert ids[0].tolist() == c["ids"]
        if "w" in c:
            np.testing.assert_allclose(w[0], c["w"], rtol=0, atol=1e-7)
    # the formula case: three logits of 7 and one of 0
    L = np.array([[-5, 7, -5, 7, 0, 7]], dtype=np.float32)
    _, w = O.gate_topk(L, 4)
    d = 3 * math.exp(7) + 1
    np.testing.assert_allclose(w[0], [math.exp(7) / d] * 3 + [1 / d], rtol=1e-14)


def test_gate_full_k_is_scipy_softmax():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((7, 12)).astype(np.float32)
    ids, w = O.gate_topk(L, 12)
    ref = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1),
                               rtol=1e-13)
    # ids are a permutation in descending-logit order
    for t in range(7):
        assert sorted(ids[t].tolist()) == list(range(12))
        assert np.all(np.diff(L[t, ids[t]]) <= 0)


def test_gate_topk_then_softmax_equals_softmax_then_renormalise():
    rng = np.random.default_rng(2)
    for E, k in [(8, 2), (128, 8), (768, 12)]:
        L = rng.standard_normal((5, E)).astype(np.float32)
        ids, w = O.gate_topk(L, k)
        full = scipy.special.softmax(L.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, ids.astype(np.int64), 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)


def test_gate_bruteforce_selection():
    rng = np.random.default_rng(3)
    # integer logits force many ties
    L = rng.integers(-3, 4, size=(40, 9)).astype(np.float32)
    for k in (1, 3, 9):
        ids, _ = O.gate_topk(L, k)
        for t in range(L.shape[0]):
            # brute force: repeatedly take the best remaining (value desc, id asc)
            left = list(range(9))
            want = []
            for _ in range(k):
                best = left[0]
                for e in left[1:]:
                    if L[t, e] > L[t, best]:
                        best = e
                want.append(best)
                left.remove(best)
            assert ids[t].tolist() == want


def test_gate_signed_zero_is_a_tie():
    L = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    ids, w = O.gate_topk(L, 2)
    assert ids[0].tolist() == [0, 1]
    np.testing.assert_allclose(w[0], [0.5, 0.5], rtol=0, atol=0)


# ----------------------------------------------------------------- routing


def test_routing_golden():
    g = _load("routing_small.json")
    counts, offsets, sc, cp = O.init_routing(np.array(g["topk_ids"]), g["n_experts"])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert sc.tolist() == g["sorted_copy"]
    assert cp.tolist() == g["copy_pos"]


def _routing_bruteforce(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    sorted_copy = [c for e in range(E) for c in range(len(flat)) if flat[c] == e]
    pos = [0] * len(flat)
    for i, c in enumerate(sorted_copy):
        pos[c] = i
    offs = [0]
    for e in range(E):
        offs.append(offs[-1] + counts[e])
    return counts, offs, sorted_copy, pos


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 4, 2), (16, 8, 2), (13, 24, 5), (0, 3, 1)])
def test_routing_bruteforce(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
    counts, offsets, sc, cp = O.init_routing(ids, E)
    bc, bo, bs, bp = _routing_bruteforce(ids, E)
    assert counts.tolist() == bc and offsets.tolist() == bo
    assert sc.tolist() == bs and cp.tolist() == bp
    # invariants
    assert counts.sum() == T * k
    flat = ids.reshape(-1)
    if T:
        assert np.all(np.diff(flat[sc]) >= 0)
        assert np.array_equal(cp[sc], np.arange(T * k))
        for e in range(E):
            seg = sc[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)


def test_routing_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.init_routing(np.array([[0, 5]]), 5)


# ----------------------------------------------------------------- MX formats


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero
    assert np.signbit(got[128]) and not np.signbit(got[0])


def test_e4m3_encode_matches_torch_rne_in_range():
    # every finite code value, every midpoint between neighbours, and random
    # values, all within [-448, 448] where torch's conversion is plain RNE
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    pos = np.unique(vals[(vals >= 0) & np.isfinite(vals)])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(4)
    rnd = rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000))
    rnd = rnd[np.abs(rnd) <= 448]
    v = np.concatenate([pos, mids, -pos, -mids, rnd]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    assert O.e4m3_encode(np.array([500.0, 1e9, -1e9, 449.0]))[:].tolist() == [126, 126, 254, 126]


def test_e2m1_table_and_midpoints():
    # OCP MX v1.0 e2m1 values for codes 0..7 (sign in bit 3)
    assert O.e2m1_decode(np.arange(8)).tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert O.e2m1_decode(np.arange(8, 16)).tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    # ties to even mantissa, saturation at 6
    mid = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0,
           5.0: 4.0, 7.0: 6.0, 100.0: 6.0}
    got = O.e2m1_decode(O.e2m1_encode(np.array(list(mid))))
    assert got.tolist() == list(mid.values())
    for c in range(16):
        assert O.e2m1_encode(O.e2m1_decode(np.array([c])))[0] == (0 if c == 8 else c) or c == 8


def test_mx_golden_blocks():
    for c in _load("mx_blocks.json")["cases"]:
        v = np.full(32, c["rest"], dtype=np.float64)
        v[0] = c["first"]
        codes, sc = O.mx_quant(v[None, :], c["fmt"])
        assert int(sc[0, 0]) == c["scale"], c
        assert int(codes[0, 0]) == c["code_first"], c
        assert np.all(codes[0, 1:] == c["code_rest"]), c


def test_mx_roundtrip_and_error_bound():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    v = O.round_bf16(v)
    codes, sc = O.mx_quant(v, "e4m3")
    d = O.mx_dequant(codes, sc, "e4m3")
    # per block: |error| <= half an e4m3 ulp at the scaled magnitude
    s = O.e8m0_decode(sc).repeat(32, axis=1)
    q = np.abs(v) / s
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.maximum(q, 1e-300))), -6) - 3)
    sat = q > 448
    assert np.all(np.abs(d - v)[~sat] <= 0.5 * ulp[~sat] * s[~sat] * (1 + 1e-12))
    # decode(encode(decode(c))) == decode(c): representable values round-trip
    codes2, sc2 = O.mx_quant(d, "e4m3")
    assert np.array_equal(O.mx_dequant(codes2, sc2, "e4m3"), d)


def test_mxfp4_unpack_nibble_order():
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)
    assert O.mxfp4_unpack(packed).tolist() == [[1, 2, 7, 15]]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(50000) * np.exp2(rng.integers(-30, 30, 50000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().double().numpy()
    assert np.array_equal(O.round_bf16(v.astype(np.float64)), ref)


# ----------------------------------------------------------------- FFN / layer


def test_silu_closed_forms():
    np.testing.assert_allclose(O.silu(np.array([0.0, 1.0, -1.0])),
                               [0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.exp(1))],
                               rtol=1e-15)


def _tiny(T=6, H=32, I=16, n_ffn=4, n_zero=0, k=2, lb=0, le=None, seed=0, residual=False):
    rng = np.random.default_rng(seed)
    E = n_ffn + n_zero
    le = E if le is None else le
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, H))
    W13 = rng.standard_normal((n_ffn, H, 2 * I)) * 0.1
    W2 = rng.standard_normal((n_ffn, I, H)) * 0.1
    res = rng.standard_normal((T, H)) if residual else None
    kw = dict(logits=logits, x=x, get_weights=lambda e: (W13[e], W2[e]), T=T, H=H,
              I=I, n_ffn=n_ffn, n_zero=n_zero, top_k=k, local_begin=lb,
              local_end=le, residual=res)
    return kw, W13, W2


def test_single_expert_is_dense_swiglu_ffn_torch():
    # E=1, k=1: the layer is one dense FFN; compare with torch's chunk + silu
    kw, W13, W2 = _tiny(T=9, n_ffn=1, k=1)
    out = O.moe_layer(act="f32", exact=True, **kw)["out"]
    x = torch.from_numpy(kw["x"])
    g, u = torch.chunk(x @ torch.from_numpy(W13[0]), 2, -1)
    ref = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(W2[0])
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cfg", [
    dict(),
    dict(n_ffn=8, k=3, T=11, residual=True),
    dict(n_ffn=5, n_zero=3, k=4, T=10),
    dict(n_ffn=6, n_zero=2, k=2, lb=2, le=7, T=12),
])
def test_routed_equals_pertoken_and_dense(cfg):
    kw, _, _ = _tiny(**cfg)
    routed = O.moe_layer(act="f32", exact=True, **kw)["out"]
    per_tok = O.moe_tokens(range(kw["T"]), act="f32", exact=True, **kw)
    dense = O.moe_dense(**kw)
    np.testing.assert_allclose(routed, dense, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(per_tok, dense, rtol=1e-12, atol=1e-12)


def test_routed_equals_pertoken_with_roundings():
    for act, act_q in [("bf16", "none"), ("f32", "none"), ("bf16", "mxfp8")]:
        kw, _, _ = _tiny(T=10, H=64, I=32, n_ffn=6, n_zero=2, k=3, residual=True)
        routed = O.moe_layer(act=act, act_q=act_q, **kw)["out"]
        per_tok = O.moe_tokens(range(10), act=act, act_q=act_q, **kw)
        assert np.array_equal(routed, per_tok)


def test_zero_gate_columns_give_residual():
    # SiLU(0) = 0: with zero gate weights every expert output is 0
    kw, W13, W2 = _tiny(residual=True)
    W13[:, :, :16] = 0.0
    out = O.moe_layer(act="f32", exact=True, **kw)["out"]
    np.testing.assert_array_equal(out, kw["residual"])


def test_identity_experts_only_return_input():
    # bias the logits so only identity experts win: MoE(x) = x
    kw, _, _ = _tiny(T=7, n_ffn=4, n_zero=3, k=3, residual=True)
    kw["logits"][:, 4:] += 100.0
    for act in ("bf16", "f32"):
        xa = O.round_to(kw["x"], act)
        ra = O.round_to(kw["residual"], act)
        # without residual the weights sum to 1 and the output is x itself
        out = O.moe_layer(act=act, **dict(kw, x=xa, residual=None))["out"]
        np.testing.assert_array_equal(out, xa)
        # with residual: x + residual, rounded once (to within one ulp, since
        # the fp64 weights sum to 1 only up to rounding and x + r may be a tie)
        out = O.moe_layer(act=act, **dict(kw, x=xa, residual=ra))["out"]
        ref = xa + ra
        ulp = np.exp2(np.floor(np.log2(np.abs(ref) + 1e-30)) - (7 if act == "bf16" else 23))
        assert np.all(np.abs(out - ref) <= ulp + 1e-15 * np.abs(xa))


def test_expert_range_partial_sums_add_up():
    kw, _, _ = _tiny(T=12, n_ffn=8, n_zero=4, k=4)
    full = O.moe_layer(act="f32", exact=True, **kw)["out"]
    parts = [O.moe_layer(act="f32", exact=True, **dict(kw, local_begin=b, local_end=e))["out"]
             for b, e in [(0, 3), (3, 8), (8, 10), (10, 12)]]
    np.testing.assert_allclose(sum(parts), full, rtol=1e-12, atol=1e-12)


def test_gemm_inputs_are_the_routed_rows():
    kw, _, _ = _tiny(T=8, n_ffn=4, n_zero=2, k=2, lb=1, le=4)
    r = O.moe_layer(act="f32", exact=True, **kw)
    ids = r["topk_ids"].reshape(-1)
    # rows of x_perm are x of the copies whose expert lies in [1, 4), sorted
    want = [c for e in range(1, 4) for c in range(ids.size) if ids[c] == e]
    np.testing.assert_array_equal(r["x_perm"], kw["x"][np.array(want, int) // 2])
    assert r["R"] == len(want)


def test_mx_activation_codes_are_rowwise():
    rng = np.random.default_rng(7)
    x = O.round_bf16(rng.standard_normal((5, 64)))
    codes, sc = O.mx_quant(x, "e4m3")
    for t in range(5):
        c1, s1 = O.mx_quant(x[t:t + 1], "e4m3")
        assert np.array_equal(c1[0], codes[t]) and np.array_equal(s1[0], sc[t])


def test_mxfp4_weights_dequant_exact():
    # dequantised MXFP4 weights are exact fp64 numbers: code value * 2^(s-127)
    packed = np.array([[0x71, 0x8F] * 16], dtype=np.uint8)      # K = 64
    scales = np.array([[120, 127]], dtype=np.uint8)
    w = O.mxfp4_dequant_rows(packed, scales)
    assert w.shape == (1, 64)
    assert w[0, :4].tolist() == [0.5 * 2**-7, 6.0 * 2**-7, -6.0 * 2**-7, -0.0]
    assert w[0, 32:36].tolist() == [0.5, 6.0, -6.0, -0.0]


# ----------------------------------------------------------------- fused norm


def _bf16_rows(rng, T, H, std=1.0):
    return torch.from_numpy(rng.standard_normal((T, H)) * std).to(torch.bfloat16)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_rms_norm_matches_torch(eps):
    """torch's own rms_norm (float64) is an independent implementation."""
    rng = np.random.default_rng(11)
    s = rng.standard_normal((7, 96)) * rng.uniform(0.01, 10.0, (7, 1))
    w = rng.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(s), (96,),
                                       torch.from_numpy(w), eps).numpy()
    np.testing.assert_allclose(O.rms_norm(s, w, eps), ref, rtol=1e-13, atol=0)


def test_rms_norm_closed_forms():
    w = np.array([0.5, -2.0, 3.0, 1.0])
    # a constant row c normalises to sign(c) * weight when eps = 0
    for c in (3.0, -0.25, 1e-20):
        np.testing.assert_allclose(O.rms_norm(np.full((1, 4), c), w, 0.0)[0],
                                   np.sign(c) * w, rtol=1e-15)
    # [3, 4]: mean of squares 12.5
    np.testing.assert_allclose(O.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0),
                               [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)
    # scale invariance without eps; with unit weight mean(y^2) = ms / (ms + eps)
    rng = np.random.default_rng(3)
    s = rng.standard_normal((5, 64))
    np.testing.assert_allclose(O.rms_norm(37.0 * s, np.ones(64), 0.0),
                               O.rms_norm(s, np.ones(64), 0.0), rtol=1e-13)
    eps = 0.3
    ms = np.mean(s * s, axis=1)
    np.testing.assert_allclose(np.mean(O.rms_norm(s, np.ones(64), eps) ** 2, axis=1),
                               ms / (ms + eps), rtol=1e-13)


def test_add_rms_norm_residual_is_fp32_sum_rounded_to_bf16():
    rng = np.random.default_rng(5)
    x = _bf16_rows(rng, 9, 160)
    r = _bf16_rows(rng, 9, 160, std=3.0)
    r[0, :8] = torch.tensor([1e-6, -1e-6, 2.0 ** -20, 3e5, -3e5, 0.0, -0.0, 1.0]).to(torch.bfloat16)
    # exponent gaps past fp32's 24 bits: the fp32 sum drops the small part
    x[0, 3:5] = torch.tensor([1e-3, -1e-3]).to(torch.bfloat16)
    w = _bf16_rows(rng, 1, 160)[0]
    y, res = O.add_rms_norm(x.double().numpy(), r.double().numpy(),
                            w.double().numpy(), 1e-6)
    # torch's fp32 add and bf16 conversion as an independent path
    ref = (x.float() + r.float()).to(torch.bfloat16).double().numpy()
    assert np.array_equal(res, ref)
    s = (x.float() + r.float()).double().numpy()
    np.testing.assert_allclose(y, O.rms_norm(s, w.double().numpy(), 1e-6), rtol=1e-15)
    # no residual: the norm of x itself, residual out = x
    y0, res0 = O.add_rms_norm(x.double().numpy(), None, w.double().numpy(), 1e-6)
    assert np.array_equal(res0, x.double().numpy())
    ref0 = torch.nn.functional.rms_norm(x.double(), (160,), w.double(), 1e-6).numpy()
    np.testing.assert_allclose(y0, ref0, rtol=1e-13)


def test_add_rms_norm_outputs():
    rng = np.random.default_rng(8)
    x = _bf16_rows(rng, 4, 128).double().numpy()
    r = _bf16_rows(rng, 4, 128).double().numpy()
    w = _bf16_rows(rng, 1, 128)[0].double().numpy()
    y32, y16, res = O.add_rms_norm_cast(x, r, w, 1e-6)
    y, res2 = O.add_rms_norm(x, r, w, 1e-6)
    # torch's float32 conversion of the exact value, and torch's bfloat16
    # conversion of that float32 value
    t32 = torch.from_numpy(y).float()
    assert np.array_equal(y32, t32.double().numpy())
    assert np.array_equal(y16, t32.to(torch.bfloat16).double().numpy())
    assert np.array_equal(res, res2)
    codes, scales, res3, yq = O.add_rms_norm_mx_quant(x, r, w, 1e-6)
    assert codes.shape == (4, 128) and scales.shape == (4, 4)
    assert np.array_equal(res3, res)
    assert np.array_equal(yq, y32)
    # the codes are torch's float8_e4m3fn conversion (round to nearest even)
    # of the fp32 y divided by the block scale
    c_ref, s_ref = _torch_mxfp8(t32)
    assert np.array_equal(codes, c_ref) and np.array_equal(scales, s_ref)
    # the MX pair reproduces y to within half an e4m3 step at the block scale
    # (values past 448 at that scale saturate)
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(yq) / sc
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)
    bound = np.where(a > 448, a - 448, 0.5 * ulp) * sc
    deq = O.mx_dequant(codes, scales, "e4m3")
    assert np.all(np.abs(deq - yq) <= bound * (1 + 1e-12))


def test_norm_outputs_round_through_fp32(monkeypatch):
    """The bf16 and MXFP8 outputs are taken of the fp32 y, not of the exact
    one: a y just above a rounding midpoint whose fp32 rounding lands on the
    midpoint itself rounds the other way (ties to even)."""
    import oracle.moe_oracle as OM
    y = np.zeros((1, 32))
    y[0, 0] = 300.0                       # block scale 2^0 for the MX output
    y[0, 1] = 1.0 + 2.0 ** -8 + 2.0 ** -30   # fp32: 1 + 2^-8, a bf16 midpoint
    y[0, 2] = 1.0 + 2.0 ** -4 + 2.0 ** -30   # fp32: 1.0625, an e4m3 midpoint
    monkeypatch.setattr(OM, "add_rms_norm", lambda *a: (y.copy(), np.zeros((1, 32))))
    y32, y16, _ = O.add_rms_norm_cast(None, None, None, 0.0)
    assert y32[0, 1] == 1.0 + 2.0 ** -8 and y32[0, 2] == 1.0625
    # bf16: the exact y would round up to 1 + 2^-7; its fp32 value ties to 1.0
    assert y16[0, 1] == 1.0
    codes, scales, _, _ = O.add_rms_norm_mx_quant(None, None, None, 0.0)
    assert scales[0, 0] == 127
    # e4m3: the exact y would round up to 1.125 (0x39); 1.0625 ties to 1.0
    assert codes[0, 2] == 0x38 and codes[0, 1] == 0x38


# ----------------------------------------------------------------- W4A8 h


def _torch_mxfp8(h32):
    """MXFP8 of fp32 rows [n, K] written another way: the block exponent from
    math.frexp of each block's amax, the element codes from torch's
    float8_e4m3fn conversion (round to nearest even) of the fp32 values
    divided by 2^s, clamped to +-448 first (torch does not saturate)."""
    n, K = h32.shape
    hb = h32.double().reshape(n, K // 32, 32)
    amax = hb.abs().amax(-1)
    s = np.zeros((n, K // 32), dtype=np.int64)
    for i in range(n):
        for b in range(K // 32):
            a = float(amax[i, b])
            s[i, b] = (math.frexp(a)[1] - 1 - 8) if a > 0 else -127
    s = np.clip(s, -127, 127)
    scaled = hb / torch.from_numpy(np.ldexp(1.0, s))[..., None]
    codes = scaled.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(n, K).numpy(), (s + 127).astype(np.uint8)


def _golden_h():
    g = _load("mx_h_blocks.json")

    def block(name, key, dtype):
        v = np.zeros(32, dtype=dtype)
        vals = g["blocks"][name][key]
        v[:len(vals)] = vals
        return v
    rows = g["rows"]
    h = np.stack([np.concatenate([block(b, "values", np.float64) for b in r]) for r in rows])
    codes = np.stack([np.concatenate([block(b, "codes", np.int64) for b in r]) for r in rows])
    deq = np.stack([np.concatenate([block(b, "dequant", np.float64) for b in r]) for r in rows])
    scales = np.array([[g["blocks"][b]["scale"] for b in r] for r in rows])
    # negative zeros of the dequantised list
    for i, r in enumerate(rows):
        for j, b in enumerate(r):
            for q, c in enumerate(g["blocks"][b]["codes"]):
                if c == 128:
                    deq[i, 32 * j + q] = -0.0
    return h, codes, scales, deq


def test_mxfp8_h_quantisation_golden(monkeypatch):
    """expert_ffn's W4A8 branch on hand-worked h rows: the SwiGLU output is
    replaced by the rows of the fixture, w2 is the identity, and the codes,
    scales, dequantised h and y must be the fixture's."""
    import oracle.moe_oracle as OM
    h_rows, codes, scales, deq = _golden_h()
    n, I = h_rows.shape
    monkeypatch.setattr(OM, "swiglu", lambda gu: h_rows.copy())
    a = np.zeros((n, 8))
    w13 = np.zeros((8, 2 * I))
    h, (hc, hs), y = O.expert_ffn(a, w13, np.eye(I), act="bf16", act_q="mxfp8")
    assert np.array_equal(hc.astype(np.int64), codes)
    assert np.array_equal(hs.astype(np.int64), scales)
    assert np.array_equal(h, deq) and np.array_equal(np.signbit(h), np.signbit(deq))
    assert np.array_equal(y, deq)


def test_mxfp8_h_matches_torch_float8():
    """expert_ffn's W4A8 branch against a second formulation in torch: h
    formed in float64 with torch's chunk and silu, rounded to fp32, blocks of
    32 along I quantised through float8_e4m3fn; then y = dequantised h @ w2
    rounded to bf16. Quantising the bf16-rounded h, blocking along the other
    axis or skipping the quantisation each change codes on these rows."""
    rng = np.random.default_rng(31)
    n, H, I = 32, 64, 96
    a = O.round_bf16(rng.standard_normal((n, H)))
    w13 = rng.standard_normal((H, 2 * I)) * 0.3
    w2 = rng.standard_normal((I, 40)) * 0.2
    h, (hc, hs), y = O.expert_ffn(a, w13, w2, act="bf16", act_q="mxfp8")

    g, u = torch.chunk(torch.from_numpy(a) @ torch.from_numpy(w13), 2, -1)
    h32 = (torch.nn.functional.silu(g) * u).float()
    c_ref, s_ref = _torch_mxfp8(h32)
    assert np.array_equal(hc, c_ref) and np.array_equal(hs, s_ref)
    dq = (torch.from_numpy(c_ref).view(torch.float8_e4m3fn).double() *
          torch.from_numpy(np.ldexp(1.0, np.repeat(s_ref.astype(np.int64) - 127, 32, 1))))
    assert np.array_equal(h, dq.numpy())
    y_ref = (dq @ torch.from_numpy(w2)).to(torch.bfloat16).double().numpy()
    # the two fp64 products may differ in their last bits, so the bf16
    # roundings may differ by one step where the sum sits on a midpoint
    ulp = np.exp2(np.floor(np.log2(np.abs(y_ref) + 1e-300)) - 7)
    assert np.all(np.abs(y - y_ref) <= ulp)
    assert np.mean(y == y_ref) > 0.99
    # the planted mistakes: bf16 h first, blocks along the rows, no quantising
    c_bf, _ = _torch_mxfp8(h32.to(torch.bfloat16).float())
    assert not np.array_equal(c_bf, c_ref)
    c_t, _ = _torch_mxfp8(h32.T.contiguous())      # blocks of 32 rows
    assert not np.array_equal(c_t.T, c_ref)
    assert not np.array_equal(h, h32.double().numpy())


# ----------------------------------------------------------------- W8A8 int8


def test_int8_quant_closed_forms():
    # amax = 127 * 2^j gives the scale 2^j exactly; codes are then rint(v / 2^j)
    # with ties to even (2.5 -> 2, -3.5 -> -4, 0.5 -> 0, 1.5 -> 2, 126.5 -> 126)
    base = np.array([127.0, 2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0, 3.25, 0.0])
    want = [127, 2, -4, 0, 0, 2, 126, -127, 3, 0]
    for j in (-12, -3, 0, 5):
        codes, sc = O.int8_quant_rows(base[None, :] * 2.0 ** j)
        assert sc.dtype == np.float32 and sc[0] == np.float32(2.0 ** j)
        assert codes.dtype == np.int8 and codes[0].tolist() == want


def test_int8_quant_zero_row_and_sign():
    codes, sc = O.int8_quant_rows(np.zeros((2, 8)))
    assert sc.tolist() == [0.0, 0.0] and not codes.any()
    # one nonzero element: it becomes +-127 and everything else 0
    v = np.zeros((2, 8))
    v[0, 3], v[1, 5] = -0.75, 2.0 ** -66
    codes, sc = O.int8_quant_rows(v)
    assert codes[0, 3] == -127 and codes[1, 5] == 127
    assert np.count_nonzero(codes) == 2


def test_int8_quant_invariants_and_error_bound():
    # every nonzero row uses the full code range (amax / fl(amax/127) rounds to
    # 127), codes keep the sign, and each code is the nearest integer to v/s
    rng = np.random.default_rng(3)
    v = O.round_bf16(rng.standard_normal((64, 256)) * rng.uniform(1e-3, 1e3, (64, 1)))
    codes, sc = O.int8_quant_rows(v)
    c = codes.astype(np.int64)
    assert np.all(np.abs(c).max(axis=1) == 127)
    assert np.all(np.abs(c) <= 127)
    assert np.all((c == 0) | (np.sign(c) == np.sign(v)))
    err = np.abs(v - c * sc.astype(np.float64)[:, None])
    assert np.all(err <= 0.5 * sc[:, None] * (1 + 1e-5))
    # homogeneity: scaling a row by a power of two scales s and keeps codes
    codes2, sc2 = O.int8_quant_rows(v * 2.0 ** -7)
    assert np.array_equal(codes2, codes)
    assert np.array_equal(sc2, (sc.astype(np.float64) * 2.0 ** -7).astype(np.float32))


def test_int8_quant_rejects_non_fp32_input():
    with pytest.raises(ValueError):
        O.int8_quant_rows(np.array([[1.0 + 2.0 ** -40, 1.0]]))


def test_int8_dequant_is_per_output_channel():
    codes = np.array([[1, -2, 3], [4, 5, -6]], dtype=np.int8)   # [N=2, K=3]
    sc = np.array([0.5, 2.0 ** -10], dtype=np.float32)
    w = O.int8_dequant_rows(codes, sc)
    assert w.tolist() == [[0.5, -1.0, 1.5], [4 * 2.0 ** -10, 5 * 2.0 ** -10, -6 * 2.0 ** -10]]


def test_w8a8_expert_is_integer_matmul_then_scales():
    # one W8A8 expert computed another way: int64 products of the codes, the
    # row scale of x and the channel scale of w applied after the sum, SwiGLU,
    # then the row quantisation of h (pinned above) and the same for GEMM2
    rng = np.random.default_rng(11)
    n, H, I = 7, 96, 64
    x = O.round_bf16(rng.standard_normal((n, H)))
    q13 = rng.integers(-127, 128, (2 * I, H)).astype(np.int8)
    s13 = rng.uniform(1e-4, 1e-3, 2 * I).astype(np.float32)
    q2 = rng.integers(-127, 128, (H, I)).astype(np.int8)
    s2 = rng.uniform(1e-4, 1e-3, H).astype(np.float32)
    qx, sx = O.int8_quant_rows(x)
    a = O.int8_dequant_rows(qx, sx)
    w13 = O.int8_dequant_rows(q13, s13).T
    w2 = O.int8_dequant_rows(q2, s2).T
    h, (qh, sh), y = O.expert_ffn(a, w13, w2, act="bf16", act_q="int8", exact=True)

    acc = qx.astype(np.int64) @ q13.astype(np.int64).T            # [n, 2I]
    gu = acc * sx.astype(np.float64)[:, None] * s13.astype(np.float64)[None, :]
    g, u = gu[:, :I], gu[:, I:]
    h_ref = g / (1.0 + np.exp(-g)) * u
    qh_ref, sh_ref = O.int8_quant_rows(h_ref.astype(np.float32))
    assert np.array_equal(qh, qh_ref) and np.array_equal(sh, sh_ref)
    acc2 = qh_ref.astype(np.int64) @ q2.astype(np.int64).T         # [n, H]
    y_ref = acc2 * sh_ref.astype(np.float64)[:, None] * s2.astype(np.float64)[None, :]
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-15)


def test_w8a8_routed_equals_pertoken():
    rng = np.random.default_rng(5)
    T, H, I, n_ffn, n_zero, k = 10, 64, 32, 6, 2, 3
    logits = rng.standard_normal((T, n_ffn + n_zero)).astype(np.float32)
    x = O.round_bf16(rng.standard_normal((T, H)))
    res = O.round_bf16(rng.standard_normal((T, H)))
    Q13 = rng.integers(-127, 128, (n_ffn, 2 * I, H)).astype(np.int8)
    Q2 = rng.integers(-127, 128, (n_ffn, H, I)).astype(np.int8)
    S13 = rng.uniform(1e-4, 1e-3, (n_ffn, 2 * I)).astype(np.float32)
    S2 = rng.uniform(1e-4, 1e-3, (n_ffn, H)).astype(np.float32)

    def get(e):
        return (O.int8_dequant_rows(Q13[e], S13[e]).T.copy(),
                O.int8_dequant_rows(Q2[e], S2[e]).T.copy())
    kw = dict(logits=logits, x=x, get_weights=get, T=T, H=H, I=I, n_ffn=n_ffn,
              n_zero=n_zero, top_k=k, local_begin=0, local_end=n_ffn + n_zero,
              residual=res, act="bf16", act_q="int8")
    r = O.moe_layer(**kw)
    per_tok = O.moe_tokens(range(T), **kw)
    assert np.array_equal(r["out"], per_tok)
    # x is quantised per token: the gathered codes are the token's codes
    qx, sx = O.int8_quant_rows(x)
    tok = r["sorted_copy"][r["row0"]:r["row0"] + r["R"]] // k
    assert np.array_equal(r["x_perm_codes"], qx[tok])
    assert np.array_equal(r["x_perm_scale"], sx[tok])


# ----------------------------------------------------------------- router linear


def test_router_logits_bruteforce_and_closed_forms():
    rng = np.random.default_rng(21)
    y = rng.standard_normal((5, 12)).astype(np.float32)
    w = rng.standard_normal((7, 12)).astype(np.float32)
    got = O.router_logits(y, w)
    want = np.array([[sum(float(y[t, h]) * float(w[e, h]) for h in range(12))
                      for e in range(7)] for t in range(5)])
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    # one-hot weight rows pick single columns of y exactly
    eye = np.zeros((3, 12), np.float32)
    eye[0, 4], eye[1, 0], eye[2, 11] = 1.0, 1.0, -2.0
    sel = O.router_logits(y, eye)
    assert np.array_equal(sel, np.stack([y[:, 4], y[:, 0], -2.0 * y[:, 11]], 1).astype(np.float64))
    with pytest.raises(ValueError):
        O.router_logits(y, w[:, :11])
