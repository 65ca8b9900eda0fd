"""Property pins of the CPU oracle (test infrastructure; no GPU).

* MX encoding, exhaustively: every finite bf16 value, in blocks of 32 --
  consecutive bit patterns (one binade per block: the top of the element
  range and its saturation) and seeded shuffles of all of them (wide blocks:
  subnormal codes, flushes to signed zero) -- against facts that do not come
  from the oracle: the block exponent read off the bf16 bit fields, torch's
  float8_e4m3fn conversion (round to nearest even) inside the e4m3 range
  with saturation to +-448 outside it (OCP MX v1.0), and a brute-force
  nearest-value search with ties to the even code for e2m1.
* Random small layers (hypothesis): the k selected experts are the k
  largest logits with ties to the lower id, in that order, their weights a
  softmax that sums to 1; routing is a stable permutation with its inverse;
  the routed layer equals per-token and dense evaluation; outputs over a
  partition of the expert range add up to the full-range output.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O

# ----------------------------------------------------------------- MX


def _finite_bf16():
    """Every finite bf16 value, by bit pattern (65280 = 2040 blocks of 32)."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    keep = np.isfinite(f)
    return f[keep].astype(np.float64), bits[keep]


def _block_exponent(bits_block):
    """floor(log2(amax)) of a block of bf16 bit patterns, from the fields:
    exponent e - 127 for normals, the mantissa's top bit - 133 for
    subnormals; None for an all-zero block."""
    mag = bits_block & 0x7FFF
    m = int(mag.max())
    if m == 0:
        return None
    e = m >> 7
    if e:
        return e - 127
    return (m & 0x7F).bit_length() - 1 - 133


def _blocks(order):
    v, bits = _finite_bf16()
    v, bits = v[order], bits[order]
    return v.reshape(-1, 32), bits.reshape(-1, 32)


def _orders():
    n = _finite_bf16()[0].size
    rng = np.random.default_rng(2024)
    return [np.arange(n)] + [rng.permutation(n) for _ in range(3)]


def test_mx_e4m3_every_finite_bf16():
    for order in _orders():
        v, bits = _blocks(order)
        codes, sc = O.mx_quant(v, "e4m3")
        for b in range(v.shape[0]):
            fl = _block_exponent(bits[b])
            s = -127 if fl is None else min(max(fl - 8, -127), 127)
            assert int(sc[b, 0]) == s + 127
            q = v[b] / 2.0 ** s  # exact: v is bf16, s an integer
            sat = np.abs(q) > 448
            ref = torch.from_numpy(q.astype(np.float32)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
            ref = np.where(sat, np.where(np.signbit(q), 0xFE, 0x7E), ref)
            assert np.array_equal(codes[b], ref), (b, v[b], codes[b], ref)


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_bruteforce(q):
    """Nearest of the 8 magnitudes, ties to the even code, sign copied."""
    a = np.abs(q)
    d = np.abs(a[:, None] - _E2M1[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes take the even one (codes 0..7: even = bit 0 clear)
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = np.where(a > 6.0, 7, code)
    return (code | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


def test_mx_e2m1_every_finite_bf16():
    for order in _orders():
        v, bits = _blocks(order)
        codes, sc = O.mx_quant(v, "e2m1")
        for b in range(v.shape[0]):
            fl = _block_exponent(bits[b])
            s = -127 if fl is None else min(max(fl - 2, -127), 127)
            assert int(sc[b, 0]) == s + 127
            want = _e2m1_bruteforce(v[b] / 2.0 ** s)
            assert np.array_equal(codes[b], want), (b, v[b], codes[b], want)


# ----------------------------------------------------------------- layer


def _problem(data):
    n_ffn = data.draw(st.integers(1, 6), label="n_ffn")
    n_zero = data.draw(st.integers(0, 3), label="n_zero")
    E = n_ffn + n_zero
    k = data.draw(st.integers(1, min(E, 5)), label="k")
    T = data.draw(st.integers(1, 9), label="T")
    H = data.draw(st.sampled_from([16, 32]), label="H")
    I = data.draw(st.sampled_from([8, 16]), label="I")
    seed = data.draw(st.integers(0, 1 << 16), label="seed")
    ties = data.draw(st.booleans(), label="ties")
    rng = np.random.default_rng(seed)
    if ties:  # small integers: many equal logits
        logits = rng.integers(-2, 3, (T, E)).astype(np.float32)
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, H))
    W13 = rng.standard_normal((n_ffn, H, 2 * I)) * 0.1
    W2 = rng.standard_normal((n_ffn, I, H)) * 0.1
    res = rng.standard_normal((T, H)) if data.draw(st.booleans(), label="res") else None
    return dict(logits=logits, x=x, get_weights=lambda e: (W13[e], W2[e]), T=T,
                H=H, I=I, n_ffn=n_ffn, n_zero=n_zero, top_k=k, local_begin=0,
                local_end=E, residual=res)


_SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                     suppress_health_check=[HealthCheck.too_slow])


@_SETTINGS
@given(st.data())
def test_gate_and_routing_properties(data):
    kw = _problem(data)
    T, E, k = kw["T"], kw["n_ffn"] + kw["n_zero"], kw["top_k"]
    ids, w = O.gate_topk(kw["logits"], k)
    L = kw["logits"]
    for t in range(T):
        want = sorted(range(E), key=lambda e: (-float(L[t, e]), e))[:k]
        assert ids[t].tolist() == want
        assert abs(w[t].sum() - 1.0) <= 1e-12
        assert np.all(w[t] > 0) and np.all(np.diff(w[t]) <= 1e-15)
        ref = np.exp(L[t, want].astype(np.float64) - L[t, want[0]])
        np.testing.assert_allclose(w[t], ref / ref.sum(), rtol=1e-13)
    counts, offsets, sc, cp = O.init_routing(ids, E)
    flat = ids.reshape(-1)
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert np.array_equal(offsets[1:] - offsets[:-1], counts)
    assert np.all(np.diff(flat[sc]) >= 0)
    for e in range(E):  # stable: copies of one expert in increasing order
        seg = sc[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)
    assert np.array_equal(cp[sc], np.arange(T * k))


@_SETTINGS
@given(st.data())
def test_layer_properties(data):
    kw = _problem(data)
    E = kw["n_ffn"] + kw["n_zero"]
    routed = O.moe_layer(act="f32", exact=True, **kw)["out"]
    dense = O.moe_dense(**kw)
    per_tok = O.moe_tokens(range(kw["T"]), act="f32", exact=True, **kw)
    np.testing.assert_allclose(routed, dense, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(per_tok, dense, rtol=1e-11, atol=1e-11)
    # a random partition of the expert range: partial outputs (no residual)
    # add up to the full output
    cuts = sorted(set(data.draw(st.lists(st.integers(1, E - 1), max_size=3),
                                label="cuts"))) if E > 1 else []
    bounds = [0] + cuts + [E]
    parts = sum(O.moe_layer(act="f32", exact=True,
                            **dict(kw, residual=None, local_begin=b,
                                   local_end=e))["out"]
                for b, e in zip(bounds[:-1], bounds[1:]))
    full = routed - (0 if kw["residual"] is None else kw["residual"])
    np.testing.assert_allclose(parts, full, rtol=1e-11, atol=1e-11)
