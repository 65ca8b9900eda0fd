"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, and rejects bad arguments on the host
before launching anything."""
import ctypes
import os
import re

import pytest

import moe_expert_layer_gate_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(m.LIB_PATH):
        from moe_expert_layer_gate_amd import build
        build.build(verbose=False)
    return m.lib()


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*MOE_API\s+(?:moe_status|const char\*|int32_t)\s+(moe_\w+)\s*\(",
                                 txt, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("moe_gate_topk", "moe_init_routing", "moe_grouped_ffn",
              "moe_finalize", "moe_layer"):
        assert n in names
    assert set(names) == set(m.SYMBOLS)


def test_every_declared_symbol_is_exported(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    for s in range(5):
        assert L.moe_status_string(s)
    assert L.moe_status_string(99) == b"unknown moe_status"
    assert L.moe_abi_version() >= 100


def _p(**kw):
    base = dict(T=32, H=2048, I=768, n_ffn=128, n_zero=0, top_k=8,
                local_begin=0, local_end=128, act="bf16", wt="bf16", act_q="none")
    base.update(kw)
    return m.problem(**base)


def _query(L, p):
    n = ctypes.c_size_t(0)
    st = L.moe_layer(ctypes.byref(p), None, None, None, None, None, None, None,
                     None, None, ctypes.byref(n), None)
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), 1), (dict(top_k=129), 1), (dict(T=-1), 1), (dict(H=0), 1),
    (dict(local_begin=5, local_end=5), 1), (dict(local_end=129), 1),
    (dict(n_ffn=0, n_zero=0), 1), (dict(H=2000), 2), (dict(I=100), 2),
    (dict(n_ffn=4096, local_end=4096), 2), (dict(top_k=65, n_ffn=128), 2),
    (dict(act="f32"), 2), (dict(wt="mxfp4"), 2),
    (dict(wt="mxfp4", act_q="mxfp8", H=2048 + 32), 2),
    # W8A8 needs int8 on both sides, H and I multiples of 128 and
    # 2 * I * H < 2^31
    (dict(wt="int8"), 2), (dict(act_q="int8"), 2),
    (dict(wt="int8", act_q="mxfp8"), 2),
    (dict(wt="int8", act_q="int8", H=2048 + 64), 2),
    (dict(wt="int8", act_q="int8", I=768 + 32), 2),
    (dict(wt="int8", act_q="int8", H=32768, I=32768), 2),
])
def test_invalid_problems_rejected_on_host(L, kw, status):
    st, _ = _query(L, _p(**kw))
    assert st == status


def test_workspace_query_and_too_small(L):
    p = _p()
    st, need = _query(L, p)
    assert st == 0 and need > 0
    # grows with T; W4A8 needs its MX buffers
    _, need2 = _query(L, _p(T=64))
    assert need2 > need
    st, _ = _query(L, _p(wt="mxfp4", act_q="mxfp8", H=4096, I=1536,
                         local_begin=32, local_end=64))
    assert st == 0
    # W8A8 adds the int8 codes of x, fp32 h and its int8 codes
    st, need8 = _query(L, _p(wt="int8", act_q="int8"))
    assert st == 0 and need8 > need
    # a buffer smaller than required is refused before any launch
    n = ctypes.c_size_t(need - 1)
    st = L.moe_layer(ctypes.byref(p), None, None, None, None, None, None, None,
                     None, ctypes.c_void_p(1 << 20), ctypes.byref(n), None)
    assert st == 3


def test_missing_pointers_rejected(L):
    p = _p()
    _, need = _query(L, p)
    n = ctypes.c_size_t(need)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: checks come first
    st = L.moe_layer(ctypes.byref(p), None, fake, None, fake, None, fake, None,
                     fake, fake, ctypes.byref(n), None)
    assert st == 1  # logits missing
    st = L.moe_layer(ctypes.byref(p), fake, fake, None, fake, fake, fake, None,
                     fake, fake, ctypes.byref(n), None)
    assert st == 1  # scale given for bf16 weights
    st = L.moe_gate_topk(ctypes.byref(p), None, fake, fake, None)
    assert st == 1
    # W8A8 weights without their channel scales
    p8 = _p(wt="int8", act_q="int8")
    _, need8 = _query(L, p8)
    n8 = ctypes.c_size_t(need8)
    st = L.moe_layer(ctypes.byref(p8), fake, fake, None, fake, None, fake, None,
                     fake, fake, ctypes.byref(n8), None)
    assert st == 1
    st = L.moe_finalize(ctypes.byref(p), fake, fake, None, fake, fake, fake,
                        None, fake, None)
    assert st == 1


def test_null_problem(L):
    assert L.moe_gate_topk(None, None, None, None, None) == 1


def test_fused_norm_host_checks(L):
    """Argument checks of the fused-norm calls happen before any launch."""
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails a check
    cast, mxq = L.moe_add_rms_norm_cast, L.moe_add_rms_norm_mx_quant
    # H not a multiple of 32, or past 8192 columns: unsupported
    assert cast(4, 100, fake, None, fake, 1e-6, fake, fake, None, None) == 2
    assert cast(4, 8224, fake, None, fake, 1e-6, fake, fake, None, None) == 2
    assert mxq(4, 48, fake, None, fake, 1e-6, fake, fake, None, None) == 2
    # bad sizes / epsilon
    assert cast(-1, 64, fake, None, fake, 1e-6, fake, fake, None, None) == 1
    assert cast(4, 0, fake, None, fake, 1e-6, fake, fake, None, None) == 1
    assert cast(4, 64, fake, None, fake, -1.0, fake, fake, None, None) == 1
    assert cast(4, 64, fake, None, fake, float("nan"), fake, fake, None, None) == 1
    assert mxq(4, 64, fake, None, fake, float("inf"), fake, fake, None, None) == 1
    # missing inputs or outputs
    assert cast(4, 64, None, None, fake, 1e-6, fake, fake, None, None) == 1
    assert cast(4, 64, fake, None, None, 1e-6, fake, fake, None, None) == 1
    assert cast(4, 64, fake, None, fake, 1e-6, None, None, fake, None) == 1
    assert mxq(4, 64, fake, None, fake, 1e-6, None, fake, None, None) == 1
    assert mxq(4, 64, fake, None, fake, 1e-6, fake, None, None, None) == 1
    # no rows: nothing to do, nothing launched
    assert cast(0, 64, None, None, None, 1e-6, None, None, None, None) == 0
    assert mxq(0, 64, None, None, None, 1e-6, None, None, None, None) == 0


def test_router_host_checks(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails a check
    r = L.moe_router_logits
    assert r(-1, 64, 32, fake, fake, fake, None) == 1
    assert r(4, 0, 32, fake, fake, fake, None) == 1
    assert r(4, 64, 0, fake, fake, fake, None) == 1
    assert r(4, 40, 32, fake, fake, fake, None) == 2     # H % 16
    assert r(4, 64, 48, fake, fake, fake, None) == 2     # E % 32
    assert r(4, 64, 4096, fake, fake, fake, None) == 2   # E > 2048
    assert r(4, 64, 32, None, fake, fake, None) == 1
    assert r(4, 64, 32, fake, None, fake, None) == 1
    assert r(4, 64, 32, fake, fake, None, None) == 1
    assert r(0, 64, 32, None, None, None, None) == 0


def test_misaligned_pointers_rejected(L):
    """Array pointers must be 16-byte aligned and the workspace 256-byte
    aligned; a misaligned one is refused on the host (never dereferenced)."""
    ok = ctypes.c_void_p(1 << 20)
    bad = ctypes.c_void_p((1 << 20) + 2)      # not 16-byte aligned
    ws_bad = ctypes.c_void_p((1 << 20) + 16)  # 16- but not 256-byte aligned
    p = _p()
    _, need = _query(L, p)
    n = ctypes.c_size_t(need)
    lay = L.moe_layer
    # logits, x, residual, w13, w13_scale, w2, w2_scale, out, workspace
    assert lay(ctypes.byref(p), bad, ok, None, ok, None, ok, None, ok, ok,
               ctypes.byref(n), None) == 1
    assert lay(ctypes.byref(p), ok, bad, None, ok, None, ok, None, ok, ok,
               ctypes.byref(n), None) == 1
    assert lay(ctypes.byref(p), ok, ok, bad, ok, None, ok, None, ok, ok,
               ctypes.byref(n), None) == 1
    assert lay(ctypes.byref(p), ok, ok, None, ok, None, bad, None, ok, ok,
               ctypes.byref(n), None) == 1
    assert lay(ctypes.byref(p), ok, ok, None, ok, None, ok, None, bad, ok,
               ctypes.byref(n), None) == 1
    assert lay(ctypes.byref(p), ok, ok, None, ok, None, ok, None, ok, ws_bad,
               ctypes.byref(n), None) == 1
    assert L.moe_gate_topk(ctypes.byref(p), bad, ok, ok, None) == 1
    assert L.moe_gate_topk(ctypes.byref(p), ok, ok, bad, None) == 1
    # finalize: topk_ids, topk_weight, copy_pos, offsets, y, x, residual, out
    assert L.moe_finalize(ctypes.byref(p), ok, ok, ok, ok, bad, ok, None, ok,
                          None) == 1
    assert L.moe_finalize(ctypes.byref(p), ok, ok, ok, ok, ok, ok, None, bad,
                          None) == 1
    # grouped FFN: offsets, x_perm, x_perm_scale, w13, w13_scale, w2,
    # w2_scale, y, workspace
    ng = ctypes.c_size_t(0)
    assert L.moe_grouped_ffn(ctypes.byref(p), None, None, None, None, None,
                             None, None, None, None, ctypes.byref(ng), None) == 0
    assert L.moe_grouped_ffn(ctypes.byref(p), ok, ok, None, bad, None, ok,
                             None, ok, ok, ctypes.byref(ng), None) == 1
    assert L.moe_grouped_ffn(ctypes.byref(p), ok, ok, None, ok, None, ok,
                             None, ok, ws_bad, ctypes.byref(ng), None) == 1
    # routing: topk_ids, x, tokens_per_expert, offsets, sorted_copy,
    # copy_pos, x_perm, x_perm_scale, workspace
    nr = ctypes.c_size_t(0)
    assert L.moe_init_routing(ctypes.byref(p), None, None, None, None, None,
                              None, None, None, None, ctypes.byref(nr),
                              None) == 0
    assert L.moe_init_routing(ctypes.byref(p), ok, ok, ok, ok, ok, ok, bad,
                              None, ok, ctypes.byref(nr), None) == 1
    assert L.moe_router_logits(4, 64, 32, ok, bad, ok, None) == 1
    assert L.moe_add_rms_norm_cast(4, 64, bad, None, ok, 1e-6, ok, ok, None,
                                   None) == 1
    assert L.moe_add_rms_norm_mx_quant(4, 64, ok, None, ok, 1e-6, ok, bad,
                                       None, None) == 1


def test_pack_weights_host_checks(L):
    ok = ctypes.c_void_p(1 << 20)
    far = ctypes.c_void_p(1 << 30)
    pk = L.moe_pack_weights
    assert pk(-1, 32, 128, ok, far, None) == 1
    assert pk(2, 0, 128, ok, far, None) == 1
    assert pk(2, 24, 128, ok, far, None) == 2         # N % 16
    assert pk(2, 32, 96, ok, far, None) == 2          # K_bytes % 64
    assert pk(2, 1 << 16, 1 << 15, ok, far, None) == 2  # N * K >= 2^31
    assert pk(2, 32, 128, None, far, None) == 1
    assert pk(2, 32, 128, ok, ctypes.c_void_p((1 << 30) + 8), None) == 1  # misaligned
    assert pk(2, 32, 128, ok, ctypes.c_void_p((1 << 20) + 4096), None) == 1  # overlap
    assert pk(0, 32, 128, None, None, None) == 0     # nothing to do


@pytest.mark.parametrize("kw,layout,status", [
    (dict(wt="mxfp4", act_q="mxfp8", H=4096, I=1536), "rowmajor", 2),
    (dict(wt="int8", act_q="int8"), "rowmajor", 2),
    (dict(act="f32", wt="f32", act_q="f32"), "packed", 2),
    (dict(I=736), "packed", 2),            # bf16 slabs: I % 128
    (dict(H=2080, I=768), "packed", 2),    # bf16 slabs: H % 256
    (dict(wt="mxfp4", act_q="mxfp8", H=4096, I=1536), "packed", 0),
    (dict(wt="int8", act_q="int8"), "packed", 0),
    (dict(), "packed", 0),
    (dict(), "rowmajor", 0),
    (dict(I=736), "rowmajor", 0),
])
def test_weight_layout_declared(L, kw, layout, status):
    """Quantised weights are read only in the packed order, fp32 ones only
    row-major, bf16 ones either way (packed: whole 256-column slabs): any
    other problem is refused before any launch, by every entry point that
    takes the problem."""
    p = _p(wt_layout=layout, **kw)
    st, _ = _query(L, p)
    assert st == status
    if status:
        fake = ctypes.c_void_p(1 << 20)  # never dereferenced
        assert L.moe_gate_topk(ctypes.byref(p), fake, fake, fake, None) == status
        n = ctypes.c_size_t(0)
        assert L.moe_grouped_ffn(ctypes.byref(p), None, None, None, None, None,
                                 None, None, None, None, ctypes.byref(n),
                                 None) == status


def test_pack_bf16_weights_host_checks(L):
    ok = ctypes.c_void_p(1 << 20)
    far = ctypes.c_void_p(1 << 34)
    pk = L.moe_pack_bf16_weights
    assert pk(-1, 64, 256, 1, ok, far, None) == 1
    assert pk(2, 0, 256, 1, ok, far, None) == 1
    assert pk(2, 64, 0, 0, ok, far, None) == 1
    assert pk(2, 64, 256, 2, ok, far, None) == 1       # glu 0 or 1
    assert pk(2, 48, 256, 1, ok, far, None) == 2       # K % 32
    assert pk(2, 64, 384, 0, ok, far, None) == 2       # N % 256
    assert pk(1 << 12, 1 << 14, 1 << 14, 0, ok, far, None) == 2  # E*K*N >= 2^40
    assert pk(2, 64, 256, 1, None, far, None) == 1
    assert pk(2, 64, 256, 1, ok, ctypes.c_void_p((1 << 34) + 8), None) == 1  # misaligned
    assert pk(2, 64, 256, 1, ok, ctypes.c_void_p((1 << 20) + 4096), None) == 1  # overlap
    assert pk(0, 64, 256, 1, None, None, None) == 0    # nothing to do


def test_quant_mxfp4_weights_host_checks(L):
    ok = ctypes.c_void_p(1 << 20)
    q = L.moe_quant_mxfp4_weights
    assert q(-1, 64, 16, ok, ok, ok, None) == 1
    assert q(2, 0, 16, ok, ok, ok, None) == 1
    assert q(2, 64, 0, ok, ok, ok, None) == 1
    assert q(2, 48, 16, ok, ok, ok, None) == 2          # K % 32
    assert q(1 << 10, 1 << 15, 1 << 15, ok, ok, ok, None) == 2  # E*N*K >= 2^40
    assert q(2, 64, 16, None, ok, ok, None) == 1
    assert q(2, 64, 16, ok, None, ok, None) == 1
    assert q(2, 64, 16, ok, ok, None, None) == 1
    assert q(2, 64, 16, ok, ctypes.c_void_p((1 << 20) + 8), ok, None) == 1
    assert q(0, 64, 16, None, None, None, None) == 0    # nothing to do


def test_prefetch_weights_host_checks(L):
    ok = ctypes.c_void_p(1 << 20)  # never dereferenced: every case returns first
    pf = L.moe_prefetch_weights
    p = _p()
    assert pf(ctypes.byref(p), None, ok, ok, 4, 1 << 20, None) == 1    # which
    assert pf(ctypes.byref(p), None, ok, ok, 1, -1, None) == 1         # bytes
    assert pf(ctypes.byref(p), None, None, ok, 1, 1 << 20, None) == 1  # no w13
    assert pf(ctypes.byref(p), None, ok, None, 2, 1 << 20, None) == 1  # no w2
    assert pf(ctypes.byref(p), None, ctypes.c_void_p((1 << 20) + 4), ok, 1,
              1 << 20, None) == 1                                      # misaligned
    assert pf(ctypes.byref(_p(act="f32", wt="f32", act_q="f32")), None, ok, ok,
              1, 1 << 20, None) == 2
    assert pf(ctypes.byref(_p(top_k=0)), None, ok, ok, 1, 1 << 20, None) == 1
    # nothing to read: no launch
    assert pf(ctypes.byref(p), None, None, None, 0, 1 << 20, None) == 0
    assert pf(ctypes.byref(p), None, ok, ok, 3, 8, None) == 0
    assert pf(ctypes.byref(_p(T=0)), None, ok, ok, 3, 1 << 20, None) == 0


def test_header_is_plain_c(L, tmp_path):
    """include/moe_mi355x.h is a C ABI: a C99 translation unit (strict,
    warnings as errors) includes it, links against the library and calls
    into it -- a size query of an invalid problem, which fails on the host
    before anything touches a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = tmp_path / "abi.c"
    src.write_text(
        '#include "moe_mi355x.h"\n'
        '#include <stdio.h>\n'
        'int main(void) {\n'
        '  moe_problem p = {0};\n'
        '  size_t n = 0;\n'
        '  moe_status s = moe_layer(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, &n, 0);\n'
        '  printf("%d %d %s\\n", (int)s, (int)moe_abi_version(),\n'
        '         moe_status_string(s));\n'
        '  return 0;\n'
        '}\n')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(m.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic",
                        "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-L", libdir, "-lmoe_mi355x",
                        "-Wl,-rpath," + libdir, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    status, version, text = r.stdout.split(" ", 2)
    assert int(status) == 1 and int(version) == L.moe_abi_version()
    assert text.startswith("MOE_ERR_INVALID_ARG")
