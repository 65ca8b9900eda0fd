"""Python binding of the MI355X MoE expert-layer library (libmoe_mi355x.so).

Argument marshalling only: torch tensors supply device pointers and torch's
current HIP stream supplies the stream; every step of the layer runs in the
library's HIP kernels. The library must be built (``__graft_entry__.build()``
or ``python moe_expert_layer_gate_amd/build.py``); importing the binding
without it raises, there is no fallback.

Calls mirror the C ABI in include/moe_mi355x.h:
  gate_topk, init_routing, ffn_up, ffn_down, grouped_ffn, finalize, layer,
  add_rms_norm_cast, add_rms_norm_mx_quant, router_logits.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "MoeProblem", "MoeError", "lib", "problem", "gate_topk",
    "init_routing", "ffn_up", "ffn_down", "grouped_ffn", "finalize", "layer",
    "layer_workspace_bytes", "layer_traced", "SYMBOLS", "STAGES",
    "add_rms_norm_cast", "add_rms_norm_mx_quant", "router_logits",
    "pack_weights", "pack_bf16_weights", "quant_mxfp4_weights",
    "layer_noalloc", "prefetch_weights",
    "NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_F32, MOE_BF16, MOE_MXFP8_E4M3, MOE_MXFP4_E2M1, MOE_INT8 = 0, 1, 2, 3, 4
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED = 0, 1
# the static scratch of moe_layer_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
_LAYOUT = {"rowmajor": MOE_LAYOUT_ROWMAJOR, "packed": MOE_LAYOUT_PACKED}
_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8_E4M3,
       "mxfp4": MOE_MXFP4_E2M1, "int8": MOE_INT8}

SYMBOLS = ["moe_gate_topk", "moe_init_routing", "moe_grouped_ffn", "moe_ffn_up",
           "moe_ffn_down", "moe_finalize", "moe_layer", "moe_layer_traced",
           "moe_layer_noalloc", "moe_prefetch_weights",
           "moe_add_rms_norm_cast", "moe_add_rms_norm_mx_quant",
           "moe_router_logits", "moe_pack_weights", "moe_pack_bf16_weights",
           "moe_quant_mxfp4_weights",
           "moe_status_string",
           "moe_abi_version"]

# stages of moe_layer_traced, in launch order
STAGES = ["gate_topk", "route_count", "route_scan", "route_scatter",
          "route_gather", "gemm1_swiglu", "gemm2", "finalize"]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class MoeProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "H", "I", "n_ffn", "n_zero", "top_k", "local_begin", "local_end",
        "act", "wt", "act_q", "wt_layout")]


_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.POINTER(ctypes.c_size_t)
_pp = ctypes.POINTER(MoeProblem)


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "moe_gate_topk": [_pp, _vp, _vp, _vp, _vp],
        "moe_init_routing": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _sz, _vp],
        "moe_grouped_ffn": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _sz, _vp],
        "moe_ffn_up": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
        "moe_ffn_down": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
        "moe_finalize": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
        "moe_layer": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                      _vp],
        "moe_layer_traced": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _sz, _vp, ctypes.POINTER(ctypes.c_void_p),
                             ctypes.c_int32],
        "moe_layer_noalloc": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
        "moe_prefetch_weights": [_pp, _vp, _vp, _vp, ctypes.c_int32,
                                 ctypes.c_int64, _vp],
    }
    _i32, _f32 = ctypes.c_int32, ctypes.c_float
    sig["moe_add_rms_norm_cast"] = [_i32, _i32, _vp, _vp, _vp, _f32, _vp, _vp,
                                    _vp, _vp]
    sig["moe_add_rms_norm_mx_quant"] = [_i32, _i32, _vp, _vp, _vp, _f32, _vp,
                                        _vp, _vp, _vp]
    sig["moe_router_logits"] = [_i32, _i32, _i32, _vp, _vp, _vp, _vp]
    sig["moe_pack_weights"] = [_i32, _i32, _i32, _vp, _vp, _vp]
    sig["moe_pack_bf16_weights"] = [_i32, _i32, _i32, _i32, _vp, _vp, _vp]
    sig["moe_quant_mxfp4_weights"] = [_i32, _i32, _i32, _vp, _vp, _vp, _vp]
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_abi_version.argtypes = []
    L.moe_abi_version.restype = ctypes.c_int32
    _lib = L
    return L


def problem(shape=None, **kw) -> MoeProblem:
    """Build a MoeProblem from an object with the shape attributes (T, H, I,
    n_ffn, n_zero, top_k, local_begin, local_end, act, wt, act_q with dtype
    names "f32" / "bf16" / "mxfp4" / "mxfp8" / "int8" / "none") and/or
    keywords. wt_layout ("rowmajor" / "packed") defaults to "packed" for
    MXFP4 and int8 weights (the form pack_weights makes) and "rowmajor"
    otherwise; bf16 weights may also be "packed" (the slab order
    pack_bf16_weights makes); the library refuses any other pairing."""
    vals = {}
    for n in ("T", "H", "I", "n_ffn", "n_zero", "top_k", "local_begin",
              "local_end", "act", "wt", "act_q", "wt_layout"):
        if n in kw:
            vals[n] = kw[n]
        elif shape is not None and hasattr(shape, n):
            vals[n] = getattr(shape, n)
    if vals.get("act_q") in (None, "none"):
        vals["act_q"] = vals["act"]
    if vals.get("wt_layout") is None:
        vals["wt_layout"] = ("packed" if vals["wt"] in ("mxfp4", "int8",
                                                         MOE_MXFP4_E2M1, MOE_INT8)
                             else "rowmajor")
    for n in ("act", "wt", "act_q"):
        if isinstance(vals[n], str):
            vals[n] = _DT[vals[n]]
    if isinstance(vals["wt_layout"], str):
        vals["wt_layout"] = _LAYOUT[vals["wt_layout"]]
    return MoeProblem(**vals)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(st: int):
    if st != 0:
        raise MoeError(st, lib().moe_status_string(st).decode())


def _ws_query(fn, *args) -> int:
    n = ctypes.c_size_t(0)
    _check(fn(*args, None, ctypes.byref(n), None))
    return n.value


def _act_dtype(p: MoeProblem):
    return torch.float32 if p.act == MOE_F32 else torch.bfloat16


def gate_topk(p: MoeProblem, logits, topk_ids=None, topk_weight=None):
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((p.T, p.top_k), dtype=torch.int32, device=dev)
    if topk_weight is None:
        topk_weight = torch.empty((p.T, p.top_k), dtype=torch.float32, device=dev)
    _check(lib().moe_gate_topk(ctypes.byref(p), _ptr(logits), _ptr(topk_ids),
                               _ptr(topk_weight), _stream()))
    return topk_ids, topk_weight


def init_routing(p: MoeProblem, topk_ids, x):
    dev = x.device
    E = p.n_ffn + p.n_zero
    N = p.T * p.top_k
    mx = p.act_q == MOE_MXFP8_E4M3
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_copy = torch.empty(N, dtype=torch.int32, device=dev)
    copy_pos = torch.empty(N, dtype=torch.int32, device=dev)
    if mx:
        x_perm = torch.empty((N, p.H), dtype=torch.uint8, device=dev)
        x_scale = torch.empty((N, p.H // 32), dtype=torch.uint8, device=dev)
    elif p.act_q == MOE_INT8:
        x_perm = torch.empty((N, p.H), dtype=torch.int8, device=dev)
        x_scale = torch.empty(N, dtype=torch.float32, device=dev)
    else:
        x_perm = torch.empty((N, p.H), dtype=_act_dtype(p), device=dev)
        x_scale = None
    L = lib()
    args = (ctypes.byref(p), _ptr(topk_ids), _ptr(x), _ptr(counts),
            _ptr(offsets), _ptr(sorted_copy), _ptr(copy_pos), _ptr(x_perm),
            _ptr(x_scale))
    nb = _ws_query(L.moe_init_routing, *args)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(ws.numel())
    _check(L.moe_init_routing(*args, _ptr(ws), ctypes.byref(n), _stream()))
    return dict(counts=counts, offsets=offsets, sorted_copy=sorted_copy,
                copy_pos=copy_pos, x_perm=x_perm, x_perm_scale=x_scale,
                workspace=ws)


def _h_buffers(p: MoeProblem, dev):
    N = p.T * p.top_k
    if p.act_q == MOE_MXFP8_E4M3:
        return (torch.empty((N, p.I), dtype=torch.uint8, device=dev),
                torch.empty((N, p.I // 32), dtype=torch.uint8, device=dev))
    if p.act_q == MOE_INT8:
        return (torch.empty((N, p.I), dtype=torch.int8, device=dev),
                torch.empty(N, dtype=torch.float32, device=dev))
    return torch.empty((N, p.I), dtype=_act_dtype(p), device=dev), None


def ffn_up(p: MoeProblem, offsets, x_perm, x_perm_scale, w13, w13_scale=None):
    dev = offsets.device
    h, hs = _h_buffers(p, dev)
    L = lib()
    args = (ctypes.byref(p), _ptr(offsets), _ptr(x_perm), _ptr(x_perm_scale),
            _ptr(w13), _ptr(w13_scale), _ptr(h), _ptr(hs))
    nb = _ws_query(L.moe_ffn_up, *args)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(ws.numel())
    _check(L.moe_ffn_up(*args, _ptr(ws), ctypes.byref(n), _stream()))
    return h, hs


def ffn_down(p: MoeProblem, offsets, h, h_scale, w2, w2_scale=None):
    dev = offsets.device
    y = torch.empty((p.T * p.top_k, p.H), dtype=_act_dtype(p), device=dev)
    L = lib()
    args = (ctypes.byref(p), _ptr(offsets), _ptr(h), _ptr(h_scale), _ptr(w2),
            _ptr(w2_scale), _ptr(y))
    nb = _ws_query(L.moe_ffn_down, *args)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(ws.numel())
    _check(L.moe_ffn_down(*args, _ptr(ws), ctypes.byref(n), _stream()))
    return y


def grouped_ffn(p: MoeProblem, offsets, x_perm, x_perm_scale, w13, w2,
                w13_scale=None, w2_scale=None):
    dev = offsets.device
    y = torch.empty((p.T * p.top_k, p.H), dtype=_act_dtype(p), device=dev)
    L = lib()
    args = (ctypes.byref(p), _ptr(offsets), _ptr(x_perm), _ptr(x_perm_scale),
            _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(y))
    nb = _ws_query(L.moe_grouped_ffn, *args)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(ws.numel())
    _check(L.moe_grouped_ffn(*args, _ptr(ws), ctypes.byref(n), _stream()))
    return y


def finalize(p: MoeProblem, topk_ids, topk_weight, copy_pos, offsets, y, x,
             residual=None, out=None):
    if out is None:
        out = torch.empty((p.T, p.H), dtype=_act_dtype(p), device=x.device)
    _check(lib().moe_finalize(ctypes.byref(p), _ptr(topk_ids),
                              _ptr(topk_weight), _ptr(copy_pos), _ptr(offsets),
                              _ptr(y), _ptr(x), _ptr(residual), _ptr(out),
                              _stream()))
    return out


def layer_workspace_bytes(p: MoeProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_layer(ctypes.byref(p), None, None, None, None, None, None,
                           None, None, None, ctypes.byref(n), None))
    return n.value


def layer_traced(p: MoeProblem, logits, x, w13, w2, events, w13_scale=None,
                 w2_scale=None, residual=None, out=None, workspace=None):
    """moe_layer with torch.cuda.Event objects (len(STAGES) + 1 of them, or
    None entries) recorded on the current stream around each stage."""
    if out is None:
        out = torch.empty((p.T, p.H), dtype=_act_dtype(p), device=x.device)
    if workspace is None:
        workspace = torch.empty(max(layer_workspace_bytes(p), 1),
                                dtype=torch.uint8, device=x.device)
    handles = []
    for e in events:
        if e is not None and not e.cuda_event:
            e.record()  # torch creates the HIP event lazily, on first record
        handles.append(None if e is None else e.cuda_event)
    arr = (ctypes.c_void_p * len(events))(*handles)
    n = ctypes.c_size_t(workspace.numel())
    _check(lib().moe_layer_traced(ctypes.byref(p), _ptr(logits), _ptr(x),
                                  _ptr(residual), _ptr(w13), _ptr(w13_scale),
                                  _ptr(w2), _ptr(w2_scale), _ptr(out),
                                  _ptr(workspace), ctypes.byref(n), _stream(),
                                  arr, len(events)))
    return out


def layer(p: MoeProblem, logits, x, w13, w2, w13_scale=None, w2_scale=None,
          residual=None, out=None, workspace=None):
    """The whole layer in one library call. `workspace` (uint8 CUDA tensor of
    at least layer_workspace_bytes(p)) may be passed to avoid reallocating."""
    if out is None:
        out = torch.empty((p.T, p.H), dtype=_act_dtype(p), device=x.device)
    if workspace is None:
        workspace = torch.empty(max(layer_workspace_bytes(p), 1),
                                dtype=torch.uint8, device=x.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(lib().moe_layer(ctypes.byref(p), _ptr(logits), _ptr(x),
                           _ptr(residual), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                           _ptr(w2_scale), _ptr(out), _ptr(workspace),
                           ctypes.byref(n), _stream()))
    return out


def layer_noalloc(p: MoeProblem, logits, x, w13, w2, w13_scale=None,
                  w2_scale=None, residual=None, out=None):
    """moe_layer_noalloc: the whole layer with the library's static scratch
    as its workspace (no allocation by the library; `out` may be passed)."""
    if out is None:
        out = torch.empty((p.T, p.H), dtype=_act_dtype(p), device=x.device)
    _check(lib().moe_layer_noalloc(ctypes.byref(p), _ptr(logits), _ptr(x),
                                   _ptr(residual), _ptr(w13), _ptr(w13_scale),
                                   _ptr(w2), _ptr(w2_scale), _ptr(out),
                                   _stream()))
    return out


def prefetch_weights(p: MoeProblem, w13, w2=None, topk_ids=None,
                     max_bytes=64 << 20, which=None):
    """moe_prefetch_weights on the current stream: read ahead up to
    max_bytes of the weight heads the layer's grouped GEMMs read first
    (which: 1 = w13, 2 = w2, 3 = both; default w13, and w2 when given)."""
    if which is None:
        which = 1 | (2 if w2 is not None else 0)
    _check(lib().moe_prefetch_weights(ctypes.byref(p), _ptr(topk_ids), _ptr(w13),
                                      _ptr(w2), int(which), int(max_bytes),
                                      _stream()))


def _norm_args(x, residual, norm_weight):
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a [T, H] bfloat16 tensor")
    T, H = x.shape
    if residual is not None and (residual.shape != x.shape or residual.dtype != x.dtype):
        raise ValueError("residual must match x")
    if norm_weight.shape != (H,) or norm_weight.dtype != torch.bfloat16:
        raise ValueError("norm_weight must be a [H] bfloat16 tensor")
    return T, H


def add_rms_norm_cast(x, residual, norm_weight, eps: float, want_f32=True,
                      want_bf16=True, want_residual=True):
    """Residual add + RMSNorm with fp32 and bf16 outputs.
    Returns (y_f32 or None, y_bf16 or None, residual_out or None)."""
    T, H = _norm_args(x, residual, norm_weight)
    y32 = torch.empty((T, H), dtype=torch.float32, device=x.device) if want_f32 else None
    y16 = torch.empty((T, H), dtype=torch.bfloat16, device=x.device) if want_bf16 else None
    res = torch.empty_like(x) if want_residual else None
    _check(lib().moe_add_rms_norm_cast(T, H, _ptr(x), _ptr(residual),
                                       _ptr(norm_weight), float(eps), _ptr(y32),
                                       _ptr(y16), _ptr(res), _stream()))
    return y32, y16, res


def add_rms_norm_mx_quant(x, residual, norm_weight, eps: float,
                          want_residual=True):
    """Residual add + RMSNorm with MXFP8 output.
    Returns (codes uint8 [T, H], scales uint8 [T, H/32], residual_out or None)."""
    T, H = _norm_args(x, residual, norm_weight)
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, H // 32 if H % 32 == 0 else 1), dtype=torch.uint8,
                         device=x.device)
    res = torch.empty_like(x) if want_residual else None
    _check(lib().moe_add_rms_norm_mx_quant(T, H, _ptr(x), _ptr(residual),
                                           _ptr(norm_weight), float(eps),
                                           _ptr(codes), _ptr(scales), _ptr(res),
                                           _stream()))
    return codes, scales, res


def router_logits(y, w_router, out=None):
    """fp32 router logits [T, E] = y [T, H] @ w_router [E, H]^T."""
    if y.dim() != 2 or y.dtype != torch.float32:
        raise ValueError("y must be a [T, H] float32 tensor")
    T, H = y.shape
    if w_router.dim() != 2 or w_router.dtype != torch.float32 or w_router.shape[1] != H:
        raise ValueError("w_router must be an [E, H] float32 tensor")
    E = w_router.shape[0]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=y.device)
    _check(lib().moe_router_logits(T, H, E, _ptr(y), _ptr(w_router), _ptr(out),
                                   _stream()))
    return out


def pack_weights(w, out=None):
    """Quantised expert weights -- int8 [E, N, K] or MXFP4 codes uint8
    [E, N, K/2], K contiguous -> the packed order the int8 and MX GEMMs read
    (same shape and bytes; see moe_pack_weights)."""
    if w.dim() != 3 or w.dtype not in (torch.int8, torch.uint8):
        raise ValueError("w must be an [E, N, K_bytes] int8 or uint8 tensor")
    E, N, Kb = w.shape
    if out is None:
        out = torch.empty_like(w)
    _check(lib().moe_pack_weights(E, N, Kb, _ptr(w), _ptr(out), _stream()))
    return out


def pack_bf16_weights(w, glu, out=None):
    """bf16 expert weights [E, K, N] (row-major, N contiguous) -> the slab
    order the bf16 GEMMs read with wt_layout="packed" (same shape and element
    count; see moe_pack_bf16_weights). glu: True for w13 (gate and up columns
    paired per slab), False for w2."""
    if w.dim() != 3 or w.dtype != torch.bfloat16:
        raise ValueError("w must be an [E, K, N] bfloat16 tensor")
    E, K, N = w.shape
    if out is None:
        out = torch.empty_like(w)
    _check(lib().moe_pack_bf16_weights(E, K, N, 1 if glu else 0, _ptr(w),
                                       _ptr(out), _stream()))
    return out


def quant_mxfp4_weights(w, codes=None, scales=None):
    """bf16 expert weights [E, K, N] (N contiguous) -> MXFP4 codes uint8
    [E, N, K/2] (low nibble = even k) and e8m0 scales uint8 [E, N, K/32]
    (see moe_quant_mxfp4_weights). The codes are row-major; pack_weights
    turns them into the order the GEMMs read."""
    if w.dim() != 3 or w.dtype != torch.bfloat16:
        raise ValueError("w must be an [E, K, N] bfloat16 tensor")
    E, K, N = w.shape
    if codes is None:
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=w.device)
    _check(lib().moe_quant_mxfp4_weights(E, K, N, _ptr(w), _ptr(codes),
                                         _ptr(scales), _stream()))
    return codes, scales
