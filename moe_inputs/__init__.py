"""Seeded synthetic inputs for the MoE expert layer.

This module is the only code shared by the HIP path (tests, bench) and the CPU
oracle. It draws random tensors and holds none of the layer's arithmetic: no
gating, routing, quantisation, GEMM or reduction happens here.

Workloads are named by what they are. Their shapes follow the models the source
pages optimise (Qwen3-MoE on Atlas A3/950 and LongCat-Flash on Atlas A3); the
values are synthetic because trained weights are not available.

Distributions ("N(0, s)" means standard deviation s):
  * router logits: fp32 N(0,1); the skewed prefill workload adds a per-expert
    bias N(0,1.5) drawn once per seed (heavy expert load imbalance);
  * hidden states x and residual: N(0,1) rounded to the activation dtype;
  * bf16/fp32 expert weights: N(0, w_std) rounded to the weight dtype;
  * MXFP4 expert weights (W4A8): drawn as bf16 N(0, w_std) like the bf16
    workloads; each side quantises them to MXFP4 itself (the library with its
    weight-quantisation call at load time, the oracle with its own MX
    quantiser), so no quantisation arithmetic lives here.
  * int8 expert weights (W8A8): codes N(0, 32) rounded and clipped to
    [-127, 127] (a per-channel amax near 127, as symmetric quantisation of a
    Gaussian column gives) with one fp32 scale per output channel drawn
    uniformly from [0.75, 1.25] * 0.02 / 32, so elements are again about
    N(0, 0.02).

Generation uses torch's seeded generator on the requested device, so the same
(workload, seed, device) always gives the same tensors; the CPU oracle receives
host copies of exactly the tensors the GPU path consumes.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional

import torch

__all__ = ["MoEShape", "WORKLOADS", "get_workload", "generate", "seed_for",
           "scaled", "generate_norm", "generate_router", "NORM_EPS"]


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int            # tokens
    H: int            # hidden size (GEMM1 K, GEMM2 N)
    I: int            # per-expert intermediate size
    n_ffn: int        # FFN experts, ids [0, n_ffn)
    n_zero: int       # identity ("zero-compute") experts, ids [n_ffn, n_ffn+n_zero)
    top_k: int
    local_begin: int  # expert range [local_begin, local_end) handled by the call
    local_end: int
    act: str          # "f32" | "bf16"  (x, residual, y, out)
    wt: str           # "f32" | "bf16" | "mxfp4" | "int8"
    act_q: str        # "none" | "mxfp8" | "int8" (dynamic activation quantisation)
    w_std: float = 0.02
    logit_bias_std: float = 0.0
    residual: bool = False

    @property
    def E_tot(self) -> int:
        return self.n_ffn + self.n_zero

    @property
    def ffn_begin(self) -> int:
        return min(self.local_begin, self.n_ffn)

    @property
    def ffn_end(self) -> int:
        return min(self.local_end, self.n_ffn)

    @property
    def E_loc(self) -> int:
        """FFN experts whose weights the call holds."""
        return max(0, self.ffn_end - self.ffn_begin)

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, MoEShape] = {
    s.name: s for s in [
        MoEShape("tiny_fp32", T=16, H=64, I=32, n_ffn=8, n_zero=0, top_k=2,
                 local_begin=0, local_end=8, act="f32", wt="f32", act_q="none",
                 w_std=0.05),
        MoEShape("qwen3_30b_a3b_decode_bf16", T=32, H=2048, I=768, n_ffn=128,
                 n_zero=0, top_k=8, local_begin=0, local_end=128, act="bf16",
                 wt="bf16", act_q="none"),
        MoEShape("qwen3_30b_a3b_prefill_skewed_bf16", T=4096, H=2048, I=768,
                 n_ffn=128, n_zero=0, top_k=8, local_begin=0, local_end=128,
                 act="bf16", wt="bf16", act_q="none", logit_bias_std=1.5,
                 residual=True),
        MoEShape("longcat_flash_zero_experts_bf16", T=1024, H=6144, I=2048,
                 n_ffn=512, n_zero=256, top_k=12, local_begin=0, local_end=768,
                 act="bf16", wt="bf16", act_q="none"),
        MoEShape("qwen3_235b_a22b_ep_rank_w4a8", T=4096, H=4096, I=1536,
                 n_ffn=128, n_zero=0, top_k=8, local_begin=32, local_end=64,
                 act="bf16", wt="mxfp4", act_q="mxfp8"),
        # W8A8 routed experts on the Qwen3-30B-A3B shapes
        MoEShape("qwen3_30b_a3b_decode_w8a8", T=32, H=2048, I=768, n_ffn=128,
                 n_zero=0, top_k=8, local_begin=0, local_end=128, act="bf16",
                 wt="int8", act_q="int8"),
        MoEShape("qwen3_30b_a3b_prefill_skewed_w8a8", T=4096, H=2048, I=768,
                 n_ffn=128, n_zero=0, top_k=8, local_begin=0, local_end=128,
                 act="bf16", wt="int8", act_q="int8", logit_bias_std=1.5,
                 residual=True),
    ]
}


def get_workload(name: str) -> MoEShape:
    return WORKLOADS[name]


def scaled(shape: MoEShape, **kw) -> MoEShape:
    """A smaller copy of a workload (same dtypes and structure)."""
    return shape.replace(name=shape.name + "_small", **kw)


def seed_for(shape: MoEShape, seed: int, role: int, index: int = 0) -> int:
    """Deterministic 63-bit seed for (workload, seed, tensor role, index)."""
    h = 1469598103934665603
    for ch in shape.name.encode():
        h = ((h ^ ch) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    for v in (seed, role, index):
        h = ((h ^ (v & 0xFFFFFFFF)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, std, dtype, device, s) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, s), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


_DT = {"f32": torch.float32, "bf16": torch.bfloat16}

# spread of the int8 weight codes (a Gaussian column whose amax is near 127)
INT8_CODE_STD = 32.0


def _int8_codes(shape, device, s) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, s), device=device,
                    dtype=torch.float32)
    return (t * INT8_CODE_STD).round_().clamp_(-127, 127).to(torch.int8)


def _channel_scales(n, w_std, device, s) -> torch.Tensor:
    u = torch.rand((n,), generator=_gen(device, s), device=device,
                   dtype=torch.float32)
    return (0.75 + 0.5 * u) * (w_std / INT8_CODE_STD)

ROLE_LOGITS, ROLE_BIAS, ROLE_X, ROLE_RES, ROLE_W13, ROLE_W2 = range(6)
ROLE_W13_SCALE, ROLE_W2_SCALE = 6, 7
ROLE_NORM_X, ROLE_NORM_RES, ROLE_NORM_W = 8, 9, 10
ROLE_ROUTER_Y, ROLE_ROUTER_W = 11, 12

# RMSNorm epsilon of the Qwen3-MoE family's configs
NORM_EPS = 1e-6


def generate(shape: MoEShape, seed: int = 0, device="cpu",
             weights: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one input set.

    Returns a dict with
      logits   fp32 [T, E_tot]
      x        act  [T, H]
      residual act  [T, H] or None
      w13      [E_loc, H, 2I] f32 / bf16 (bf16 also for mxfp4, quantised by
               the consumer) | int8 codes [E_loc, 2I, H]
      w13_scale None | fp32 [E_loc, 2I] (int8)
      w2       [E_loc, I, H] f32 / bf16 | int8 codes [E_loc, H, I]
      w2_scale None | fp32 [E_loc, H] (int8)
    Weights are drawn per expert (seeded by global expert id), so an expert's
    weights do not depend on the local range.
    """
    dev = torch.device(device)
    T, H, I, E = shape.T, shape.H, shape.I, shape.E_tot
    out: Dict[str, Optional[torch.Tensor]] = {}
    logits = _normal((T, E), 1.0, torch.float32, dev,
                     seed_for(shape, seed, ROLE_LOGITS))
    if shape.logit_bias_std:
        bias = _normal((E,), shape.logit_bias_std, torch.float32, dev,
                       seed_for(shape, seed, ROLE_BIAS))
        logits += bias[None, :]
    out["logits"] = logits.contiguous()
    adt = _DT[shape.act]
    out["x"] = _normal((T, H), 1.0, adt, dev, seed_for(shape, seed, ROLE_X))
    out["residual"] = (_normal((T, H), 1.0, adt, dev,
                               seed_for(shape, seed, ROLE_RES))
                       if shape.residual else None)
    out["w13"] = out["w2"] = out["w13_scale"] = out["w2_scale"] = None
    if not weights:
        return out
    El = shape.E_loc
    experts = range(shape.ffn_begin, shape.ffn_end)
    if shape.wt in ("f32", "bf16", "mxfp4"):
        # MXFP4 weights are drawn in bf16 and quantised by the consumer
        wdt = _DT["bf16" if shape.wt == "mxfp4" else shape.wt]
        w13 = torch.empty((El, H, 2 * I), dtype=wdt, device=dev)
        w2 = torch.empty((El, I, H), dtype=wdt, device=dev)
        for i, e in enumerate(experts):
            w13[i] = _normal((H, 2 * I), shape.w_std, wdt, dev,
                             seed_for(shape, seed, ROLE_W13, e))
            w2[i] = _normal((I, H), shape.w_std, wdt, dev,
                            seed_for(shape, seed, ROLE_W2, e))
        out["w13"], out["w2"] = w13, w2
    elif shape.wt == "int8":
        w13 = torch.empty((El, 2 * I, H), dtype=torch.int8, device=dev)
        w2 = torch.empty((El, H, I), dtype=torch.int8, device=dev)
        s13 = torch.empty((El, 2 * I), dtype=torch.float32, device=dev)
        s2 = torch.empty((El, H), dtype=torch.float32, device=dev)
        for i, e in enumerate(experts):
            w13[i] = _int8_codes((2 * I, H), dev, seed_for(shape, seed, ROLE_W13, e))
            w2[i] = _int8_codes((H, I), dev, seed_for(shape, seed, ROLE_W2, e))
            s13[i] = _channel_scales(2 * I, shape.w_std, dev,
                                     seed_for(shape, seed, ROLE_W13_SCALE, e))
            s2[i] = _channel_scales(H, shape.w_std, dev,
                                    seed_for(shape, seed, ROLE_W2_SCALE, e))
        out["w13"], out["w2"], out["w13_scale"], out["w2_scale"] = w13, w2, s13, s2
    else:
        raise ValueError(shape.wt)
    return out


def generate_norm(T: int, H: int, seed: int = 0, device="cpu",
                  residual: bool = True, name: str = "fused_norm"
                  ) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of the fused residual add + RMSNorm in front of the MoE block:
      x, residual  bf16 [T, H], N(0, 1) (the attention output and the residual
                   stream);
      weight       bf16 [H], 1 + N(0, 0.1) (a norm weight near one).
    """
    dev = torch.device(device)
    key = MoEShape(name, T=T, H=H, I=32, n_ffn=1, n_zero=0, top_k=1,
                   local_begin=0, local_end=1, act="bf16", wt="bf16",
                   act_q="none")
    x = _normal((T, H), 1.0, torch.bfloat16, dev, seed_for(key, seed, ROLE_NORM_X))
    r = (_normal((T, H), 1.0, torch.bfloat16, dev, seed_for(key, seed, ROLE_NORM_RES))
         if residual else None)
    w = _normal((H,), 0.1, torch.float32, dev, seed_for(key, seed, ROLE_NORM_W))
    w = (w + 1.0).to(torch.bfloat16)
    return {"x": x, "residual": r, "weight": w}


def generate_router(T: int, H: int, E: int, seed: int = 0, device="cpu",
                    name: str = "router") -> Dict[str, torch.Tensor]:
    """Inputs of the fp32 router linear in front of the gate:
      y  fp32 [T, H], N(0, 1) (the normalised hidden states, RMS about one);
      w  fp32 [E, H], N(0, 1/sqrt(H)) (so the logits are about N(0, 1)).
    """
    dev = torch.device(device)
    key = MoEShape(name, T=T, H=H, I=32, n_ffn=E, n_zero=0, top_k=1,
                   local_begin=0, local_end=E, act="f32", wt="f32",
                   act_q="none")
    y = _normal((T, H), 1.0, torch.float32, dev, seed_for(key, seed, ROLE_ROUTER_Y))
    w = _normal((E, H), H ** -0.5, torch.float32, dev,
                seed_for(key, seed, ROLE_ROUTER_W))
    return {"y": y, "w": w}
