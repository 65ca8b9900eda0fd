"""Benchmark of the MoE expert layer on one MI355X.

One step = one pass of the whole layer (gate top-k softmax, routing, gather,
GEMM1 + SwiGLU, GEMM2, finalize) over one batch of synthetic inputs that are
already resident in HBM, through the library's C ABI (moe_layer_traced, which
records caller-supplied events at stage boundaries on the launch stream).

Prints ONE JSON line: whole-step tokens/s plus
  roofline     the dominant kernel (GEMM1 + SwiGLU) timed by the two events
               around it in every fifth of the timed steps, against the
               MI355X peak of the bound it hits (HBM 8 TB/s for decode-size
               batches, dense MFMA for prefill-size batches);
  stages_us    every stage from an untimed pass after the timed steps, with
               an event at each stage boundary (each event adds a few
               microseconds);
  cpu_baseline the CPU oracle timed on the host on a bounded sample of the
               same workload (a reported baseline, not the target).

Before the W warm-up steps, untimed steps run for 2 s of wall time so that
the GPU has reached its working clocks when the (short) timed region starts.

Static expert weights are prepared once before timing, as at model load:
int8 and MXFP4 weights packed (moe_pack_weights); bf16 weights in the layout
that suits the model's experts (--wt-layout auto): slab-packed
(moe_pack_bf16_weights) for the LongCat-shaped experts, whose GEMMs stream
6144 x 2048 experts in long blocks (layer 6072 -> 5850 us), row-major for
the Qwen3-30B-A3B ones (slab-packed was 3-4 % slower at decode sizes and
neutral in prefill). config.wt_layout says which.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--op layer|norm_cast|norm_mx]
                       [--wt-layout auto|rowmajor|packed]

--op norm_cast / norm_mx time the fused residual add + RMSNorm in front of the
MoE block instead (dual fp32/bf16 output, or MXFP8), on the workload's T x H
rows; its JSON line has the same fields with the norm kernel as the roofline
kernel (HBM bound). --op router times the fp32 router linear (T x H hidden
states times the E_tot x H router weight; fp32 MFMA bound).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("MoE layer tokens/s; grouped-GEMM % of MFMA peak (prefill) / "
          "% HBM BW (decode)")
# the largest single-GPU workload: LongCat-Flash-shaped, 512 FFN experts of
# 6144 x 2048 plus 256 identity experts, 1024 tokens, top-12 (38.65 GB of
# expert weights per layer)
DEFAULT_WORKLOAD = "longcat_flash_zero_experts_bf16"

PEAK_HBM_GBS = 8000.0
# dense MFMA peaks (int8: 5.0 POP/s, reported in the same unit as tera-ops)
PEAK_TFLOPS = {"bf16": 2500.0, "mx": 5000.0, "i8": 5000.0, "f32": 157.3}


# HBM bytes of one launch of the dominant kernel, from two rocprofv3 --pmc
# runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch,
# averaged over the timed dispatches), each scaled by what the same counter
# reads for a plain device copy of known size (--copy-calibration): a
# 256 MiB copy reads FETCH_SIZE = 131080 KiB (factor 2.0) and WRITE_SIZE =
# 262144 KiB (factor 1.0). An entry holds only while the kernel's sources
# hash to the recorded value; otherwise traffic is reported as null.
COPY_FACTORS = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
KERNEL_SOURCES = {
    # the kernel's source and the headers with device code it includes
    # (launch.h: the Tile struct and the item order of the tiled kernels)
    "gemm_bf16_stream": ["gemm_bf16_stream.hip", "common.h", "launch.h"],
    "gemm_bf16_tiled": ["gemm_bf16_tiled.hip", "lds_dma.h", "common.h", "launch.h"],
    "gemm_mx_tiled": ["gemm_mx_tiled.hip", "lds_dma.h", "common.h", "launch.h"],
    "gemm_i8_stream": ["gemm_i8_stream.hip", "common.h", "launch.h"],
}
# bf16 workloads whose weights bench.py slab-packs by default (measured:
# the LongCat-shaped layer 6071.9 -> 5849.5 us; the Qwen3-30B-A3B decode
# layer 181.6 -> 186.6 us at 32 tokens and 199.6 -> 208.0 us at 128, its
# skewed prefill 464.0 -> 463.8 us, outputs bit-identical)
BF16_PACKED = {"longcat_flash_zero_experts_bf16"}

TRAFFIC = {
    # workload: (kernel source set, sha256[:16] of its sources, FETCH KiB,
    #            WRITE KiB) per GEMM1 dispatch, taken with the weight layout
    #            bench.py uses by default for the workload
    "qwen3_30b_a3b_decode_bf16":
        ("gemm_bf16_stream", "a94d9ea2fd68934f", 341624.4, 384.0),
    "qwen3_30b_a3b_prefill_skewed_bf16":
        ("gemm_bf16_tiled", "6f9a7fe77c7f360a", 521882.2, 49152.0),
    "longcat_flash_zero_experts_bf16":
        ("gemm_bf16_stream", "a94d9ea2fd68934f", 12835682.3, 32528.0),
    "qwen3_235b_a22b_ep_rank_w4a8":
        ("gemm_mx_tiled", "9837db651f8489a6", 164054.5, 12895.2),
    "qwen3_30b_a3b_decode_w8a8":
        ("gemm_i8_stream", "f183022218c91c87", 171200.5, 768.1),
    "qwen3_30b_a3b_prefill_skewed_w8a8":
        ("gemm_bf16_tiled", "6f9a7fe77c7f360a", 226607.8, 98304.0),
}


def _sources_sha(kind):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_layer_gate_amd", "csrc")
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, default_layout=True):
    ent = TRAFFIC.get(workload)
    if ent is None or not default_layout:
        return None
    kind, sha, fetch_kib, write_kib = ent
    if _sources_sha(kind) != sha:
        return None
    return int((fetch_kib * COPY_FACTORS["FETCH_SIZE"] +
                write_kib * COPY_FACTORS["WRITE_SIZE"]) * 1024)


def _copy_calibration():
    """A plain device copy of 256 MiB, five times: the reference dispatch for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "dispatches": 5}), flush=True)


def _settle(step, seconds=2.0):
    """Untimed steps for `seconds` of wall time before the warm-up: the GPU
    reaches its working clocks only after some time under load, and a short
    timed region would otherwise be measured on a ramping clock (the
    LongCat-shaped layer, row-major weights: 164.5 k tokens/s after 0.1 s of
    such steps, 168.5 k after 1 s; slab-packed: 174.7 k after 1 s, 179.4 k
    after 2 s and 179.1 k after 4 s, each pair on one box)."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the reference copy for counter scaling")
    ap.add_argument("--op", default="layer",
                    choices=["layer", "norm_cast", "norm_mx", "router"],
                    help="what one step is: the MoE layer (default) or the "
                         "fused add + RMSNorm in front of it")
    ap.add_argument("--wt-layout", default="auto",
                    choices=["auto", "rowmajor", "packed"],
                    help="layout of bf16 expert weights (auto: the one "
                         "BF16_PACKED picks for the workload)")
    ap.add_argument("--print-source-sha", action="store_true",
                    help="print the source hashes that key the traffic table")
    return ap.parse_args()


def _routing_stats(m, p, shape, inp):
    """Touched experts and routed rows of the local range, read back once
    after the timed region from the library's own routing calls."""
    import torch
    ids, _ = m.gate_topk(p, inp["logits"])
    r = m.init_routing(p, ids, inp["x"])
    counts = r["counts"].cpu().numpy()
    loc = counts[shape.ffn_begin:shape.ffn_end]
    torch.cuda.synchronize()
    return int((loc > 0).sum()), int(loc.sum())


def _gemm1_units(shape, touched, R):
    """Algorithmic work of one GEMM1 + SwiGLU launch."""
    H, I = shape.H, shape.I
    if shape.wt == "mxfp4":
        wbytes = touched * (2 * I * H // 2 + 2 * I * H // 32)
        abytes = R * (H + H // 32) + R * (I + I // 32)
    elif shape.wt == "int8":
        # int8 codes + fp32 channel scales; int8 rows of x + fp32 row scales
        # in, h out in fp32 (quantised to int8 by the next launch)
        wbytes = touched * (2 * I * H + 2 * I * 4)
        abytes = R * (H + 4) + R * I * 4
    else:
        eb = 4 if shape.wt == "f32" else 2
        wbytes = touched * H * 2 * I * eb
        abytes = R * H * eb + R * I * eb
    flops = 2.0 * R * H * 2 * I
    return wbytes + abytes, flops


def _bound(shape, R, touched):
    """Decode-size batches stream weights (HBM bound); prefill-size batches
    are MFMA bound. Chosen by arithmetic intensity of GEMM1 against the
    ridge point of the format's peak."""
    nbytes, flops = _gemm1_units(shape, touched, R)
    kind = {"mxfp4": "mx", "int8": "i8", "f32": "f32"}.get(shape.wt, "bf16")
    ridge = PEAK_TFLOPS[kind] * 1e12 / (PEAK_HBM_GBS * 1e9)
    return ("mfma" if flops / nbytes > ridge else "hbm"), kind


def _cpu_baseline(shape, inp, target_s):
    """The oracle as it stands, on the host, over a bounded token sample."""
    import numpy as np
    import torch

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = max(blas, torch.get_num_threads())
    host = {k: (None if v is None else v.cpu()) for k, v in inp.items()
            if k in ("logits", "x", "residual")}
    fb = shape.ffn_begin
    note = ""
    if shape.wt == "mxfp4":
        # the oracle quantises the bf16 weights itself (its MX quantiser),
        # once per local expert before the timed sample: W4A8 weights are
        # static, quantised when a model is loaded
        cache = {}
        for i in range(shape.E_loc):
            a = inp["w13_bf16"][i].double().cpu().numpy().T
            b = inp["w2_bf16"][i].double().cpu().numpy().T
            c, sc = O.mx_quant(a, "e2m1")
            A = O.mx_dequant(c, sc, "e2m1").T.copy()
            c, sc = O.mx_quant(b, "e2m1")
            cache[fb + i] = (A, O.mx_dequant(c, sc, "e2m1").T.copy())
        note = "; MXFP4 weights quantised by the oracle before timing"

        def get(e):
            return cache[e]
    elif shape.wt == "int8":
        # the row-major int8 weights (the GPU path takes them packed)
        def get(e):
            i = e - fb
            a = O.int8_dequant_rows(inp["w13_rowmajor"][i].cpu().numpy(),
                                    inp["w13_scale"][i].cpu().numpy())
            b = O.int8_dequant_rows(inp["w2_rowmajor"][i].cpu().numpy(),
                                    inp["w2_scale"][i].cpu().numpy())
            return a.T.copy(), b.T.copy()
    else:
        # one expert's row-major weights fetched from the device when the
        # oracle asks (the GPU path may take them slab-packed)
        w13 = inp.get("w13_rowmajor", inp["w13"])
        w2 = inp.get("w2_rowmajor", inp["w2"])

        def get(e):
            i = e - fb
            return (w13[i].cpu().double().numpy(), w2[i].cpu().double().numpy())
    kw = dict(logits=host["logits"].numpy(), x=host["x"].double().numpy(),
              residual=None if host["residual"] is None else host["residual"].double().numpy(),
              get_weights=get, T=shape.T, H=shape.H, I=shape.I,
              n_ffn=shape.n_ffn, n_zero=shape.n_zero, top_k=shape.top_k,
              local_begin=shape.local_begin, local_end=shape.local_end,
              act=shape.act, act_q=shape.act_q)
    # sample: whole layer when small enough, else a growing prefix of tokens
    # evaluated per token (weights fetched once per expert)
    done, t0 = 0, time.perf_counter()
    if shape.T <= 64:
        reps = 0
        while True:
            O.moe_layer(**kw)
            reps += 1
            el = time.perf_counter() - t0
            if el >= target_s or reps >= 5:
                break
        done = reps * shape.T
        sample = f"whole layer ({shape.T} tokens) x{reps} via the routed oracle"
    else:
        rng = np.random.default_rng(0)
        toks = rng.permutation(shape.T)
        n = 8
        while True:
            O.moe_tokens(toks[done:done + n], cache_weights=False, **kw)
            done += n
            el = time.perf_counter() - t0
            if el >= target_s or done >= shape.T:
                break
            n = min(2 * n, shape.T - done)
        sample = f"{done} of {shape.T} tokens via the per-token oracle{note}"
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "sample": sample, "seconds": round(el, 2)}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (the expert-parallel case is one rank's expert range on "
              "one GPU). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.print_source_sha:
        print(json.dumps({k: _sources_sha(k) for k in KERNEL_SOURCES}))
        return
    if args.copy_calibration:
        _copy_calibration()
        return
    import torch

    import moe_expert_layer_gate_amd as m
    from moe_inputs import generate, get_workload

    m.lib()
    if args.op == "router":
        return _bench_router(args, m)
    if args.op != "layer":
        return _bench_norm(args, m)
    shape = get_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = generate(shape, seed=args.seed, device=dev)
    if shape.wt in ("int8", "mxfp4"):
        # static quantised weights are prepared once, as at model load
        # (untimed): MXFP4 quantised from the bf16 draw by the library, then
        # packed; the CPU baseline keeps the originals
        for k in ("w13", "w2"):
            if shape.wt == "mxfp4":
                inp[k + "_bf16"] = inp[k]
                codes, inp[k + "_scale"] = m.quant_mxfp4_weights(inp[k])
                inp[k] = m.pack_weights(codes)
                del codes
            else:
                inp[k + "_rowmajor"] = inp[k]
                inp[k] = m.pack_weights(inp[k])
    layout = "rowmajor" if shape.wt == "f32" else "packed"
    if shape.wt == "bf16":
        want = args.wt_layout
        if want == "auto":
            want = "packed" if shape.name in BF16_PACKED else "rowmajor"
        if shape.I % 128 or shape.H % 256:
            want = "rowmajor"  # the slab order needs whole 256-column slabs
        layout = want
    if shape.wt == "bf16" and layout == "packed":
        # static bf16 weights in the slab order, packed once as at model
        # load (untimed); the CPU baseline keeps the row-major originals
        for k, glu in (("w13", True), ("w2", False)):
            inp[k + "_rowmajor"] = inp[k]
            inp[k] = m.pack_bf16_weights(inp[k], glu=glu)
    p = m.problem(shape, wt_layout=layout)
    ws = torch.empty(max(m.layer_workspace_bytes(p), 1), dtype=torch.uint8, device=dev)
    dt = torch.float32 if shape.act == "f32" else torch.bfloat16
    out = torch.empty((shape.T, shape.H), dtype=dt, device=dev)
    nst = len(m.STAGES) + 1

    def step(events):
        m.layer_traced(p, inp["logits"], inp["x"], inp["w13"], inp["w2"],
                       events, inp["w13_scale"], inp["w2_scale"],
                       residual=inp["residual"], out=out, workspace=ws)

    none = [None] * nst
    g1 = m.STAGES.index("gemm1_swiglu")

    def events(n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n)]
              for _ in range(args.steps)]
        for row in ev:  # torch creates the HIP event on first record
            for e in row:
                e.record()
        return ev

    def stage_pass():
        """Untimed pass with an event at every stage boundary (each event
        record costs a few microseconds of stream time, so these events stay
        out of the timed steps)."""
        ev = events(nst)
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(ev[i])
        torch.cuda.synchronize()
        st = {}
        for s, name in enumerate(m.STAGES):
            d = [ev[i][s].elapsed_time(ev[i][s + 1]) * 1e3 for i in range(args.steps)]
            st[name] = round(sum(d) / len(d), 2)
        tot = sum(ev[i][0].elapsed_time(ev[i][nst - 1]) * 1e3
                  for i in range(args.steps)) / args.steps
        return st, tot

    def bracket_pass(cold):
        """Steps timed one by one with an event pair, the first pass around
        the layer, the second around GEMM1; returns the two medians in
        microseconds. cold: a 512 MB buffer (twice the 256 MB MALL, far more
        than the 8 x 4 MB of L2) is read before every step, outside the
        events, as the rest of a model's layers would between two calls of
        one layer. (It is read, not written: a write would leave the caches
        full of dirty lines whose write-back then competes with the next
        step's reads, which a model's other layers need not cause.)"""
        scrub = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
        res = []
        for a, b in ((0, nst - 1), (g1, g1 + 1)):
            ev = events(2)
            torch.cuda.synchronize()
            for i in range(args.steps):
                if cold:
                    scrub.amax()
                row = list(none)
                row[a], row[b] = ev[i]
                step(row)
            torch.cuda.synchronize()
            d = sorted(ev[i][0].elapsed_time(ev[i][1]) * 1e3
                       for i in range(args.steps))
            res.append(d[len(d) // 2])
        del scrub
        return res

    _settle(lambda: step(none))
    for _ in range(args.warmup):
        step(none)
    # Timed region: the only events inside it bracket the GEMM1 launch of
    # every EVERY-th step (a timed event pair costs about 10 us of stream time
    # per step on this layer, so bracketing every step would understate the
    # layer's throughput by ~5 % at decode sizes).
    EVERY = 5
    sampled = list(range(0, args.steps, EVERY))
    ev = events(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        row = list(none)
        if i % EVERY == 0:
            row[g1], row[g1 + 1] = ev[i]
        step(row)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    gemm1_us = sum(ev[i][0].elapsed_time(ev[i][1]) * 1e3
                   for i in sampled) / len(sampled)
    # per-stage breakdown, reported from a pass after the timed region
    stage_us, traced_step_us = stage_pass()
    cold_layer_us, cold_gemm1_us = bracket_pass(True)
    warm_layer_us, warm_gemm1_us = bracket_pass(False)

    touched, R = _routing_stats(m, p, shape, inp)
    bound, kind = _bound(shape, R, touched)
    nbytes, flops = _gemm1_units(shape, touched, R)
    dur = gemm1_us * 1e-6
    if bound == "hbm":
        ach = nbytes / dur / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": _traffic(shape.name, args.wt_layout == "auto"
                                    or shape.wt != "bf16")}
    else:
        ach = flops / dur / 1e12
        peak = PEAK_TFLOPS[kind]
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": _traffic(shape.name, args.wt_layout == "auto"
                                    or shape.wt != "bf16")}
    # both fractions for every workload: the bound one is "frac"; prefill
    # workloads are graded on MFMA peak and sit near the HBM ridge
    peak_f = PEAK_TFLOPS[kind]
    roof["hbm_frac"] = round(nbytes / dur / 1e9 / PEAK_HBM_GBS, 4)
    roof["mfma_frac"] = round(flops / dur / 1e12 / peak_f, 4)
    roof["mfma_peak_tflops"] = peak_f
    cold_frac = roof["frac"] * gemm1_us / cold_gemm1_us
    roof.update({"kernel": "gemm1_swiglu", "avg_us": round(gemm1_us, 2),
                 "algorithmic_bytes": int(nbytes), "algorithmic_flops": flops,
                 "touched_experts": touched, "routed_rows": R})
    rec = {
        "metric": METRIC,
        "value": round(shape.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "mxfp4": "mxfp8xmxfp4",
                  "int8": "int8xint8"}[shape.wt],
        "data": "synthetic",
        "config": {"workload": shape.name, "T": shape.T, "H": shape.H,
                   "I": shape.I, "n_ffn": shape.n_ffn, "n_zero": shape.n_zero,
                   "top_k": shape.top_k,
                   "local_experts": [shape.local_begin, shape.local_end],
                   "act": shape.act, "wt": shape.wt, "act_q": shape.act_q,
                   "wt_layout": layout, "residual": shape.residual,
                   "seed": args.seed},
        "traced_step_us": round(traced_step_us, 2),
        "stages_us": stage_us,
        "roofline": roof,
        # medians of per-step event pairs with the caches cleared before
        # every step, and of the same pairs on back-to-back steps
        "cold": {"layer_us": round(cold_layer_us, 2),
                 "tokens_per_s": round(shape.T / (cold_layer_us * 1e-6), 1),
                 "gemm1_us": round(cold_gemm1_us, 2),
                 "gemm1_roofline_frac": round(cold_frac, 4),
                 "warm_layer_us": round(warm_layer_us, 2),
                 "warm_gemm1_us": round(warm_gemm1_us, 2)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _cpu_baseline(shape, inp, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def _bench_norm(args, m):
    """One step = one fused residual add + RMSNorm over the workload's T x H
    hidden states (bf16 x and residual resident in HBM)."""
    import numpy as np
    import torch

    from moe_inputs import NORM_EPS, generate_norm, get_workload

    shape = get_workload(args.workload)
    T, H = shape.T, shape.H
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = generate_norm(T, H, seed=args.seed, device=dev)
    mx = args.op == "norm_mx"
    y32 = torch.empty((T, H), dtype=torch.float32, device=dev)
    y16 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    codes = torch.empty((T, H), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    res = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    L = m.lib()
    from moe_expert_layer_gate_amd import _ptr, _stream

    def step():
        if mx:
            st = L.moe_add_rms_norm_mx_quant(T, H, _ptr(inp["x"]), _ptr(inp["residual"]),
                                             _ptr(inp["weight"]), NORM_EPS, _ptr(codes),
                                             _ptr(scales), _ptr(res), _stream())
        else:
            st = L.moe_add_rms_norm_cast(T, H, _ptr(inp["x"]), _ptr(inp["residual"]),
                                         _ptr(inp["weight"]), NORM_EPS, _ptr(y32),
                                         _ptr(y16), _ptr(res), _stream())
        assert st == 0, st

    _settle(step)
    for _ in range(args.warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    us = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / args.steps
    # algorithmic bytes: x and residual read, new residual and y written
    # (fp32 + bf16, or e4m3 codes + e8m0 scales), the norm weight read once
    per_tok = 2 * H + 2 * H + 2 * H + ((H + H // 32) if mx else (4 * H + 2 * H))
    nbytes = T * per_tok + 2 * H
    ach = nbytes / (us * 1e-6) / 1e9
    rec = {
        "metric": "fused residual add + RMSNorm tokens/s",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->mxfp8" if mx else "bf16->f32+bf16", "data": "synthetic",
        "config": {"workload": f"add_rms_norm_{'mx' if mx else 'cast'} of {shape.name}",
                   "T": T, "H": H, "eps": NORM_EPS, "residual": True,
                   "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "add_rms_norm_" + ("mx" if mx else "cast"),
                     "avg_us": round(us, 2), "algorithmic_bytes": int(nbytes)},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        x = inp["x"].double().cpu().numpy()
        r = inp["residual"].double().cpu().numpy()
        w = inp["weight"].double().cpu().numpy()
        fn = O.add_rms_norm_mx_quant if mx else O.add_rms_norm_cast
        done, t0 = 0, time.perf_counter()
        while True:
            fn(x, r, w, NORM_EPS)
            done += T
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or done >= 20 * T:
                break
        rec["cpu_baseline"] = {"value": round(done / el, 1), "unit": "tokens/s",
                               "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": f"all {T} rows x{done // T}",
                               "seconds": round(el, 1)}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def _bench_router(args, m):
    """One step = one fp32 router linear over the workload's T tokens: logits
    [T, E_tot] = y [T, H] @ w_router [E_tot, H]^T (inputs resident in HBM)."""
    import torch

    from moe_inputs import generate_router, get_workload

    shape = get_workload(args.workload)
    T, H, E = shape.T, shape.H, shape.E_tot
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = generate_router(T, H, E, seed=args.seed, device=dev)
    out = torch.empty((T, E), dtype=torch.float32, device=dev)

    def step():
        m.router_logits(inp["y"], inp["w"], out=out)

    _settle(step)
    for _ in range(args.warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    us = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / args.steps
    flops = 2.0 * T * H * E
    nbytes = 4 * (T * H + E * H + T * E)
    ach = flops / (us * 1e-6) / 1e12
    peak = PEAK_TFLOPS["f32"]
    rec = {
        "metric": "fp32 router linear tokens/s",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"router_logits of {shape.name}", "T": T,
                   "H": H, "E": E, "seed": args.seed},
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                     "traffic": None, "kernel": "router_logits",
                     "avg_us": round(us, 2), "algorithmic_flops": flops,
                     "algorithmic_bytes": int(nbytes)},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        y = inp["y"].double().cpu().numpy()
        w = inp["w"].double().cpu().numpy()
        done, t0 = 0, time.perf_counter()
        while True:
            O.router_logits(y, w)
            done += T
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or done >= 20 * T:
                break
        rec["cpu_baseline"] = {"value": round(done / el, 1), "unit": "tokens/s",
                               "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": f"all {T} tokens x{done // T}",
                               "seconds": round(el, 1)}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
