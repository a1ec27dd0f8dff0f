#!/usr/bin/env python3
"""Benchmark: one tensor-parallel rank's shard of a pre-LN GPT layer,
forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 7b_tp2]

One step is the whole shard path on one batch: LayerNorm, the column-parallel
QKV GEMM, causal attention over the rank's heads, the row-parallel output
projection, the t-way partial sum (the other ranks' partials are resident
inputs, precomputed once), the second LayerNorm, the FC1/GeLU and FC2 pair,
their partial sum, and the mirror-image backward with every weight and bias
gradient.  Inputs are resident in HBM before the timed region.  The timed
region is bracketed by torch.cuda.synchronize() and HIP events on the
stream the kernels run on.

Printed: one JSON line with the achieved model TFLOP/s (causal attention
counted as s(s+1)/2 pairs), the fraction of the bf16 dense MFMA peak,
tokens/s, the roofline of the dominant kernel (measured with HIP events
around its launches inside the timed region) and the fp64 CPU oracle timed
on the host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TP-shard layer fwd+bwd TFLOP/s, % bf16 MFMA peak, tokens/s on 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

# The dominant kernel is the bf16 GEMM (about three quarters of the step).
# Its roofline is measured on the forward launches, which run with nothing
# beside them; the weight-gradient launches run on a second stream
# concurrently with the data-gradient chain, so their durations include
# sharing the CUs and are reported separately.
FWD_TAGS = ("qkv_fwd", "proj_fwd", "fc1_fwd", "fc2_fwd")
# Every call of one step, in issue order (the per-call times of the probed steps).
CALL_TAGS = ("ln1", "qkv_fwd", "attn_fwd", "proj_fwd", "sum_proj_ln2", "fc1_fwd", "fc2_fwd",
             "sum_fc2", "fc2_dgrad", "fc2_wgrad", "fc2_bias", "fc1_dgrad", "fc1_wgrad", "ln2_bwd",
             "proj_dgrad", "proj_wgrad", "proj_bias", "attn_bwd", "qkv_dgrad", "qkv_wgrad",
             "ln1_bwd", "qkv_bias", "quant", "quant_w")
HEAD_TAGS = ("vocab_fwd", "ce_stats", "ce_combine", "ce_bwd", "vocab_bwd", "sum_vocab_dy")
PROBE_EVERY = 10
WGRAD_TAGS = ("fc2_wgrad", "fc1_wgrad", "proj_wgrad", "qkv_wgrad")
FWD_KERNEL = "gemm_bf16_kernel, forward layout (k-major A and B, bf16 C, fused bias/GeLU)"
WGRAD_KERNEL = "gemm_bf16_kernel, weight-gradient layout (m-major A, n-major B, fp32 C)"
FP8_KERNEL = "gemm_bf16_kernel<..., F8> (E4M3 operands, forward layout)"
FP8_WGRAD_KERNEL = ("gemm_bf16_kernel<..., F8, A5> (E5M2 gradient x E4M3 activation codes, "
                    "weight gradient, fp32 C)")


def seq_pairs(cu) -> int:
    """Number of (query, visible key) pairs: sum over sequences of L(L+1)/2."""
    return sum((b - a) * (b - a + 1) // 2 for a, b in zip(cu[:-1], cu[1:]))


def shard_flops(cfg, cu) -> dict:
    """Model FLOPs of one rank shard, forward + backward (3x forward)."""
    T, h, t = cfg.tokens, cfg.hidden, cfg.tp
    hl, fl, al, d = h // t, cfg.ffn // t, cfg.heads // t, cfg.head_dim
    f1 = 2 * fl if cfg.swiglu else fl  # FC1 output width (SwiGLU: gate and up)
    gemm_fwd = 2 * T * (3 * h * hl + hl * h + h * f1 + h * fl)
    attn_fwd = 4 * d * al * seq_pairs(cu)
    vocab_fwd = 2 * T * h * (cfg.vocab // t) if cfg.vocab else 0
    return {
        "total": 3 * (gemm_fwd + attn_fwd + vocab_fwd),
        "gemm": 3 * gemm_fwd, "attn": 3 * attn_fwd, "vocab": 3 * vocab_fwd,
        # per-call flops (M*N*K*2) of the GEMMs whose launches are probed
        "call": {"qkv_fwd": 2 * T * 3 * hl * h, "proj_fwd": 2 * T * hl * h,
                 "fc1_fwd": 2 * T * h * f1, "fc2_fwd": 2 * T * fl * h,
                 "fc2_wgrad": 2 * h * fl * T, "fc1_wgrad": 2 * f1 * h * T,
                 "proj_wgrad": 2 * h * hl * T, "qkv_wgrad": 2 * 3 * hl * h * T},
    }


def source_digest() -> str:
    """Digest of the GEMM source's code: comments and whitespace removed, so
    that an edit of a comment does not retire the counter figures."""
    p = os.path.join(ROOT, "tensor_transformer_layer_04_amd", "csrc", "gemm.hip")
    src = open(p).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch of a GEMM family in a workload from the committed
    counter runs, if they were taken on the current kernel source and on
    that workload (null otherwise)."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha") != source_digest():
        return None
    return t.get("workloads", {}).get(workload, {}).get("bytes_per_launch", {}).get(kernel)


def roofline(kernel, tags, probes, flops, ms, steps, workload, peak=None) -> dict:
    """Roofline entry of one GEMM family: model flops of its probed launches
    over their summed HIP-event durations (``steps``: the probed steps)."""
    dur_ms = sum(a.elapsed_time(b) for t in tags for a, b in probes[t])
    launches = sum(len(probes[t]) for t in tags)
    fl = sum(flops[t] * len(probes[t]) for t in tags)
    achieved = fl / (dur_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if peak is None else peak
    return {
        "kernel": kernel,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic_for(kernel, workload),
        "launches_per_step": launches // max(steps, 1),
        "avg_launch_us": round(1e3 * dur_ms / max(launches, 1), 2),
        "share_of_step": round(dur_ms / (ms * steps), 4),
        "probed_steps": steps,
    }


def cpu_baseline(cfg, data) -> dict:
    """The fp64 oracle (as it stands) on the host: one unsharded fwd+bwd."""
    import numpy as np
    import oracle
    blas = "numpy BLAS"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads", 0) for i in info), default=0)
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                                 for i in info if i.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover
        threads = 0
    threads = threads or len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    # The whole layer when it is small enough for tens of seconds of host
    # work, else the first P tokens (a causal layer's output on a token
    # prefix depends on that prefix only), P sized to about 2.5 TFLOP.
    cu = data["cu_seqlens"].tolist()
    layer_only = cfg.replace(tp=1, vocab=0)

    def prefix_flops(n):
        return shard_flops(layer_only.replace(seq_len=n, micro_batch=1, varlen_tokens=0),
                           prefix_cu(cu, n))["total"]
    P = cfg.tokens
    while P > 64 and prefix_flops(P) > 2.5e12:
        P //= 2
    pcu = prefix_cu(cu, P)
    p64 = {k: oracle.to64(v) for k, v in data.items()
           if k not in ("cu_seqlens", "targets", "emb", "x", "dy")}
    x64 = oracle.to64(data["x"][:P])
    dy64 = oracle.to64(data["dy"][:P]) if "dy" in data else np.ones_like(x64)
    starts = oracle.doc_starts(pcu, P)
    # Passes are repeated until about 10 s of host time; the rate is the
    # average over them.
    passes, total = 0, 0.0
    while passes < 4 and (passes == 0 or total < 10.0):
        t0 = time.perf_counter()
        c = oracle.layer_forward(p64, x64, cfg.heads, cfg.eps, starts,
                                 fp8=bool(getattr(cfg, "fp8", False)))
        oracle.layer_backward(p64, c, dy64, cfg.heads, starts)
        total += time.perf_counter() - t0
        passes += 1
    dt = total / passes
    fl = prefix_flops(P)
    what = (f"{passes} x one unsharded fp64 forward+backward of the {cfg.name} layer ({P} tokens, "
            f"all {cfg.tp} shards' work; {fl / 1e9:.0f} model GFLOP per pass), numpy fp64")
    if P < cfg.tokens or cfg.vocab:
        what += (f"; the first {P} of {cfg.tokens} tokens"
                 + (", layer without the vocab head" if cfg.vocab else ""))
    del np
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(total, 2), "cpu_model": cpu_model, "blas": blas,
            "tokens_per_s": round(P / dt, 1), "sample": what}


def prefix_cu(cu, P):
    """Sequence offsets of the first P tokens of a packed batch."""
    out = [c for c in cu if c < P] + [P]
    return out if out[0] == 0 else [0] + out


PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA: twice the bf16 rate


def fp8_gemm_probe(cfg, L, reps: int = 20) -> dict:
    """The four forward GEMMs of the timed shard with E4M3 operands and
    per-tensor scales, against the same calls in bf16, each call timed alone
    (median of ``reps``) on the layer's own inputs: the FP8 GEMM by itself,
    and with the quantization of its activation (the weights' codes are
    made once, as a training step would after its update)."""
    import torch
    from tensor_transformer_layer_04_amd import mtp
    r = L.ranks[0]
    d, w, a = L.descs[r], L.w[r], L.a[r]
    T, h = cfg.tokens, cfg.hidden
    hl, fl = h // cfg.tp, cfg.ffn // cfg.tp

    def q8(t):
        q = torch.empty(t.numel(), dtype=torch.uint8, device=t.device)
        s = torch.empty(2, dtype=torch.float32, device=t.device)
        mtp.mtp_quantize_fp8(d, t, t.numel(), q, s)
        return q, s

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)[reps // 2]

    out_y = {"qkv": a["qkv"], "proj": a["p"], "fc1": a["g"], "fc2": a["q"]}
    cases = {  # name: (kind, activation, weight, bias, flop)
        "qkv": (mtp.MTP_QKV, L.ln1, w["wqkv"], w["bqkv"], 2 * T * 3 * hl * h),
        "proj": (mtp.MTP_PROJ, a["ctx"], w["wo"], None, 2 * T * hl * h),
        "fc1": (mtp.MTP_FC1, L.ln2, w["w1"], w["b1"], 2 * T * fl * h),
        "fc2": (mtp.MTP_FC2, a["g"], w["w2"], None, 2 * T * fl * h),
    }
    res, tot = {}, {"bf16": 0.0, "fp8": 0.0, "fp8_with_quant": 0.0, "flop": 0}
    for name, (kind, x, wt, b, flop) in cases.items():
        y, u = out_y[name], (a["u"] if kind == mtp.MTP_FC1 else None)
        qw, sw = q8(wt)
        qx, sx = q8(x)
        if kind in (mtp.MTP_QKV, mtp.MTP_FC1):
            bf = lambda: mtp.mtp_col_linear_fwd(d, kind, x, wt, b, y, u)
        else:
            bf = lambda: mtp.mtp_row_linear_fwd(d, kind, x, wt, y)
        f8 = lambda: mtp.mtp_linear_fwd_fp8(d, kind, qx, sx, qw, sw, b, y, u)

        def f8q():
            mtp.mtp_quantize_fp8(d, x, x.numel(), qx, sx)
            f8()
        t_bf, t_f8, t_f8q = timed(bf), timed(f8), timed(f8q)
        res[name] = {"bf16_us": round(t_bf, 1), "fp8_us": round(t_f8, 1),
                     "fp8_with_quant_us": round(t_f8q, 1),
                     "fp8_tflops": round(flop / t_f8 / 1e6, 1)}
        tot["bf16"] += t_bf
        tot["fp8"] += t_f8
        tot["fp8_with_quant"] += t_f8q
        tot["flop"] += flop
    ach = tot["flop"] / tot["fp8"] / 1e6
    return {"per_gemm": res, "bf16_us": round(tot["bf16"], 1), "fp8_us": round(tot["fp8"], 1),
            "fp8_with_quant_us": round(tot["fp8_with_quant"], 1),
            "roofline": {"kernel": FP8_KERNEL,
                         "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4),
                         # the same four GEMMs as the FP8 step of this shard
                         "traffic": traffic_for(FP8_KERNEL, cfg.name + "_fp8")}}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="7b_tp2")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run 5 plain 256 MiB device-to-device copies: the reference "
                         "of known size that scales the HBM byte counters")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every rank shard of the layer runs on the same "
              "device and the tensor-parallel sum is an on-device kernel, so there is no "
              f"multi-GPU run (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        return 2

    import torch
    import synth
    from tensor_transformer_layer_04_amd.layer import TPLayer, VocabHead

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU (no GPU visible)", file=sys.stderr)
        return 1
    if args.copy_probe:
        a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print("copy probe: 5 x 256 MiB read + 256 MiB written", flush=True)
        return 0
    cfg = synth.get_config(args.config)
    data = synth.generate(cfg)
    cu = data["cu_seqlens"].tolist()
    dev = "cuda"
    x = data["x"].to(dev)
    # With a vocab head the layer's upstream gradient comes from the head.
    dy = data["dy"].to(dev) if not cfg.vocab else None

    ext, head_ext = None, ((), ())
    if cfg.tp > 1:
        # The other ranks' partials of this very step (and, with a vocab head,
        # their CE stats and dy partials), computed once and kept resident:
        # the timed shard's t-way sums read them as inputs.
        full = TPLayer(cfg, data, device=dev, cu_seqlens=data["cu_seqlens"])
        full.forward(x)
        if cfg.vocab:
            head = VocabHead(cfg, data, device=dev)
            head.forward(full.y)
            full.backward(head.backward())
            stats, dys = head.partials()
            others = [i for i, r in enumerate(head.ranks) if r != args.rank]
            head_ext = ([stats[i] for i in others], [dys[i] for i in others])
            del head
        else:
            full.backward(dy)
        parts = full.partials()
        ext = {k: [v[i] for i, r in enumerate(full.ranks) if r != args.rank] for k, v in parts.items()}
        torch.cuda.synchronize()
    def make_layer(overlap):
        lay = TPLayer(cfg, data, ranks=[args.rank], device=dev, cu_seqlens=data["cu_seqlens"],
                      overlap=overlap)
        if cfg.tp > 1 and lay.sp:
            # The other ranks' row blocks of the token-sharded activations and
            # gradients (what the all-gathers would deliver) stay resident.
            lay.adopt_rows(full)
        return lay
    # L: weight and bias gradients on a second stream beside the data
    # gradients (the timed step); L1: the same step on one stream, for the
    # HIP-graph replay (a graph captured from two streams replays slower).
    L = make_layer(True)
    L1 = make_layer(False)
    if cfg.tp > 1:
        del full
    H = VocabHead(cfg, data, ranks=[args.rank], device=dev) if cfg.vocab else None

    def step_of(lay):
        def step():
            lay.forward(x, ext)
            if H is None:
                lay.backward(dy, ext)
            else:
                H.forward(lay.y, head_ext[0])
                lay.backward(H.backward(head_ext[1]), ext)
        return step
    step = step_of(L)
    step1 = step_of(L1)

    # The comparison passes (one-stream eager and graph replays, per-call
    # times) run first and the headline region last: the GPU
    # comes out of the idle of the set-up at low clocks, and its first tens
    # of milliseconds of steps run several % slower than the steady state a
    # training job sees (measured: 30 steps after 5 warm-up steps 1.217 ms
    # per step, the next 30 1.176; after 2 s idle 1.254, then 1.168).

    # The same step replayed from a HIP graph (captured once, inputs
    # unchanged): the one-stream step, and the two-stream one beside it.
    def graph_replay_ms(fn):
        try:
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                fn()
            torch.cuda.current_stream().wait_stream(cs)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            del g
            return round(a.elapsed_time(b) / args.steps, 4)
        except RuntimeError as exc:  # capture unsupported: report it, keep the eager figure
            return f"capture failed: {exc}"[:200]

    # the one-stream step launched eagerly, for comparison with its graph
    def eager_ms(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a1, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a1.record()
        for _ in range(args.steps):
            fn()
        b1.record()
        torch.cuda.synchronize()
        return round(a1.elapsed_time(b1) / args.steps, 4)
    # eager and graph in turn, twice; the second of each is reported (both
    # then run at the settled clock)
    eager_ms(step1)
    graph_replay_ms(step1)
    eager_one_stream_ms = eager_ms(step1)
    graph_ms = graph_replay_ms(step1)
    graph_ms_two_streams = graph_replay_ms(step)

    # Per-call times: a few steps with events around every call.
    calls = {t: [] for t in CALL_TAGS + HEAD_TAGS}
    n_call_steps = 5
    L.probe = calls
    if H is not None:
        H.probe = calls
    for _ in range(n_call_steps):
        step()
    torch.cuda.synchronize()
    L.probe = None
    if H is not None:
        H.probe = None
    call_us = {t: round(1e3 * sum(a.elapsed_time(b) for a, b in calls[t]) / n_call_steps, 1)
               for t in CALL_TAGS + HEAD_TAGS if calls[t]}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Every PROBE_EVERY-th timed step records HIP events around the probed
    # launches (each event adds a few us of gap, so not every step does).
    probes = {t: [] for t in FWD_TAGS + WGRAD_TAGS}
    probed = [i for i in range(args.steps) if (i + 1) % PROBE_EVERY == 0] or [args.steps - 1]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        L.probe = probes if i in probed else None
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    L.probe = None

    # Spread: the same steps once more, each between its own pair of events
    # (which adds the events' own gaps to every step).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in ev)

    def pct(q):
        return round(per_step[min(len(per_step) - 1, int(q * len(per_step)))], 4)

    fl = shard_flops(cfg, cu)
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8/bf16" if getattr(cfg, "fp8", False)
                  else "bf16" if cfg.dtype == "bf16" else "f32"),
        "data": "synthetic: seeded x, dy ~ N(0,1), weights ~ N(0,0.02), biases 0, LN gamma 1",
        "config": {
            "workload": f"{cfg.name}: TP rank {args.rank} of {cfg.tp}, pre-LN layer shard"
                        + (" with sequence parallelism" if L.sp else "")
                        + (f", attention over {L.cp} context-parallel chunks"
                           f" ({len(L.cp_pairs())} off-diagonal block pairs)" if L.cp > 1 else "")
                        + (" + vocab-parallel CE head" if cfg.vocab else "")
                        + (", twelve GEMMs on FP8 codes (E4M3 forward, E5M2 gradients, per-tensor "
                           "scales; weights quantized inside the step)" if L.fp8 else "")
                        + " fwd+bwd",
            "hidden": cfg.hidden, "heads": cfg.heads, "ffn": cfg.ffn, "tp": cfg.tp,
            "rank": args.rank, "seq_len": cfg.seq_len, "micro_batch": cfg.micro_batch,
            "tokens": cfg.tokens, "global_batch": cfg.micro_batch,
            "parallelism": f"tp{cfg.tp}" + ("-sp" if L.sp else "")
                           + (f"-cp{L.cp}" if L.cp > 1 else "") + "-shard",
        },
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(cfg.tokens / (ms * 1e-3), 1),
        "model_gflop_per_step": round(fl["total"] / 1e9, 2),
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "graph_replay_ms_per_step": graph_ms,
        "graph_replay_two_streams_ms_per_step": graph_ms_two_streams,
        "eager_one_stream_ms_per_step": eager_one_stream_ms,
        "call_us_per_step": call_us,
        # The step without the forward sums of the ranks' row-parallel partials
        # (charged in full above): the FFN output sum, and the projection sum
        # fused with LN2 less a LayerNorm of the same shape (ln1).  The
        # backward sums are fused into the LayerNorm backward and stay in.
        "ms_per_step_less_forward_tp_sums": (
            round(ms - 1e-3 * (call_us["sum_fc2"] + call_us["sum_proj_ln2"] - call_us["ln1"]), 4)
            if all(k in call_us for k in ("sum_fc2", "sum_proj_ln2", "ln1")) else None),
        "roofline": roofline(FP8_KERNEL if L.fp8 else FWD_KERNEL, FWD_TAGS, probes, fl["call"], ms,
                             len(probed), cfg.name, PEAK_FP8_TFLOPS if L.fp8 else None),
        "roofline_wgrad_overlapped": roofline(FP8_WGRAD_KERNEL if L.fp8 else WGRAD_KERNEL,
                                              WGRAD_TAGS, probes, fl["call"], ms, len(probed),
                                              cfg.name, PEAK_FP8_TFLOPS if L.fp8 else None),
    }
    if cfg.dtype == "bf16" and not cfg.swiglu and not L.fp8 and cfg.tokens % 8 == 0:
        # the same shard's forward GEMMs on the FP8 matrix cores (not part of the step)
        out["fp8_forward_gemms"] = fp8_gemm_probe(cfg, L)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, data)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
