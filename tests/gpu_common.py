"""Helpers shared by the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys
import time
from typing import Dict

import numpy as np
import pytest
import torch

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tensor_transformer_layer_04_amd import mtp
    mtp.lib()  # raises if libmtp.so is missing: no fallback exists


def rel(got, ref) -> float:
    return oracle.rel_frobenius(got, ref)


def check(name: str, got, ref, tol: float, report: Dict[str, float], floor: float = 0.0) -> None:
    """rel-Frobenius error <= tol.  ``floor`` bounds the denominator from
    below for tensors whose exact value is (near) zero, e.g. the query
    gradient of a one-token sequence."""
    got64, ref64 = oracle.to64(got), oracle.to64(ref)
    den = max(float(np.linalg.norm(ref64.ravel())), floor)
    e = float(np.linalg.norm((got64 - ref64).ravel())) / den if den > 0 else (
        0.0 if not np.any(got64) else float("inf"))
    report[name] = e
    assert np.isfinite(e) and e <= tol, f"{name}: rel-Frobenius {e:.3e} > {tol:.1e}"


def run_gpu_layer(cfg, data, ranks=None, dy=None, with_backward=True):
    """Run the full layer (all ranks unless given) through libmtp."""
    from tensor_transformer_layer_04_amd.layer import TPLayer
    dev = "cuda"
    L = TPLayer(cfg, data, ranks=ranks, device=dev, cu_seqlens=data["cu_seqlens"])
    x = data["x"].to(dev).contiguous()
    L.forward(x)
    if with_backward:
        d = (dy if dy is not None else data["dy"]).to(dev).contiguous()
        L.backward(d)
    torch.cuda.synchronize()
    return L


def oracle_layer(cfg, data, dy=None):
    starts = oracle.doc_starts(data["cu_seqlens"], cfg.tokens)
    c = oracle.layer_forward(data, data["x"], cfg.heads, cfg.eps, starts)
    g = oracle.layer_backward(data, c, dy if dy is not None else data["dy"], cfg.heads, starts)
    return c, g


def compare_layer(cfg, L, c, g, data, report, rows=None, ranks=None):
    """Element-wise comparison of every per-rank and summed tensor."""
    tol = TOL[cfg.dtype]
    sl = slice(None) if rows is None else slice(0, rows)
    ranks = L.ranks if ranks is None else ranks
    cpu = lambda t: t.detach().float().cpu()
    p64 = {k: oracle.to64(v) for k, v in data.items()
           if k not in ("x", "dy", "targets", "cu_seqlens", "emb")}
    check("y1", cpu(L.y1)[sl], c["y1"][sl], tol, report)
    check("y", cpu(L.y)[sl], c["y"][sl], tol, report)
    check("ln1", cpu(L.ln1)[sl], c["ln1"][sl], tol, report)
    check("ln2", cpu(L.ln2)[sl], c["ln2"][sl], tol, report)
    check("mu1", cpu(L.mu1)[sl], c["mu1"][sl], tol, report)
    check("rstd2", cpu(L.rs2)[sl], c["rstd2"][sl], tol, report)
    for r in ranks:
        v = oracle.rank_view(c, g, p64, cfg.heads, cfg.tp, r)
        a, gr = L.a[r], L.grads[r]
        check(f"r{r}.qkv", cpu(a["qkv"])[sl], v["qkv"][sl], tol, report)
        check(f"r{r}.ctx", cpu(a["ctx"])[sl], v["ctx"][sl], tol, report)
        check(f"r{r}.lse", cpu(a["lse"])[:, sl], v["lse"][:, sl], tol, report)
        check(f"r{r}.proj_partial", cpu(a["p"])[sl], v["proj_partial"][sl], tol, report)
        if getattr(cfg, "swiglu", False):
            from tensor_transformer_layer_04_amd.layer import swiglu_split
            ug, uu = swiglu_split(cpu(a["u"]), 1)
            check(f"r{r}.u_gate", ug[sl], v["u"][sl], tol, report)
            check(f"r{r}.u_up", uu[sl], v["u3"][sl], tol, report)
        else:
            check(f"r{r}.u", cpu(a["u"])[sl], v["u"][sl], tol, report)
        check(f"r{r}.g", cpu(a["g"])[sl], v["g"][sl], tol, report)
        check(f"r{r}.fc2_partial", cpu(a["q"])[sl], v["fc2_partial"][sl], tol, report)
        if getattr(cfg, "swiglu", False):
            dg_, du_ = swiglu_split(cpu(a["du"]), 1)
            check(f"r{r}.du_gate", dg_[sl], v["du"][sl], tol, report)
            check(f"r{r}.du_up", du_[sl], v["du3"][sl], tol, report)
        else:
            check(f"r{r}.du", cpu(a["du"])[sl], v["du"][sl], tol, report)
        check(f"r{r}.fc1_dx_partial", cpu(a["dln2"])[sl], v["fc1_dx_partial"][sl], tol, report)
        check(f"r{r}.dctx", cpu(a["dctx"])[sl], v["dctx"][sl], tol, report)
        check(f"r{r}.dqkv", cpu(a["dqkv"])[sl], v["dqkv"][sl], tol, report)
        check(f"r{r}.qkv_dx_partial", cpu(a["dln1"])[sl], v["qkv_dx_partial"][sl], tol, report)
        check(f"r{r}.dw2", cpu(gr["dw2"]), v["dw2"], tol, report)
        if getattr(cfg, "swiglu", False):
            w1g, w3g = swiglu_split(cpu(gr["dw1"]), 0)
            check(f"r{r}.dw1", w1g, v["dw1"], tol, report)
            check(f"r{r}.dw3", w3g, v["dw3"], tol, report)
        else:
            check(f"r{r}.dw1", cpu(gr["dw1"]), v["dw1"], tol, report)
            check(f"r{r}.db1", cpu(gr["db1"]), v["db1"], tol, report)
        check(f"r{r}.dwo", cpu(gr["dwo"]), v["dwo"], tol, report)
        check(f"r{r}.dwqkv", cpu(gr["dwqkv"]), v["dwqkv"], tol, report)
        check(f"r{r}.dbqkv", cpu(gr["dbqkv"]), v["dbqkv"], tol, report)
    check("dy1", cpu(L.dy1)[sl], g["dy1"][sl], tol, report)
    check("dx", cpu(L.dx)[sl], g["dx"][sl], tol, report)
    rg = L.rgrads
    for k in ("dln1_g", "dln1_b", "dln2_g", "dln2_b", "dbo", "db2"):
        check(k, cpu(rg[k]), g[k], tol, report)


def fmt_report(report: Dict[str, float]) -> str:
    worst = sorted(report.items(), key=lambda kv: -kv[1])[:6]
    return ", ".join(f"{k}={v:.2e}" for k, v in worst)
