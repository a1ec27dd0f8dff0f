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
# End to end, an FP8 layer is not determined by its inputs to better than
# its formats' steps: a code is a discontinuous function of its input, so an
# input that differs by a relative d (the bf16 path against the fp64 oracle,
# d ~ 2^-8) lands on the neighbouring code with probability ~2d/e, moving the
# value by e (the relative step: e ~ 2^-3.5 for E4M3, 2^-2.5 for E5M2): a
# quantized product then deviates by ~sqrt(2 d e), about 3e-2 after one E4M3
# product and about 1e-1 after the E5M2 gradient products that follow it.
# The FP8 step is held to the bf16 tolerance product by product, on the
# GPU's own codes (which are bit-exact), and end to end to this bound.
FP8_E2E_TOL = 0.15


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


# Per-row bound: every row of a 2-D tensor (a token, a head's lse row, an
# output feature of a weight gradient) must itself be within ROW_MULT x tol
# of the oracle's row, relative to the larger of the row's own norm and
# ROW_FLOOR x the tensor's RMS row norm.  Rows much smaller than the tensor's
# scale are measured against that scale: the query gradient of a document's
# second token, for one, is P0 P1 (dP0 - dP1)(k0 - k1)/sqrt(d), tiny when one
# key dominates, while its rounding error (D = rowsum(dO * O) from the
# stored O) is not.  A wrong row or tile, which the per-tensor Frobenius
# error of a [2048, 4096] tensor could dilute below tol, gives a row error
# near 1.
ROW_MULT = 3.0
ROW_FLOOR = 0.5


def check(name: str, got, ref, tol: float, report: Dict[str, float], floor: float = 0.0) -> None:
    """rel-Frobenius error <= tol, and the per-row bound above.  ``floor``
    bounds the denominator from below for tensors whose exact value is
    identically zero (the query and key gradients when every document holds
    one token)."""
    got64, ref64 = oracle.to64(got), oracle.to64(ref)
    assert got64.shape == ref64.shape, f"{name}: shape {got64.shape} != {ref64.shape}"
    den = max(float(np.linalg.norm(ref64.ravel())), floor)
    e = float(np.linalg.norm((got64 - ref64).ravel())) / den if den > 0 else (
        0.0 if not np.any(got64) else float("inf"))
    report[name] = e
    assert np.isfinite(e) and e <= tol, f"{name}: rel-Frobenius {e:.3e} > {tol:.1e}"
    if ref64.ndim == 2 and ref64.shape[0] > 1 and ref64.size:
        rn = np.linalg.norm(ref64, axis=1)
        scale = max(den, 1e-300) / np.sqrt(ref64.shape[0])
        rden = np.maximum(rn, ROW_FLOOR * scale)
        rerr = np.linalg.norm(got64 - ref64, axis=1) / rden
        worst = int(np.argmax(rerr))
        report[name + "@row"] = float(rerr[worst])
        assert np.all(np.isfinite(rerr)) and rerr[worst] <= ROW_MULT * tol, (
            f"{name}: row {worst} relative error {rerr[worst]:.3e} > {ROW_MULT * tol:.1e}")


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


def compare_layer(cfg, L, c, g, data, report, rows=None, ranks=None, tol=None):
    """Element-wise comparison of every per-rank and summed tensor (at the
    dtype's tolerance unless ``tol`` is given)."""
    tol = TOL[cfg.dtype] if tol is None else tol
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
    tensor = {k: v for k, v in report.items() if not k.endswith("@row")}
    rows = {k: v for k, v in report.items() if k.endswith("@row")}
    worst = sorted(tensor.items(), key=lambda kv: -kv[1])[:5]
    worst_rows = sorted(rows.items(), key=lambda kv: -kv[1])[:3]
    return ", ".join(f"{k}={v:.2e}" for k, v in worst + worst_rows)


def oracle_head(cfg, data, c):
    """The oracle's vocab head on the layer output c["y"]: per-token loss,
    mean loss, dlogits, the head's input gradient and dE (unsharded)."""
    tg = data["targets"].numpy().astype(np.int64)
    loss, z, lse = oracle.vocab_ce_forward(c["y"], data["emb"], tg)
    dy_head, demb, dz = oracle.vocab_ce_backward(c["y"], data["emb"], tg, z, lse)
    per_tok = lse - z[np.arange(z.shape[0]), tg]
    return {"loss": loss, "per_tok": per_tok, "dz": dz, "dy": dy_head, "demb": demb}


def compare_head(cfg, H, h, report, ranks=None):
    """Every per-rank and summed output of the vocab head against ``h``
    (``oracle_head``): per-token loss, mean loss, each rank's dlogits,
    vocab weight gradient dE_r and input-gradient partial, and the summed
    input gradient."""
    tol = TOL[cfg.dtype]
    ranks = H.ranks if ranks is None else ranks
    vl = cfg.vocab // cfg.tp
    cpu = lambda t: t.detach().float().cpu()
    check("head.loss_rows", cpu(H.loss), h["per_tok"], tol, report)
    lm = float(H.loss_mean.item())
    report["head.loss_mean"] = abs(lm - h["loss"]) / abs(h["loss"])
    assert report["head.loss_mean"] <= tol, f"loss mean {lm} vs {h['loss']}"
    for r in ranks:
        cols = slice(r * vl, (r + 1) * vl)
        check(f"r{r}.dlogits", cpu(H.dlogits[r]), h["dz"][:, cols], tol, report)
        check(f"r{r}.demb", cpu(H.demb[r]), h["demb"][cols], tol, report)
        check(f"r{r}.head_dy_partial", cpu(H.dy_part[r]),
              h["dz"][:, cols] @ oracle.to64(H.emb[r].cpu()), tol, report)
    check("head.dy", cpu(H.dy), h["dy"], tol, report)


def run_gpu_layer_with_head(cfg, data):
    """Layer + vocab head, every rank, forward and backward (the layer's
    upstream gradient is the head's input gradient)."""
    from tensor_transformer_layer_04_amd.layer import TPLayer, VocabHead
    L = TPLayer(cfg, data, device="cuda", cu_seqlens=data["cu_seqlens"])
    H = VocabHead(cfg, data, device="cuda")
    y = L.forward(data["x"].cuda().contiguous())
    H.forward(y)
    L.backward(H.backward())
    torch.cuda.synchronize()
    return L, H


def compare_fp8_components(cfg, L, report):
    """The FP8 step of a layer that ran every rank, component by component:
    (a) every code and scale it used, bit for bit against the oracle's
    quantization of the GPU's own tensor (the whole tensor: its ranks'
    shards together), in both layouts; (b) every FP8 product against the
    oracle's product of those codes, at the bf16 tolerance."""
    from oracle import fp8 as f8
    tol = TOL["bf16"]
    cpu = lambda t: t.detach().float().cpu()
    R = L.ranks
    assert R == list(range(cfg.tp)), "components need every rank"

    def codes(name, shards, slots, fmt):
        whole = np.concatenate([cpu(x).numpy().reshape(-1) for x in shards])
        qw, s = f8.quantize_per_tensor(whole, fmt)
        enc = f8.fp8_encode(qw, fmt)
        out, off = [], 0
        for x, sl in zip(shards, slots):
            n = x.numel()
            rows, cols = x.shape
            q = qw[off:off + n].reshape(rows, cols)
            e = enc[off:off + n].reshape(rows, cols)
            off += n
            assert float(sl["s"][0]) == float(s), f"{name}: scale {float(sl['s'][0])} != {float(s)}"
            assert np.array_equal(sl["q"].cpu().numpy(), e), f"{name}: codes differ"
            assert np.array_equal(sl["qt"].cpu().numpy(), e.T), f"{name}: transposed codes differ"
            out.append((q, s))
        report[f"codes.{name}"] = 0.0
        return out
    E4, E5 = "e4m3", "e5m2"
    (ln1,), (ln2,) = codes("ln1", [L.ln1], [L.q8["ln1"]], E4), codes("ln2", [L.ln2], [L.q8["ln2"]], E4)
    (dy,), (dy1,) = (codes("dy", [L.dy_seen], [L.q8["dy"]], E5),
                     codes("dy1", [L.dy1], [L.q8["dy1"]], E5))
    split = {}
    for name, src, fmt in (("wqkv", lambda r: L.w[r]["wqkv"], E4), ("wo", lambda r: L.w[r]["wo"], E4),
                           ("w1", lambda r: L.w[r]["w1"], E4), ("w2", lambda r: L.w[r]["w2"], E4),
                           ("ctx", lambda r: L.a[r]["ctx"], E4), ("g", lambda r: L.a[r]["g"], E4),
                           ("du", lambda r: L.a[r]["du"], E5), ("dqkv", lambda r: L.a[r]["dqkv"], E5)):
        split[name] = codes(name, [src(r) for r in R], [L.r8[r][name] for r in R], fmt)
    for r in R:
        a, gr, w = L.a[r], L.grads[r], L.w[r]
        (qwqkv, swqkv), (qwo, swo) = split["wqkv"][r], split["wo"][r]
        (qw1, sw1), (qw2, sw2) = split["w1"][r], split["w2"][r]
        (qctx, sctx), (qg, sg) = split["ctx"][r], split["g"][r]
        (qdu, sdu), (qdq, sdq) = split["du"][r], split["dqkv"][r]
        u = oracle.to64(cpu(a["u"]))
        check(f"r{r}.fp8_qkv", cpu(a["qkv"]), f8.fp8_linear(*ln1, qwqkv, swqkv, oracle.to64(w["bqkv"].cpu())), tol, report)
        check(f"r{r}.fp8_proj", cpu(a["p"]), f8.fp8_linear(qctx, sctx, qwo, swo), tol, report)
        if getattr(cfg, "swiglu", False):
            # gate|up interleaved in groups of 4 columns (rows of W1|W3)
            from tensor_transformer_layer_04_amd.layer import swiglu_split
            uref = f8.fp8_linear(*ln2, qw1, sw1)
            check(f"r{r}.fp8_u", cpu(a["u"]), uref, tol, report)
            gt, up = (oracle.to64(t) for t in swiglu_split(torch.from_numpy(u), 1))
            gr_, ur_ = (t.numpy() for t in swiglu_split(torch.from_numpy(uref), 1))
            check(f"r{r}.fp8_g", cpu(a["g"]), oracle.silu(gr_) * ur_, tol, report)
            dg = f8.fp8_dgrad(*dy, qw2, sw2)
            dgate, dup = (t.float() for t in swiglu_split(cpu(a["du"]), 1))
            check(f"r{r}.fp8_dgate", dgate, dg * up * oracle.silu_grad(gt), tol, report)
            check(f"r{r}.fp8_dup", dup, dg * oracle.silu(gt), tol, report)
        else:
            uref = f8.fp8_linear(*ln2, qw1, sw1, oracle.to64(w["b1"].cpu()))
            check(f"r{r}.fp8_u", cpu(a["u"]), uref, tol, report)
            check(f"r{r}.fp8_g", cpu(a["g"]), oracle.gelu_tanh(uref), tol, report)
            check(f"r{r}.fp8_du", cpu(a["du"]), f8.fp8_dgrad(*dy, qw2, sw2) * oracle.gelu_tanh_grad(u), tol, report)
        check(f"r{r}.fp8_fc2", cpu(a["q"]), f8.fp8_linear(qg, sg, qw2, sw2), tol, report)
        check(f"r{r}.fp8_dw2", cpu(gr["dw2"]), f8.fp8_wgrad(*dy, qg, sg), tol, report)
        check(f"r{r}.fp8_dln2", cpu(a["dln2"]), f8.fp8_dgrad(qdu, sdu, qw1, sw1), tol, report)
        check(f"r{r}.fp8_dw1", cpu(gr["dw1"]), f8.fp8_wgrad(qdu, sdu, *ln2), tol, report)
        check(f"r{r}.fp8_dctx", cpu(a["dctx"]), f8.fp8_dgrad(*dy1, qwo, swo), tol, report)
        check(f"r{r}.fp8_dwo", cpu(gr["dwo"]), f8.fp8_wgrad(*dy1, qctx, sctx), tol, report)
        check(f"r{r}.fp8_dln1", cpu(a["dln1"]), f8.fp8_dgrad(qdq, sdq, qwqkv, swqkv), tol, report)
        check(f"r{r}.fp8_dwqkv", cpu(gr["dwqkv"]), f8.fp8_wgrad(qdq, sdq, *ln1), tol, report)
