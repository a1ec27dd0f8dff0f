"""Full-layer parity of the HIP path against the fp64 oracle (GPU).

Every per-rank tensor (QKV shard, attention context and log-sum-exp,
row-parallel partials, FC1 pre-activation and GeLU output, all gradients)
and every summed tensor is compared element-wise by relative Frobenius
error: <= 1e-4 for fp32 shards, <= 2e-2 for bf16 with fp32 accumulation.

Full sizes the oracle cannot finish in seconds are checked on a prefix: by
causality (and the block-diagonal mask), the first P output rows depend
only on the first P input rows, and a backward whose upstream gradient is
zero beyond row P equals the prefix problem's backward exactly (every
gradient, weight gradients included).  The GPU still runs the whole
sequence in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import (TOL, check, compare_layer, fmt_report, log, oracle_layer, require_gpu,
                        run_gpu_layer)

pytestmark = pytest.mark.gpu

SMALL = ["tiny_tp2", "small_f32_tp4", "small_bf16_tp2", "small_bf16_d64_tp4", "small_bf16_mb2",
         "small_varlen_tp1", "one_token_bf16", "small_bf16_tp2_sp", "small_f32_tp4_sp",
         "tiny_swiglu_tp2", "small_bf16_swiglu_tp2", "small_bf16_swiglu_sp_tp4",
         "small_bf16_tp2_cp2", "small_bf16_d64_cp4", "small_varlen_cp4",
         "small_varlen_d64_tp2_cp3"]


@pytest.mark.parametrize("name", SMALL)
def test_layer_parity_small(name):
    require_gpu()
    cfg = synth.get_config(name)
    log(f"layer parity {name}: T={cfg.tokens} h={cfg.hidden} tp={cfg.tp} {cfg.dtype}")
    data = synth.generate(cfg)
    L = run_gpu_layer(cfg, data)
    c, g = oracle_layer(cfg, data)
    report = {}
    compare_layer(cfg, L, c, g, data, report)
    log(f"  worst: {fmt_report(report)}")


def test_layer_parity_7b_tp2_full():
    """Pages' 7B-style layer, both TP=2 shards, full size, full oracle."""
    require_gpu()
    cfg = synth.CONFIGS["7b_tp2"]
    log("layer parity 7b_tp2 (full size, both ranks)")
    data = synth.generate(cfg)
    L = run_gpu_layer(cfg, data)
    log("  GPU done; running oracle")
    c, g = oracle_layer(cfg, data)
    report = {}
    compare_layer(cfg, L, c, g, data, report)
    log(f"  worst: {fmt_report(report)}")


@pytest.mark.parametrize("name", ["7b_tp2_sp", "7b_tp2_swiglu", "7b_tp2_cp2"])
def test_layer_parity_7b_variants_full(name):
    """The 7B-style TP=2 layer with sequence parallelism and with the SwiGLU
    FFN: both shards at full size against the full oracle."""
    require_gpu()
    cfg = synth.CONFIGS[name]
    log(f"layer parity {name} (full size, both ranks)")
    data = synth.generate(cfg)
    L = run_gpu_layer(cfg, data)
    log("  GPU done; running oracle")
    c, g = oracle_layer(cfg, data)
    report = {}
    compare_layer(cfg, L, c, g, data, report)
    log(f"  worst: {fmt_report(report)}")


def _prefix_case(name, P):
    require_gpu()
    cfg = synth.CONFIGS[name]
    log(f"layer prefix parity {name}: T={cfg.tokens}, prefix {P}")
    data = synth.generate(cfg)
    dy = torch.zeros(cfg.tokens, cfg.hidden, dtype=cfg.torch_dtype)
    dy[:P] = torch.randn(P, cfg.hidden, generator=torch.Generator().manual_seed(cfg.seed + 1)).to(dy.dtype)
    L = run_gpu_layer(cfg, data, dy=dy)
    log("  GPU done; running oracle on the prefix")
    pre = cfg.replace(varlen_tokens=P if cfg.varlen_tokens else 0, seq_len=P, micro_batch=1)
    pdata = dict(data)
    pdata["x"] = data["x"][:P]
    cu = data["cu_seqlens"].tolist()
    pdata["cu_seqlens"] = torch.tensor([v for v in cu if v < P] + [P], dtype=torch.int32)
    c, g = oracle_layer(pre, pdata, dy=dy[:P])
    report = {}
    compare_layer(pre, L, c, g, pdata, report, rows=P)
    # rows past the prefix received zero upstream gradient: their input
    # gradient is exactly zero.
    assert float(L.dx[P:].abs().max()) == 0.0
    log(f"  worst: {fmt_report(report)}")


def test_layer_prefix_wide_tp8():
    _prefix_case("wide_tp8", 192)


def test_layer_prefix_varlen_tp1():
    cfg = synth.CONFIGS["varlen_tp1"]
    data_cu = synth.generate(cfg.replace(hidden=64, heads=1, ffn=64))["cu_seqlens"]
    # two full documents and part of the third
    P = int(data_cu[2]) + 100
    _prefix_case("varlen_tp1", min(P, 1024))


def test_layer_prefix_bench_tp4_with_vocab_head():
    """Benchmark-shaped layer plus the vocab-parallel CE head, all 4 ranks."""
    require_gpu()
    from tensor_transformer_layer_04_amd.layer import TPLayer, VocabHead
    cfg = synth.CONFIGS["bench_tp4_vocab"]
    P = 128
    log(f"bench_tp4_vocab: T={cfg.tokens} V={cfg.vocab}, prefix {P}")
    data = synth.generate(cfg)
    L = TPLayer(cfg, data, device="cuda", cu_seqlens=data["cu_seqlens"])
    H = VocabHead(cfg, data, device="cuda")
    y = L.forward(data["x"].cuda())
    H.forward(y)
    dyh = H.backward()
    torch.cuda.synchronize()
    log("  GPU forward + head done; oracle on the prefix")
    pre = cfg.replace(seq_len=P)
    pdata = dict(data)
    pdata["x"] = data["x"][:P]
    pdata["cu_seqlens"] = torch.tensor([0, P], dtype=torch.int32)
    starts = oracle.doc_starts(pdata["cu_seqlens"], P)
    c = oracle.layer_forward(pdata, pdata["x"], cfg.heads, cfg.eps, starts)
    tol = TOL[cfg.dtype]
    report = {}
    check("y", y[:P].float().cpu(), c["y"], tol, report)
    # per-token loss and dlogits rows of the prefix (row-wise quantities);
    # the oracle's mean is over its P rows, the GPU's over T: rescale.
    tg = data["targets"][:P].numpy()
    loss, z, lse = oracle.vocab_ce_forward(c["y"], data["emb"], tg)
    per_tok = lse - z[np.arange(P), tg]
    check("loss_rows", H.loss[:P].cpu(), per_tok, tol, report)
    _, _, dz = oracle.vocab_ce_backward(c["y"], data["emb"], tg, z, lse)
    vl = cfg.vocab // cfg.tp
    dl = torch.cat([H.dlogits[r][:P].float().cpu() for r in range(cfg.tp)], 1) * (cfg.tokens / P)
    check("dlogits_rows", dl, dz, tol, report)
    dy_head = dz @ oracle.to64(data["emb"]) * (P / cfg.tokens)
    check("head_dy_rows", dyh[:P].float().cpu(), dy_head, tol, report)
    log(f"  worst: {fmt_report(report)}")
    del vl


def test_layer_causality_bitwise():
    """Perturbing tokens after i leaves outputs 0..i bit-identical on the GPU."""
    require_gpu()
    cfg = synth.get_config("small_bf16_tp2")
    data = synth.generate(cfg)
    L = run_gpu_layer(cfg, data, with_backward=False)
    y0 = L.y.clone()
    i = 150
    d2 = dict(data)
    x = data["x"].clone()
    x[i + 1:] = torch.randn(x[i + 1:].shape, generator=torch.Generator().manual_seed(9)).to(x.dtype)
    d2["x"] = x
    L2 = run_gpu_layer(cfg, d2, with_backward=False)
    assert torch.equal(y0[:i + 1], L2.y[:i + 1])
    assert not torch.equal(y0[i + 1:], L2.y[i + 1:])


def test_layer_deterministic():
    """Two runs give bitwise-equal outputs and gradients (no atomics)."""
    require_gpu()
    cfg = synth.get_config("small_varlen_tp1")
    data = synth.generate(cfg)
    A = run_gpu_layer(cfg, data)
    B = run_gpu_layer(cfg, data)
    assert torch.equal(A.y, B.y) and torch.equal(A.dx, B.dx)
    for r in A.ranks:
        for k in A.grads[r]:
            assert torch.equal(A.grads[r][k], B.grads[r][k]), k


def test_sum_of_partials_equals_unsharded():
    """Pages' invariant on the GPU path: the t-way sum of row-parallel
    partials equals the oracle's unsharded product (TP=2 and TP=4 of the
    same weights give the same layer output)."""
    require_gpu()
    base = synth.get_config("small_bf16_tp2")
    outs = []
    for tp in (1, 2, 4):
        cfg = base.replace(tp=tp)
        data = synth.generate(cfg)
        L = run_gpu_layer(cfg, data, with_backward=False)
        outs.append(L.y.float().cpu())
    c, _ = oracle_layer(base, synth.generate(base))
    for y in outs:
        assert oracle.rel_frobenius(y, c["y"]) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["small_bf16_tp2_sp", "small_f32_tp4_sp"])
def test_sequence_parallel_matches_replicated(name):
    """Sequence parallelism only moves the per-token work onto row blocks:
    every row-wise output is bit-identical to the replicated layer's, and
    the LayerNorm and row-parallel bias gradients (column sums now added
    rank by rank) agree to fp32 rounding."""
    require_gpu()
    cfg = synth.get_config(name)
    data = synth.generate(cfg)
    L_sp = run_gpu_layer(cfg, data)
    L_rep = run_gpu_layer(cfg.replace(sequence_parallel=False), data)
    assert L_sp.sp and not L_rep.sp
    for k in ("ln1", "mu1", "rs1", "y1", "ln2", "mu2", "rs2", "y", "dy1", "dx"):
        a, b = getattr(L_sp, k), getattr(L_rep, k)
        assert torch.equal(a, b), f"{name}: {k} differs"
    for r in L_sp.ranks:
        for k in L_sp.a[r]:
            assert torch.equal(L_sp.a[r][k], L_rep.a[r][k]), f"{name}: r{r}.{k} differs"
    for k in L_sp.rgrads:
        a, b = L_sp.rgrads[k].double().cpu(), L_rep.rgrads[k].double().cpu()
        err = float((a - b).norm() / max(float(b.norm()), 1e-30))
        log(f"  {k}: rel diff {err:.2e}")
        assert err <= 1e-5, f"{name}: {k} rel diff {err}"


def test_sequence_parallel_one_rank_with_resident_rows():
    """The timed shard of the sequence-parallel workload: rank 0 alone, the
    other rank's partials and row blocks resident from a full run, gives
    rank 0's rows of every row-wise output bit-identically."""
    require_gpu()
    from tensor_transformer_layer_04_amd.layer import TPLayer
    cfg = synth.get_config("small_bf16_tp2_sp")
    data = synth.generate(cfg)
    full = run_gpu_layer(cfg, data)
    ref = {k: getattr(full, k).clone() for k in ("y1", "y", "dy1", "dx", "ln1", "ln2")}
    parts = full.partials()
    ext = {k: [v[i] for i, r in enumerate(full.ranks) if r != 0] for k, v in parts.items()}
    L = TPLayer(cfg, data, ranks=[0], device="cuda", cu_seqlens=data["cu_seqlens"])
    L.adopt_rows(full)
    # poison rank 0's rows of the shared buffers: the shard must rewrite them
    rows = L.rows[0]
    for k in ("ln1", "y1", "ln2", "y", "dy1", "dx"):
        getattr(L, k)[rows] = float("nan")
    L.forward(data["x"].cuda().contiguous(), ext)
    L.backward(data["dy"].cuda().contiguous(), ext)
    torch.cuda.synchronize()
    for k, v in ref.items():
        assert torch.equal(getattr(L, k)[rows], v[rows]), f"rank-0 rows of {k} differ"
