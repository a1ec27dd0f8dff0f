"""Host-side logic of the layer driver (CPU): the SwiGLU weight interleave,
the sequence-parallel row split checks, and the arithmetic identity the FP8
convert kernel relies on.  No GPU work."""
import os
import shutil
import subprocess

import pytest
import torch

import synth
from tensor_transformer_layer_04_amd.layer import TPLayer, swiglu_interleave, swiglu_split


def test_swiglu_interleave_layout_and_inverse():
    f, h = 16, 3
    gate = torch.arange(f * h, dtype=torch.float32).reshape(f, h)
    up = -gate - 1
    w = swiglu_interleave(gate, up)
    assert w.shape == (2 * f, h)
    # rows 8j..8j+3 are gate rows 4j..4j+3, rows 8j+4..8j+7 the up rows
    for j in range(f // 4):
        assert torch.equal(w[8 * j:8 * j + 4], gate[4 * j:4 * j + 4])
        assert torch.equal(w[8 * j + 4:8 * j + 8], up[4 * j:4 * j + 4])
    g2, u2 = swiglu_split(w, 0)
    assert torch.equal(g2, gate) and torch.equal(u2, up)
    # the same order along the columns of an activation [T, 2f]
    a = w.T.contiguous()
    g3, u3 = swiglu_split(a, 1)
    assert torch.equal(g3, gate.T) and torch.equal(u3, up.T)


@pytest.mark.parametrize("T,tp,ok", [(304, 2, True), (300, 2, False), (80, 4, True), (76, 4, False)])
def test_sequence_parallel_row_blocks(T, tp, ok):
    """Each rank's row block must be a multiple of 4 rows (16-byte aligned
    fp32 statistics); the blocks tile [0, T) in rank order."""
    cfg = synth.PARITY_CASES["small_bf16_tp2_sp"].replace(
        seq_len=T, tp=tp, hidden=256, heads=4, ffn=512)
    data = synth.generate(cfg)
    if not ok:
        with pytest.raises(ValueError):
            TPLayer(cfg, data, device="cpu", overlap=False)
        return
    # constructing the driver allocates host buffers only (no kernel runs)
    L = TPLayer(cfg, data, device="cpu", overlap=False)
    assert L.sp
    blocks = [L.rows[r] for r in range(tp)]
    assert blocks[0].start == 0 and blocks[-1].stop == T
    assert all(b.stop - b.start == T // tp and (b.stop - b.start) % 4 == 0 for b in blocks)
    assert all(blocks[r].stop == blocks[r + 1].start for r in range(tp - 1))


def _brute_pairs(chunks, cu):
    """Pairs (j, i < j) with some query of chunk j that sees some key of
    chunk i: same document and key before query, by enumeration."""
    doc = {}
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for t in range(a, b):
            doc[t] = s
    live = set()
    for j, (q0, q1) in enumerate(chunks):
        for i in range(j):
            k0, k1 = chunks[i]
            if any(doc[k] == doc[q] for q in range(q0, q1) for k in range(k0, k1)):
                live.add((j, i))
    return live


@pytest.mark.parametrize("T,cp,seed", [(1000, 4, 0), (960, 3, 1), (64, 8, 2), (777, 7, 3)])
def test_context_parallel_pairs_match_brute_force(T, cp, seed):
    """The block pairs the context-parallel path launches are exactly the
    pairs holding a visible (query, key) pair, for random packed documents
    (chunk edges inside and on document edges), in ring order; one sequence
    launches every pair."""
    from tensor_transformer_layer_04_amd.layer import cp_block_pairs
    g = torch.Generator().manual_seed(seed)
    L = T // cp
    chunks = [(c * L, (c + 1) * L) for c in range(cp)]
    T = L * cp
    for trial in range(20):
        cuts = sorted(set(torch.randint(1, T, (int(torch.randint(0, 12, (1,), generator=g)),),
                                        generator=g).tolist()))
        if trial == 0:
            cuts = [c for c in range(L, T, L)]  # documents exactly on the chunk edges
        cu = [0] + cuts + [T]
        got = cp_block_pairs(chunks, cu)
        assert set(got) == _brute_pairs(chunks, cu)
        for j in range(cp):  # ring order within a query chunk
            ii = [i for (jj, i) in got if jj == j]
            assert ii == sorted(ii, reverse=True)
        if trial == 0:
            assert got == []
    assert set(cp_block_pairs(chunks, None)) == {(j, i) for j in range(cp) for i in range(j)}


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU; asked for more it exits with a message
    before touching any device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_bench_model_flops_closed_forms():
    """The model FLOPs bench.py divides by: 2MNK per linear map and 4 d
    flops per visible (query, key) pair and local head, forward; the
    backward twice the forward.  At the 7B TP=2 shard (T = 2048, causal)
    that is 322.1 GFLOP of forward GEMMs, 17.2 GFLOP of forward attention
    and 1017.9 GFLOP per step; the SwiGLU FFN adds a third FFN matrix
    (another 2 T h f_l per direction)."""
    import bench
    import synth
    cfg = synth.get_config("7b_tp2")
    T, h, hl, fl = 2048, 4096, 2048, 5504
    cu = [0, T]
    f = bench.shard_flops(cfg, cu)
    gemm_fwd = 2 * T * hl * h * 3 + 2 * T * h * hl + 2 * 2 * T * h * fl
    attn_fwd = 4 * 128 * 16 * (T * (T + 1) // 2)
    assert f["gemm"] == 3 * gemm_fwd and round(gemm_fwd / 1e9, 1) == 322.1
    assert f["attn"] == 3 * attn_fwd and round(attn_fwd / 1e9, 1) == 17.2
    assert f["total"] == 3 * (gemm_fwd + attn_fwd) and round(f["total"] / 1e9, 1) == 1017.9
    assert sum(f["call"][k] for k in ("qkv_fwd", "proj_fwd", "fc1_fwd", "fc2_fwd")) == gemm_fwd
    sw = bench.shard_flops(synth.get_config("7b_tp2_swiglu_fp8"), cu)
    assert sw["total"] - f["total"] == 3 * 2 * T * h * fl
    assert sw["call"]["fc1_fwd"] == 2 * f["call"]["fc1_fwd"]
    # a document split adds no pair across documents
    assert bench.seq_pairs([0, 100, 300]) == 100 * 101 // 2 + 200 * 201 // 2


def test_bench_traffic_only_for_measured_workloads(monkeypatch):
    """The counter traffic bench.py reports is that of the workload and GEMM
    family the committed counter runs measured, and null for any other
    workload or once the GEMM source has changed."""
    import json
    import bench
    t = json.load(open(bench.TRAFFIC_FILE))
    assert t["gemm_source_sha"] == bench.source_digest(), "counter figures are stale"
    for w, e in t["workloads"].items():
        for k, v in e["bytes_per_launch"].items():
            assert bench.traffic_for(k, w) == v
            assert v >= e["algorithmic_bytes_per_launch"][k] > 0
    assert bench.traffic_for(bench.FWD_KERNEL, "7b_tp2") is not None
    assert bench.traffic_for(bench.FWD_KERNEL, "wide_tp8") is None
    assert bench.traffic_for(bench.FP8_KERNEL, "7b_tp2") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.traffic_for(bench.FWD_KERNEL, "7b_tp2") is None


def test_fp8_division_free_quotient_is_exact_on_every_bf16_pair(tmp_path):
    """The FP8 convert kernel forms fl32(x / s) as x * fl32(1/s) plus one FMA
    residual correction, with the sign of x, when s >= 2^-60.
    tests/host/fp8_quotient_check.c compares that with the IEEE quotient for
    every pair of bf16 values |x| <= amax and both formats' scales (about
    2e9 pairs): no pair may differ in a way that can change a code."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    src = os.path.join(os.path.dirname(__file__), "host", "fp8_quotient_check.c")
    exe = str(tmp_path / "fp8_quotient_check")
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(out.stdout.strip())
    assert out.returncode == 0, out.stdout
    assert out.stdout.split()[-1] == "0"
