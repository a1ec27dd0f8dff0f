"""Context-parallel attention over packed documents at full size (GPU).

The packed 16384-token batch (documents of 256..4096 tokens, seeded) split
into 4 chunks of 4096 tokens, 32 heads of 128: each chunk's diagonal block,
then the earlier chunks its documents reach, merged by log-sum-exp, and the
backward of every launched block pair, through the C ABI in the order the
layer issues them.

Pinned two ways: (1) every document that crosses a chunk edge is a
self-contained attention problem, so the fp64 oracle runs on it alone (two
heads) and the whole document's ctx, lse, dq, dk, dv are compared; (2) every
row of every head is compared with the single-launch attention
(`mtp_attn_fwd` / `mtp_attn_bwd` over the same documents), itself pinned to
the oracle by the per-op and layer tests.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import TOL, check, log, require_gpu

pytestmark = pytest.mark.gpu


def test_context_parallel_varlen_full():
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    from tensor_transformer_layer_04_amd.layer import cp_block_pairs
    cfg = synth.CONFIGS["varlen_tp1_cp4"]
    T, al, D, cp = cfg.tokens, cfg.heads, cfg.head_dim, cfg.context_parallel
    h = al * D
    cu = synth.generate(cfg.replace(hidden=64, heads=1, ffn=64))["cu_seqlens"].tolist()
    L = T // cp
    chunks = [(c * L, (c + 1) * L) for c in range(cp)]
    pairs = cp_block_pairs(chunks, cu)
    log(f"cp varlen: T={T} heads={al} d={D} chunks={cp} docs={len(cu) - 1} pairs={pairs}")
    assert pairs, "the drawn documents cross no chunk edge"

    g = torch.Generator().manual_seed(7)
    qkv_h = torch.randn(T, 3 * h, generator=g).to(torch.bfloat16)
    dctx_h = torch.randn(T, h, generator=g).to(torch.bfloat16)
    qkv, dctx = qkv_h.cuda(), dctx_h.cuda()
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    n = len(cu) - 1
    d = mtp.make_desc(h, al, 0, 1, 0, T, 1, mtp.MTP_BF16)
    wsb = max(mtp.mtp_workspace_size(d, mtp.MTP_OP_ATTN_BWD), 256)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    E = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device="cuda")

    # single launch over the same documents
    ctx1, lse1, dqkv1 = E(T, h), E(al, T, dt=torch.float32), E(T, 3 * h)
    mtp.mtp_attn_fwd(d, qkv, ctx1, lse1, cu_t, n)
    mtp.mtp_attn_bwd(d, qkv, ctx1, lse1, dctx, dqkv1, cu_t, n, ws, wsb)

    # context-parallel blocks
    ctx, lse, dqkv = E(T, h), E(al, T, dt=torch.float32), E(T, 3 * h)
    ctx_p, lse_p = E(T, h), E(al, T, dt=torch.float32)
    for (q0, q1) in chunks:
        mtp.mtp_attn_fwd_block(d, qkv, q0, q1, q0, q1, ctx, lse, cu_t, n)
    for j, i in pairs:
        (q0, q1), (k0, k1) = chunks[j], chunks[i]
        mtp.mtp_attn_fwd_block(d, qkv, q0, q1, k0, k1, ctx_p, lse_p, cu_t, n)
        mtp.mtp_attn_merge(d, ctx, lse, ctx_p, lse_p, q0, q1)
    for (q0, q1) in chunks:
        mtp.mtp_attn_bwd_block(d, qkv, ctx, lse, dctx, dqkv, q0, q1, q0, q1, 0, ws, wsb, cu_t, n)
    for j, i in pairs:
        (q0, q1), (k0, k1) = chunks[j], chunks[i]
        mtp.mtp_attn_bwd_block(d, qkv, ctx, lse, dctx, dqkv, q0, q1, k0, k1, 1, ws, wsb, cu_t, n)
    torch.cuda.synchronize()
    log("  GPU done")

    got = {"ctx": ctx.float().cpu(), "lse": lse.cpu(), "dqkv": dqkv.float().cpu()}
    assert all(bool(torch.isfinite(v).all()) for v in got.values())

    # (2) every row against the single launch
    rep = {}
    check("ctx vs single launch", got["ctx"], ctx1.float().cpu().numpy().astype(np.float64),
          TOL["bf16"], rep)
    check("lse vs single launch", got["lse"], lse1.cpu().numpy().astype(np.float64), 1e-4, rep)
    check("dqkv vs single launch", got["dqkv"], dqkv1.float().cpu().numpy().astype(np.float64),
          TOL["bf16"], rep)

    # (1) the documents that cross a chunk edge, whole, against the oracle
    crossing = [(a, b) for a, b in zip(cu[:-1], cu[1:])
                if any(a < e < b for e in range(L, T, L))]
    assert crossing
    Q = oracle.to64(qkv_h)
    dO = oracle.to64(dctx_h)
    for (a, b) in crossing:
        for head in (0, al - 1):
            cols = slice(head * D, (head + 1) * D)
            q = Q[a:b, cols]
            k = Q[a:b, h + head * D:h + (head + 1) * D]
            v = Q[a:b, 2 * h + head * D:2 * h + (head + 1) * D]
            starts = oracle.doc_starts([0, b - a], b - a)
            rctx, rlse = oracle.attention_forward(q, k, v, 1, starts)
            dq, dk, dv = oracle.attention_backward(q, k, v, dO[a:b, cols], 1, starts)
            tag = f"doc [{a},{b}) head {head}"
            check(f"{tag} ctx", got["ctx"][a:b, cols], rctx, TOL["bf16"], rep)
            check(f"{tag} lse", got["lse"][head, a:b], rlse[0], TOL["bf16"], rep)
            g3 = got["dqkv"]
            check(f"{tag} dq", g3[a:b, cols], dq, TOL["bf16"], rep)
            check(f"{tag} dk", g3[a:b, h + head * D:h + (head + 1) * D], dk, TOL["bf16"], rep)
            check(f"{tag} dv", g3[a:b, 2 * h + head * D:2 * h + (head + 1) * D], dv, TOL["bf16"],
                  rep)
    log("  " + ", ".join(f"{k}={v:.1e}" for k, v in rep.items()))
