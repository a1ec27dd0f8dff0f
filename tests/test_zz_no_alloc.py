"""The attention backward entry point that allocates nothing
(mtp_attn_bwd_noalloc) against the workspace one (mtp_attn_bwd), through
the C ABI (GPU): bit-identical outputs on two calls in a row, the second
with a smaller input, so the shared device buffer's leftover contents from
the first call must not leak into the second."""
import pytest
import torch

from gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(al, D, T, seed):
    g = torch.Generator().manual_seed(seed)
    qkv = (torch.randn(T, 3 * al * D, generator=g)).to(torch.bfloat16).cuda()
    dctx = torch.randn(T, al * D, generator=g).to(torch.bfloat16).cuda()
    return qkv, dctx


def _run(mtp, al, D, T, cu, seed):
    h = al * D
    d = mtp.make_desc(h, al, 0, 1, 0, T, 1, mtp.MTP_BF16)
    qkv, dctx = _inputs(al, D, T, seed)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu else None
    n = len(cu) - 1 if cu else 0
    ctx = torch.empty(T, h, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(al, T, dtype=torch.float32, device="cuda")
    mtp.mtp_attn_fwd(d, qkv, ctx, lse, cu_t, n)
    ref = torch.empty(T, 3 * h, dtype=torch.bfloat16, device="cuda")
    wsb = mtp.mtp_workspace_size(d, mtp.MTP_OP_ATTN_BWD)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    mtp.mtp_attn_bwd(d, qkv, ctx, lse, dctx, ref, cu_t, n, ws, wsb)
    got = torch.full((T, 3 * h), float("nan"), dtype=torch.bfloat16, device="cuda")
    mtp.mtp_attn_bwd_noalloc(d, qkv, ctx, lse, dctx, got, cu_t, n)
    torch.cuda.synchronize()
    return ref, got


def test_attn_bwd_noalloc_matches_workspace_call():
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    # first call: 16 heads of 128 over 2048 tokens (the 7B TP=2 shard);
    # second, smaller: 4 heads of 64 over 300 tokens in three documents
    for al, D, T, cu, seed in [(16, 128, 2048, None, 1), (4, 64, 300, [0, 7, 170, 300], 2)]:
        log(f"noalloc attention backward: a_l={al} d={D} T={T} cu={cu}")
        ref, got = _run(mtp, al, D, T, cu, seed)
        assert torch.equal(ref, got), f"a_l={al} T={T}: outputs differ"
