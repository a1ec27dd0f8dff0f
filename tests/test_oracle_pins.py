"""Pins of the fp64 oracle against things other than itself.

Brute force on tiny inputs, closed forms, library special cases (torch CPU
fp64 used only as an independent pin), invariants of the pages' column/row
split, causality and central finite differences.  Each test is chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign or index,
a transposed operand) fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------- matmul
@pytest.mark.parametrize("m,k,n", [(3, 5, 7), (17, 9, 13)])
def test_linear_matches_triple_loop(m, k, n):
    r = rng(1)
    x, w, b = r.normal(size=(m, k)), r.normal(size=(n, k)), r.normal(size=n)
    ref = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = b[j]
            for kk in range(k):
                acc += x[i, kk] * w[j, kk]
            ref[i, j] = acc
    got = oracle.linear(x, w, b)
    assert np.max(np.abs(got - ref)) <= 1e-13 * np.max(np.abs(ref))


# ------------------------------------------------------------------ LayerNorm
def test_layernorm_matches_torch_and_moments():
    r = rng(2)
    x = r.normal(size=(37, 96)) * 3 + 1.5
    g, b = 1 + 0.1 * r.normal(size=96), 0.1 * r.normal(size=96)
    got, mu, rstd = oracle.layernorm(x, g, b, 1e-5)
    ref = F.layer_norm(torch.tensor(x), (96,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    # gamma = 1, beta = 0: each row has mean 0 and variance var/(var+eps)
    y, mu, rstd = oracle.layernorm(x, np.ones(96), np.zeros(96), 1e-5)
    var = x.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-12
    assert np.max(np.abs(y.var(axis=1) - var / (var + 1e-5))) < 1e-12
    assert np.allclose(mu, x.mean(axis=1), atol=1e-13)
    assert np.allclose(rstd, 1 / np.sqrt(var + 1e-5), rtol=1e-13)


def test_layernorm_backward_finite_difference():
    r = rng(3)
    x = r.normal(size=(5, 24))
    g, b = 1 + 0.1 * r.normal(size=24), 0.1 * r.normal(size=24)
    dout = r.normal(size=(5, 24))
    _, mu, rstd = oracle.layernorm(x, g, b, 1e-5)
    dx, dg, db = oracle.layernorm_backward(dout, x, g, mu, rstd)

    def L(x_, g_, b_):
        return float((oracle.layernorm(x_, g_, b_, 1e-5)[0] * dout).sum())
    eps = 1e-6
    for grad, which in ((dx, 0), (dg, 1), (db, 2)):
        v = r.normal(size=grad.shape)
        args_p = [x, g, b]
        args_m = [x, g, b]
        args_p[which] = args_p[which] + eps * v
        args_m[which] = args_m[which] - eps * v
        fd = (L(*args_p) - L(*args_m)) / (2 * eps)
        an = float((grad * v).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


# ----------------------------------------------------------------------- GeLU
def test_gelu_closed_forms_and_torch():
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu_tanh(np.array([10.0]))[0] - 10.0) < 1e-12
    assert abs(oracle.gelu_tanh(np.array([-10.0]))[0]) < 1e-12
    u = np.linspace(-6, 6, 1001)
    ref = F.gelu(torch.tensor(u), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu_tanh(u) - ref)) < 1e-14
    # derivative: central difference, and torch autograd as a second pin
    eps = 1e-6
    fd = (oracle.gelu_tanh(u + eps) - oracle.gelu_tanh(u - eps)) / (2 * eps)
    assert np.max(np.abs(fd - oracle.gelu_tanh_grad(u))) < 1e-8
    ut = torch.tensor(u, requires_grad=True)
    F.gelu(ut, approximate="tanh").sum().backward()
    assert np.max(np.abs(ut.grad.numpy() - oracle.gelu_tanh_grad(u))) < 1e-13
    # GeLU'(0) = 1/2
    assert abs(oracle.gelu_tanh_grad(np.array([0.0]))[0] - 0.5) < 1e-15


def test_silu_closed_forms_and_torch():
    """SiLU of the SwiGLU variant: SiLU(0) = 0, SiLU(z) -> z for large z and
    -> 0 for very negative z, torch's silu on a grid, and the derivative
    against central differences, autograd and SiLU'(0) = 1/2."""
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-14
    z = np.linspace(-12, 12, 1201)
    ref = F.silu(torch.tensor(z)).numpy()
    assert np.max(np.abs(oracle.silu(z) - ref)) < 1e-14
    eps = 1e-6
    fd = (oracle.silu(z + eps) - oracle.silu(z - eps)) / (2 * eps)
    assert np.max(np.abs(fd - oracle.silu_grad(z))) < 1e-8
    zt = torch.tensor(z, requires_grad=True)
    F.silu(zt).sum().backward()
    assert np.max(np.abs(zt.grad.numpy() - oracle.silu_grad(z))) < 1e-13
    assert abs(oracle.silu_grad(np.array([0.0]))[0] - 0.5) < 1e-15


# ------------------------------------------------------------------ attention
def _qkv(T, heads, d, seed):
    r = rng(seed)
    return (r.normal(size=(T, heads * d)), r.normal(size=(T, heads * d)),
            r.normal(size=(T, heads * d)))


def test_attention_rows_sum_to_one_and_causal_zeros():
    q, k, v = _qkv(19, 3, 8, 4)
    starts = oracle.doc_starts([0, 7, 19], 19)
    p = oracle.attention_probabilities(q, k, 3, starts)
    assert np.max(np.abs(p.sum(axis=2) - 1.0)) < 1e-12
    for i in range(19):
        for j in range(19):
            if j > i or j < starts[i]:
                assert np.all(p[:, i, j] == 0.0)


def test_attention_first_row_and_equal_keys():
    T, H, d = 23, 2, 16
    q, k, v = _qkv(T, H, d, 5)
    starts = oracle.doc_starts([0, 10, 23], T)
    ctx, _ = oracle.attention_forward(q, k, v, H, starts)
    # the first token of a document only sees itself
    for s in (0, 10):
        assert np.array_equal(ctx[s], v[s])
    # identical keys: uniform weights over the visible prefix
    k_eq = np.tile(k[:1], (T, 1))
    ctx2, _ = oracle.attention_forward(q, k_eq, v, H, starts)
    for i in range(T):
        ref = v[starts[i]:i + 1].mean(axis=0)
        assert np.max(np.abs(ctx2[i] - ref)) < 1e-13


def test_attention_matches_torch_sdpa_and_lse():
    T, H, d = 70, 3, 32
    q, k, v = _qkv(T, H, d, 6)
    starts = np.zeros(T, dtype=np.int64)
    ctx, lse = oracle.attention_forward(q, k, v, H, starts, row_block=16)
    qt = torch.tensor(q).view(T, H, d).transpose(0, 1)
    kt = torch.tensor(k).view(T, H, d).transpose(0, 1)
    vt = torch.tensor(v).view(T, H, d).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref.transpose(0, 1).reshape(T, H * d).numpy()
    assert np.max(np.abs(ctx - ref)) < 1e-12
    s = (qt @ kt.transpose(1, 2)) / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -math.inf)
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def test_attention_backward_matches_autograd_and_fd():
    T, H, d = 29, 2, 16
    q, k, v = _qkv(T, H, d, 7)
    starts = oracle.doc_starts([0, 12, 29], T)
    dctx = rng(8).normal(size=(T, H * d))
    dq, dk, dv = oracle.attention_backward(q, k, v, dctx, H, starts, row_block=8)
    # autograd through an explicit masked softmax in torch (library pin)
    allowed = torch.tensor(oracle.attention_probabilities(q, k, H, starts)[0] > 0)
    qt, kt, vt = (torch.tensor(a).view(T, H, d).transpose(0, 1).requires_grad_() for a in (q, k, v))
    s = (qt @ kt.transpose(1, 2)) / math.sqrt(d)
    s = s.masked_fill(~allowed, -math.inf)
    out = torch.softmax(s, dim=-1) @ vt
    out.transpose(0, 1).reshape(T, H * d).backward(torch.tensor(dctx))
    for got, t in ((dq, qt), (dk, kt), (dv, vt)):
        ref = t.grad.transpose(0, 1).reshape(T, H * d).numpy()
        assert np.max(np.abs(got - ref)) < 1e-12
    # central finite differences along random directions
    def L(q_, k_, v_):
        return float((oracle.attention_forward(q_, k_, v_, H, starts)[0] * dctx).sum())
    eps = 1e-6
    r = rng(9)
    for which, grad in enumerate((dq, dk, dv)):
        dirn = r.normal(size=grad.shape)
        a_p, a_m = [q, k, v], [q, k, v]
        a_p[which] = a_p[which] + eps * dirn
        a_m[which] = a_m[which] - eps * dirn
        fd = (L(*a_p) - L(*a_m)) / (2 * eps)
        an = float((grad * dirn).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_varlen_equals_separate_documents():
    T, H, d = 41, 2, 8
    q, k, v = _qkv(T, H, d, 10)
    cu = [0, 1, 15, 16, 41]
    starts = oracle.doc_starts(cu, T)
    ctx, lse = oracle.attention_forward(q, k, v, H, starts, row_block=7)
    dctx = rng(11).normal(size=(T, H * d))
    grads = oracle.attention_backward(q, k, v, dctx, H, starts, row_block=7)
    for a, b in zip(cu[:-1], cu[1:]):
        z = np.zeros(b - a, dtype=np.int64)
        c1, l1 = oracle.attention_forward(q[a:b], k[a:b], v[a:b], H, z)
        assert np.max(np.abs(ctx[a:b] - c1)) < 1e-13
        assert np.max(np.abs(lse[:, a:b] - l1)) < 1e-13
        g1 = oracle.attention_backward(q[a:b], k[a:b], v[a:b], dctx[a:b], H, z)
        for full, part in zip(grads, g1):
            assert np.max(np.abs(full[a:b] - part)) < 1e-12


# --------------------------------------------------------------- whole layer
def _tiny(seed=0, affine=True):
    cfg = synth.CONFIGS["tiny_tp2"].replace(affine_random=affine, seed=seed)
    data = synth.generate(cfg)
    starts = oracle.doc_starts(data["cu_seqlens"], cfg.tokens)
    return cfg, data, starts


def test_layer_causality_bit_identical():
    cfg, data, starts = _tiny()
    y0 = oracle.layer_forward(data, data["x"], cfg.heads, cfg.eps, starts)["y"]
    i = 60
    x = data["x"].clone()
    x[i + 1:] += torch.randn(x[i + 1:].shape, generator=torch.Generator().manual_seed(5))
    y1 = oracle.layer_forward(data, x, cfg.heads, cfg.eps, starts)["y"]
    assert np.array_equal(y0[:i + 1], y1[:i + 1])
    assert not np.allclose(y0[i + 1:], y1[i + 1:])


PARAM_GRADS = [("x", "dx"), ("ln1_g", "dln1_g"), ("ln1_b", "dln1_b"), ("wq", "dwq"),
               ("wk", "dwk"), ("wv", "dwv"), ("bqkv", "dbqkv"), ("wo", "dwo"), ("bo", "dbo"),
               ("ln2_g", "dln2_g"), ("ln2_b", "dln2_b"), ("w1", "dw1"), ("b1", "db1"),
               ("w2", "dw2"), ("b2", "db2")]


SWIGLU_PARAM_GRADS = [pg for pg in PARAM_GRADS if pg[0] != "b1"] + [("w3", "dw3")]


@pytest.mark.parametrize("variant", ["gelu", "swiglu"])
def test_layer_gradients_finite_difference(variant):
    """Central differences of L = sum(dy * y) on the tiny config, in fp64
    (GeLU FFN, and the SwiGLU FFN without its input bias)."""
    if variant == "gelu":
        cfg, data, starts = _tiny()
        param_grads = PARAM_GRADS
    else:
        cfg = synth.get_config("tiny_swiglu_tp2")
        data = synth.generate(cfg)
        starts = oracle.doc_starts(data["cu_seqlens"], cfg.tokens)
        param_grads = SWIGLU_PARAM_GRADS
    p64 = {k: oracle.to64(v) for k, v in data.items() if k not in ("cu_seqlens",)}
    dy = p64["dy"]
    cache = oracle.layer_forward(p64, p64["x"], cfg.heads, cfg.eps, starts)
    grads = oracle.layer_backward(p64, cache, dy, cfg.heads, starts)

    def L(pp):
        return float((oracle.layer_forward(pp, pp["x"], cfg.heads, cfg.eps, starts)["y"] * dy).sum())
    r = rng(12)
    eps = 1e-6
    for pname, gname in param_grads:
        grad = grads[gname]
        # one random direction plus one sampled single entry per tensor
        dirs = [r.normal(size=grad.shape)]
        e = np.zeros(grad.size)
        e[int(np.argmax(np.abs(grad).ravel()))] = 1.0
        dirs.append(e.reshape(grad.shape))
        for dirn in dirs:
            pp, pm = dict(p64), dict(p64)
            pp[pname] = p64[pname] + eps * dirn
            pm[pname] = p64[pname] - eps * dirn
            fd = (L(pp) - L(pm)) / (2 * eps)
            an = float((grad * dirn).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (pname, fd, an)


@pytest.mark.parametrize("name", ["tiny_tp2", "small_varlen_tp1"])
def test_layer_matches_torch_encoder_layer(name):
    """The whole layer's composition against a library special case: torch's
    ``nn.TransformerEncoderLayer`` with the LayerNorm first, no dropout and
    the tanh GeLU, in fp64 on the CPU, given the same weights and the causal
    (per-document) mask, with its gradients by autograd.  Every output and
    gradient of the oracle must agree to fp64 rounding."""
    cfg = synth.get_config(name).replace(affine_random=True)
    data = synth.generate(cfg)
    T, h = cfg.tokens, cfg.hidden
    p = {k: torch.as_tensor(oracle.to64(v)) for k, v in data.items()
         if k not in ("cu_seqlens", "targets")}
    layer = torch.nn.TransformerEncoderLayer(
        d_model=h, nhead=cfg.heads, dim_feedforward=cfg.ffn, dropout=0.0,
        activation=lambda u: F.gelu(u, approximate="tanh"), layer_norm_eps=cfg.eps,
        batch_first=True, norm_first=True, dtype=torch.float64)
    layer.train()
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(torch.cat([p["wq"], p["wk"], p["wv"]]))
        layer.self_attn.in_proj_bias.copy_(p["bqkv"])
        layer.self_attn.out_proj.weight.copy_(p["wo"])
        layer.self_attn.out_proj.bias.copy_(p["bo"])
        layer.linear1.weight.copy_(p["w1"])
        layer.linear1.bias.copy_(p["b1"])
        layer.linear2.weight.copy_(p["w2"])
        layer.linear2.bias.copy_(p["b2"])
        layer.norm1.weight.copy_(p["ln1_g"])
        layer.norm1.bias.copy_(p["ln1_b"])
        layer.norm2.weight.copy_(p["ln2_g"])
        layer.norm2.bias.copy_(p["ln2_b"])
    starts = oracle.doc_starts(data["cu_seqlens"], T)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    blocked = torch.as_tensor(~((j <= i) & (j >= starts[:, None])))  # True: not attended
    x = p["x"].clone().requires_grad_(True)
    y = layer(x[None], src_mask=blocked)[0]
    (y * p["dy"]).sum().backward()
    c = oracle.layer_forward(data, data["x"], cfg.heads, cfg.eps, starts)
    g = oracle.layer_backward(data, c, data["dy"], cfg.heads, starts)

    def close(a, b, what):
        a = a.detach().numpy() if isinstance(a, torch.Tensor) else a
        err = np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel())
        assert err <= 1e-10, f"{what}: rel {err:.2e}"
    close(y, c["y"], "y")
    close(x.grad, g["dx"], "dx")
    sa = layer.self_attn
    close(sa.in_proj_weight.grad, np.concatenate([g["dwq"], g["dwk"], g["dwv"]]), "dWqkv")
    close(sa.in_proj_bias.grad, g["dbqkv"], "dbqkv")
    close(sa.out_proj.weight.grad, g["dwo"], "dWo")
    close(sa.out_proj.bias.grad, g["dbo"], "dbo")
    close(layer.linear1.weight.grad, g["dw1"], "dW1")
    close(layer.linear1.bias.grad, g["db1"], "db1")
    close(layer.linear2.weight.grad, g["dw2"], "dW2")
    close(layer.linear2.bias.grad, g["db2"], "db2")
    close(layer.norm1.weight.grad, g["dln1_g"], "dln1_g")
    close(layer.norm1.bias.grad, g["dln1_b"], "dln1_b")
    close(layer.norm2.weight.grad, g["dln2_g"], "dln2_g")
    close(layer.norm2.bias.grad, g["dln2_b"], "dln2_b")


@pytest.mark.parametrize("tp,swiglu", [(1, False), (2, False), (4, False), (2, True), (4, True)])
def test_column_row_split_is_exact(tp, swiglu):
    """Sum over ranks of the row-parallel partials equals the unsharded product."""
    if swiglu:
        cfg = synth.get_config("tiny_swiglu_tp2").replace(seed=3)
        data = synth.generate(cfg)
        starts = oracle.doc_starts(data["cu_seqlens"], cfg.tokens)
    else:
        cfg, data, starts = _tiny(seed=3)
    p64 = {k: oracle.to64(v) for k, v in data.items() if k not in ("cu_seqlens",)}
    c = oracle.layer_forward(p64, p64["x"], cfg.heads, cfg.eps, starts)
    g = oracle.layer_backward(p64, c, p64["dy"], cfg.heads, starts)
    views = [oracle.rank_view(c, g, p64, cfg.heads, tp, r) for r in range(tp)]
    def tol(a):
        return 1e-12 * max(1.0, np.max(np.abs(a)))
    s = sum(v["proj_partial"] for v in views)
    assert np.max(np.abs(s - c["ctx"] @ p64["wo"].T)) < tol(s)
    s = sum(v["fc2_partial"] for v in views)
    assert np.max(np.abs(s - c["g"] @ p64["w2"].T)) < tol(s)
    s = sum(v["fc1_dx_partial"] for v in views)
    assert np.max(np.abs(s - g["dln2"])) < tol(s)
    s = sum(v["qkv_dx_partial"] for v in views)
    assert np.max(np.abs(s - g["dln1"])) < tol(s)
    # per-rank attention over the rank's local heads equals its slice
    h, hl, al = cfg.hidden, cfg.hidden // tp, cfg.heads // tp
    for r, v in enumerate(views):
        qkv_r = v["qkv"]
        ctx_r, lse_r = oracle.attention_forward(qkv_r[:, :hl], qkv_r[:, hl:2 * hl],
                                                qkv_r[:, 2 * hl:], al, starts)
        assert np.max(np.abs(ctx_r - v["ctx"])) < 1e-12
        assert np.max(np.abs(lse_r - v["lse"])) < 1e-12
    # concatenating rank slices restores the unsharded tensors
    assert np.array_equal(np.concatenate([v["ctx"] for v in views], axis=1), c["ctx"])
    assert np.array_equal(np.concatenate([v["u"] for v in views], axis=1), c["u"])
    assert np.array_equal(np.concatenate([v["dw1"] for v in views], axis=0), g["dw1"])


# ------------------------------------------------------------ vocab CE head
def test_vocab_ce_matches_torch_and_fd():
    r = rng(13)
    T, h, V = 9, 16, 50
    y, emb = r.normal(size=(T, h)), 0.3 * r.normal(size=(V, h))
    tg = r.integers(0, V, size=T)
    loss, z, lse = oracle.vocab_ce_forward(y, emb, tg)
    ref = F.cross_entropy(torch.tensor(y) @ torch.tensor(emb).T, torch.tensor(tg)).item()
    assert abs(loss - ref) < 1e-13
    dy, demb, dz = oracle.vocab_ce_backward(y, emb, tg, z, lse)
    assert np.max(np.abs(dz.sum(axis=1))) < 1e-15 * V
    yt, et = torch.tensor(y, requires_grad=True), torch.tensor(emb, requires_grad=True)
    F.cross_entropy(yt @ et.T, torch.tensor(tg)).backward()
    assert np.max(np.abs(yt.grad.numpy() - dy)) < 1e-14
    assert np.max(np.abs(et.grad.numpy() - demb)) < 1e-14
    eps = 1e-6
    for which, grad in ((0, dy), (1, demb)):
        dirn = r.normal(size=grad.shape)
        a_p, a_m = [y, emb], [y, emb]
        a_p[which] = a_p[which] + eps * dirn
        a_m[which] = a_m[which] - eps * dirn
        fd = (oracle.vocab_ce_forward(*a_p, tg)[0] - oracle.vocab_ce_forward(*a_m, tg)[0]) / (2 * eps)
        assert abs(fd - float((grad * dirn).sum())) < 1e-8


def test_vocab_ce_zero_logits_golden():
    """Zero logits over the pages' 131072-entry vocabulary: loss = ln V."""
    gold = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    V = gold["vocab_size"]["value"]
    T, h = 3, 4
    loss, _, _ = oracle.vocab_ce_forward(np.ones((T, h)), np.zeros((V, h)), np.array([0, 7, V - 1]))
    assert abs(loss - gold["zero_logit_cross_entropy"]["value"]) < 1e-12
    assert abs(loss - 17 * math.log(2)) < 1e-12


# ------------------------------------------------------------------- FP8
def test_e4m3_round_matches_torch_and_format():
    """E4M3 rounding against torch's float8_e4m3fn conversion (a library
    special case) on a grid with every tie, subnormal and binade edge, and
    the format's closed forms."""
    from oracle import fp8
    codes = np.arange(256)
    vals = fp8.e4m3_decode(codes)
    finite = np.sort(np.unique(vals[np.isfinite(vals)]))
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert np.min(finite[finite > 0]) == 2.0 ** -9
    mids = (finite[1:] + finite[:-1]) / 2          # every tie between neighbours
    r = rng(21)
    grid = np.concatenate([finite, mids, r.uniform(-448, 448, 4000),
                           r.uniform(-0.02, 0.02, 4000)])
    ref = torch.tensor(grid, dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_round(grid)
    assert np.array_equal(got, ref)
    # encode / decode are inverse on every finite value
    enc = fp8.e4m3_encode(finite)
    assert np.array_equal(fp8.e4m3_decode(enc), finite)
    assert fp8.e4m3_encode(np.array([448.0]))[0] == 0x7E
    assert fp8.e4m3_encode(np.array([-2.0 ** -9]))[0] == 0x81


def test_quantize_per_tensor_scale_and_linear():
    from oracle import fp8
    r = rng(22)
    x = r.normal(size=(37, 64)).astype(np.float32) * 3.0
    q, s = fp8.quantize_per_tensor(x)
    assert s == np.float32(np.max(np.abs(x)) / np.float32(448.0))
    assert np.max(np.abs(q)) == 448.0                  # amax maps to the largest value
    # dequantized values are within half an E4M3 step (relative 2^-4) of x
    big = np.abs(x) > 2.0 ** -6 * s
    assert np.all(np.abs(q * s - x)[big] <= np.abs(x)[big] * 2.0 ** -4 * 1.0001)
    qz, sz = fp8.quantize_per_tensor(np.zeros((3, 8), np.float32))
    assert sz == 1.0 and not qz.any()
    w = r.normal(size=(9, 64)).astype(np.float32)
    qw, sw = fp8.quantize_per_tensor(w)
    y = fp8.fp8_linear(q, s, qw, sw)
    brute = np.array([[sum(q[i, k] * qw[j, k] for k in range(64)) for j in range(9)]
                      for i in range(37)]) * (float(s) * float(sw))
    assert np.max(np.abs(y - brute)) <= 1e-12 * np.max(np.abs(brute))


def test_e5m2_round_matches_torch_and_format():
    """E5M2 rounding (the gradient format) against torch's float8_e5m2
    conversion on every finite value, every tie between neighbours and
    random values, and the format's closed forms."""
    from oracle import fp8
    codes = np.arange(256)
    vals = fp8.fp8_decode(codes, "e5m2")
    finite = np.sort(np.unique(vals[np.isfinite(vals)]))
    assert finite.max() == 57344.0 and finite.min() == -57344.0
    assert np.min(finite[finite > 0]) == 2.0 ** -16
    assert np.isinf(fp8.fp8_decode(np.array([0x7C]), "e5m2")[0])
    assert np.isnan(fp8.fp8_decode(np.array([0x7D]), "e5m2")[0])
    mids = (finite[1:] + finite[:-1]) / 2
    r = rng(23)
    grid = np.concatenate([finite, mids, r.uniform(-57344, 57344, 4000),
                           r.uniform(-1e-3, 1e-3, 4000)])
    ref = torch.tensor(grid, dtype=torch.float64).to(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(fp8.fp8_round(grid, "e5m2"), ref)
    enc = fp8.fp8_encode(finite, "e5m2")
    assert np.array_equal(fp8.fp8_decode(enc, "e5m2"), finite)
    assert fp8.fp8_encode(np.array([57344.0]), "e5m2")[0] == 0x7B
    assert fp8.fp8_encode(np.array([-2.0 ** -16]), "e5m2")[0] == 0x81
    # the two formats share nothing but the sign bit position
    assert fp8.fp8_encode(np.array([1.0]), "e5m2")[0] == 0x3C
    assert fp8.fp8_encode(np.array([1.0]), "e4m3")[0] == 0x38


def test_quantize_e5m2_and_gradient_products():
    from oracle import fp8
    r = rng(24)
    dy = r.normal(size=(33, 40)).astype(np.float32) * 0.01
    q, s = fp8.quantize_per_tensor(dy, "e5m2")
    assert s == np.float32(np.max(np.abs(dy)) / np.float32(57344.0))
    assert np.max(np.abs(q)) == 57344.0
    big = np.abs(dy) > 2.0 ** -14 * s
    assert np.all(np.abs(q * s - dy)[big] <= np.abs(dy)[big] * 2.0 ** -3 * 1.0001)
    w = r.normal(size=(40, 24)).astype(np.float32)       # y = x W^T with W [40, 24]
    qw, sw = fp8.quantize_per_tensor(w, "e4m3")
    x = r.normal(size=(33, 24)).astype(np.float32)
    qx, sx = fp8.quantize_per_tensor(x, "e4m3")
    dx = fp8.fp8_dgrad(q, s, qw, sw)
    dw = fp8.fp8_wgrad(q, s, qx, sx)
    brute_dx = np.array([[sum(q[i, n] * qw[n, k] for n in range(40)) for k in range(24)]
                         for i in range(33)]) * (float(s) * float(sw))
    brute_dw = np.array([[sum(q[t, n] * qx[t, k] for t in range(33)) for k in range(24)]
                         for n in range(40)]) * (float(s) * float(sx))
    assert np.max(np.abs(dx - brute_dx)) <= 1e-12 * np.max(np.abs(brute_dx))
    assert np.max(np.abs(dw - brute_dw)) <= 1e-12 * np.max(np.abs(brute_dw))


def _torch_fp8_quantize(x, fmt):
    """Per-tensor quantization written with torch's own float8 casts."""
    dt, mx = ((torch.float8_e4m3fn, 448.0) if fmt == "e4m3" else (torch.float8_e5m2, 57344.0))
    x32 = x.detach().float()
    amax = x32.abs().max()
    s = amax / torch.tensor(mx, dtype=torch.float32) if amax > 0 else torch.tensor(1.0)
    v = (x32 / s).clamp(-mx, mx)
    return v.to(dt).to(torch.float64), s.double()


class _TorchFP8Linear(torch.autograd.Function):
    """y = x W^T + b on E4M3 codes; gradients on the E5M2 codes of dy."""

    @staticmethod
    def forward(ctx, x, w, b):
        qx, sx = _torch_fp8_quantize(x, "e4m3")
        qw, sw = _torch_fp8_quantize(w, "e4m3")
        ctx.save_for_backward(qx, sx, qw, sw)
        return (qx @ qw.T) * (sx * sw) + b

    @staticmethod
    def backward(ctx, gy):
        qx, sx, qw, sw = ctx.saved_tensors
        qg, sg = _torch_fp8_quantize(gy, "e5m2")
        return (qg @ qw) * (sg * sw), (qg.T @ qx) * (sg * sx), gy.sum(0)


@pytest.mark.parametrize("name", ["tiny_tp2", "small_varlen_tp1", "tiny_swiglu_tp2"])
def test_fp8_layer_matches_torch_autograd(name):
    """The FP8 layer (forward and backward) against an independent build of
    it from torch library pieces: layer_norm, scaled_dot_product_attention
    with the same mask, tanh GeLU (or SiLU(gate) * up with the gate and up
    projections as one FP8 map), autograd for the chain rule, and an FP8
    linear function on torch's float8 casts.  Agreement to fp64 rounding."""
    import torch.nn.functional as F
    cfg = synth.get_config(name).replace(affine_random=True, dtype="f32")
    data = synth.generate(cfg)
    T, h, a = cfg.tokens, cfg.hidden, cfg.heads
    d = h // a
    P = {k: torch.as_tensor(oracle.to64(v)).clone().requires_grad_(True) for k, v in data.items()
         if k not in ("cu_seqlens", "targets", "x", "dy")}
    x = torch.as_tensor(oracle.to64(data["x"])).clone().requires_grad_(True)
    dy = torch.as_tensor(oracle.to64(data["dy"]))
    starts = oracle.doc_starts(data["cu_seqlens"], T)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    allowed = torch.as_tensor((j <= i) & (j >= starts[:, None]))
    wqkv = torch.cat([P["wq"], P["wk"], P["wv"]])
    ln1 = F.layer_norm(x, (h,), P["ln1_g"], P["ln1_b"], cfg.eps)
    qkv = _TorchFP8Linear.apply(ln1, wqkv, P["bqkv"])
    q, k, v = (qkv[:, n * h:(n + 1) * h].reshape(T, a, d).transpose(0, 1) for n in range(3))
    ctx = F.scaled_dot_product_attention(q, k, v, attn_mask=allowed).transpose(0, 1).reshape(T, h)
    y1 = x + _TorchFP8Linear.apply(ctx, P["wo"], P["bo"])
    ln2 = F.layer_norm(y1, (h,), P["ln2_g"], P["ln2_b"], cfg.eps)
    if cfg.swiglu:
        f = cfg.ffn
        u13 = _TorchFP8Linear.apply(ln2, torch.cat([P["w1"], P["w3"]]),
                                    torch.zeros(2 * f, dtype=torch.float64))
        g = F.silu(u13[:, :f]) * u13[:, f:]
    else:
        g = F.gelu(_TorchFP8Linear.apply(ln2, P["w1"], P["b1"]), approximate="tanh")
    y = y1 + _TorchFP8Linear.apply(g, P["w2"], P["b2"])
    (y * dy).sum().backward()
    c = oracle.layer_forward(data, data["x"], a, cfg.eps, starts, fp8=True)
    gr = oracle.layer_backward(data, c, data["dy"], a, starts)
    exact = oracle.layer_forward(data, data["x"], a, cfg.eps, starts)

    def close(t, ref, what, tol=1e-10):
        t = t.detach().numpy()
        err = np.linalg.norm((t - ref).ravel()) / np.linalg.norm(ref.ravel())
        assert err <= tol, f"{what}: rel {err:.2e}"
    close(y, c["y"], "y")
    close(x.grad, gr["dx"], "dx")
    for pn, gn in (SWIGLU_PARAM_GRADS if cfg.swiglu else PARAM_GRADS)[1:]:
        close(P[pn].grad, gr[gn], gn)
    # the FP8 layer is not the exact one, but within the formats' error
    e = np.linalg.norm(c["y"] - exact["y"]) / np.linalg.norm(exact["y"])
    assert 1e-4 < e < 5e-2, e


@pytest.mark.parametrize("tp,swiglu", [(2, False), (4, False), (2, True), (4, True)])
def test_fp8_column_row_split_is_exact(tp, swiglu):
    """With whole-tensor scales the ranks' FP8 partials still sum to the
    unsharded FP8 products (forward and backward), also with the SwiGLU
    FFN's gate and up rows taken per rank from the one map [W1; W3]."""
    if swiglu:
        cfg = synth.get_config("tiny_swiglu_tp2").replace(seed=4)
        data = synth.generate(cfg)
        starts = oracle.doc_starts(data["cu_seqlens"], cfg.tokens)
    else:
        cfg, data, starts = _tiny(seed=4)
    c = oracle.layer_forward(data, data["x"], cfg.heads, cfg.eps, starts, fp8=True)
    g = oracle.layer_backward(data, c, data["dy"], cfg.heads, starts)
    p64 = {k: oracle.to64(v) for k, v in data.items() if k not in ("cu_seqlens",)}
    views = [oracle.rank_view(c, g, p64, cfg.heads, tp, r) for r in range(tp)]
    proj = c["y1"] - p64["x"] - p64["bo"]
    fc2 = c["y"] - c["y1"] - p64["b2"]
    for key, ref in (("proj_partial", proj), ("fc2_partial", fc2)):
        tot = sum(v[key] for v in views)
        assert np.max(np.abs(tot - ref)) <= 1e-12 * np.max(np.abs(ref)), key
    # the column-dgrad partials sum to the FP8 input gradients of FC1 and QKV
    from oracle import fp8
    f8, g8 = c["fp8"], g["fp8"]
    dln2 = fp8.fp8_dgrad(g8["fc1"]["qdy"], g8["fc1"]["sdy"], f8["fc1"]["qw"], f8["fc1"]["sw"])
    dln1 = fp8.fp8_dgrad(g8["qkv"]["qdy"], g8["qkv"]["sdy"], f8["qkv"]["qw"], f8["qkv"]["sw"])
    for key, ref in (("fc1_dx_partial", dln2), ("qkv_dx_partial", dln1)):
        tot = sum(v[key] for v in views)
        assert np.max(np.abs(tot - ref)) <= 1e-12 * np.max(np.abs(ref)), key
