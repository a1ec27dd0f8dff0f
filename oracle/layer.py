"""fp64 CPU oracle of one pre-LN GPT transformer layer, forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path and imports nothing from it; inputs come from the
seeded generators in ``synth`` (which hold no arithmetic of the layer).

What it computes
----------------
The tensor-parallel split of the pages (column-parallel Q/K/V projections
with the input broadcast to every rank, row-parallel output projection whose
per-rank partials are summed) reaches exactly the result of the unsharded
layer (page "Megatron-LM 3D parallelism guide", §2.1 "Tensor parallelism").
So the oracle is the plain definition of the unsharded pre-LN layer:

    ln1 = LN(x)                          qkv = ln1 Wqkv^T + bqkv
    ctx = softmax(q k^T / sqrt(d) + mask) v      (per head, fp64 softmax)
    y1  = x + ctx Wo^T + bo
    ln2 = LN(y1)      u = ln2 W1^T + b1     g = GeLU_tanh(u)
    y   = y1 + g W2^T + b2

or, in the SwiGLU variant without linear biases on the FFN input (present
when the parameters hold an up projection ``w3``; page "Megatron-LM 3D
parallelism guide", §3.3 launch flags ``--swiglu --disable-bias-linear``):

    u = ln2 W1^T (gate)    u3 = ln2 W3^T (up)    g = SiLU(u) * u3

and its backward by the chain rule.  The rank view (which slice of each
tensor a given rank computes) is in ``rank_view``.

With ``fp8=True`` the same layer runs its twelve products on FP8 codes with
per-tensor scales (``oracle.fp8``): each forward map on the E4M3 codes of
its input and weight, each data and weight gradient on the E5M2 codes of the
incoming gradient and the forward's E4M3 codes; everything else (LayerNorm,
attention, GeLU / SwiGLU, residuals, bias gradients) stays as above.  In the
SwiGLU variant the gate and up projections are one FFN input map,
[u | u3] = ln2 [W1; W3]^T, whose weight [W1; W3] is one tensor with one
scale, and whose incoming gradient [du | du3] is one E5M2 tensor (reading:
the pages name the flags, not a recipe; one map, one scale each).

Readings where the pages are silent (each is a stated choice, not a fact of the pages):
pre-LN; LayerNorm with population variance and eps inside the square root;
score scale 1/sqrt(head_dim); the mask keeps key j for query i iff
j <= i and j lies in i's document; GeLU is the tanh form; Wqkv stacks
separate Wq, Wk, Wv blocks, head n owning columns n*d .. n*d+d-1 of each;
row-parallel biases are added once after the sum; no dropout.

The parity of these functions is pinned in tests/test_oracle_pins.py against
brute force, closed forms, library special cases (torch CPU fp64),
invariants and central finite differences.  The pages print no worked
numeric example, so no value is pinned to a printed one.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "to64", "linear", "layernorm", "layernorm_backward", "gelu_tanh", "gelu_tanh_grad",
    "silu", "silu_grad",
    "doc_starts", "attention_probabilities", "attention_forward", "attention_backward",
    "layer_forward", "layer_backward", "vocab_ce_forward", "vocab_ce_backward",
    "rank_view", "rel_frobenius",
]

GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


def to64(t) -> np.ndarray:
    """Any torch tensor / array-like -> float64 numpy array (exact for bf16/fp32)."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F (0 when both are zero)."""
    got = to64(got)
    ref = to64(ref)
    num = float(np.linalg.norm((got - ref).ravel()))
    den = float(np.linalg.norm(ref.ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


# ---------------------------------------------------------------- linear maps
def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x W^T + b with W stored [out, in] (nn.Linear convention).

    The pages' ColumnParallelLinear / RowParallelLinear wrap exactly this map
    (page "Megatron-LM: NVIDIA's large-model training framework", section
    "Tensor parallelism" snippet).
    """
    y = x @ w.T
    if b is not None:
        y = y + b
    return y


# ------------------------------------------------------------------ LayerNorm
def layernorm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float):
    """Textbook LayerNorm over the last axis (Ba, Kiros & Hinton 2016).

    mu = mean(x), var = mean((x-mu)^2) (population), xhat = (x-mu)/sqrt(var+eps),
    out = gamma*xhat + beta.  The pages name a fused LayerNorm kernel
    (page "Megatron-LM 3D parallelism guide", §4.2); under the column/row split
    every rank sees the whole hidden vector, so the statistics are local.
    Returns (out, mean[T], rstd[T]).
    """
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    out = (x - mu) * rstd * gamma + beta
    return out, mu[..., 0], rstd[..., 0]


def layernorm_backward(dout, x, gamma, mean, rstd):
    """Gradient of ``layernorm`` w.r.t. x, gamma, beta.

    With xhat = (x-mu)*rstd and gh = dout*gamma, the Jacobian of the
    normalisation gives dx = rstd*(gh - mean(gh) - xhat*mean(gh*xhat)).
    dgamma = sum_T dout*xhat, dbeta = sum_T dout.
    """
    xhat = (x - mean[:, None]) * rstd[:, None]
    gh = dout * gamma
    dx = rstd[:, None] * (gh - gh.mean(axis=1, keepdims=True)
                          - xhat * (gh * xhat).mean(axis=1, keepdims=True))
    return dx, (dout * xhat).sum(axis=0), dout.sum(axis=0)


# ----------------------------------------------------------------------- GeLU
def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """GeLU, tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(GELU_C * (u + GELU_A * u ** 3)))


def gelu_tanh_grad(u: np.ndarray) -> np.ndarray:
    """d/du of ``gelu_tanh`` (product and chain rule, tanh' = 1 - tanh^2)."""
    z = GELU_C * (u + GELU_A * u ** 3)
    th = np.tanh(z)
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th ** 2) * GELU_C * (1.0 + 3.0 * GELU_A * u ** 2)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU (swish): z * sigmoid(z), the sigmoid written as (1 + tanh(z/2)) / 2
    so that it stays finite for every z."""
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of ``silu``: s + z s (1 - s) with s = sigmoid(z)."""
    s = 0.5 * (1.0 + np.tanh(0.5 * z))
    return s * (1.0 + z * (1.0 - s))


# ------------------------------------------------------------------ attention
def doc_starts(cu_seqlens, tokens: int) -> np.ndarray:
    """For every packed token, the index of the first token of its document.

    ``cu_seqlens`` holds the document boundaries [0, n0, n0+n1, ..., T].
    A fixed-length micro-batch of b sequences of length s is the case
    cu_seqlens = [0, s, 2s, ..., bs].
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    starts = np.empty(tokens, dtype=np.int64)
    for a, b in zip(cu[:-1], cu[1:]):
        starts[a:b] = a
    return starts


def _row_blocks(tokens: int, block: int):
    for r0 in range(0, tokens, block):
        yield r0, min(tokens, r0 + block)


def _allowed(starts: np.ndarray, r0: int, r1: int, c0: int, c1: int) -> np.ndarray:
    rows = np.arange(r0, r1)[:, None]
    cols = np.arange(c0, c1)[None, :]
    return (cols <= rows) & (cols >= starts[r0:r1, None])


def attention_probabilities(q, k, heads: int, starts) -> np.ndarray:
    """Full [heads, T, T] probability tensor (small inputs only, for pins)."""
    T, h = q.shape
    d = h // heads
    allowed = _allowed(starts, 0, T, 0, T)
    probs = np.zeros((heads, T, T))
    for n in range(heads):
        sl = slice(n * d, (n + 1) * d)
        s = np.where(allowed, q[:, sl] @ k[:, sl].T / math.sqrt(d), -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        probs[n] = e / e.sum(axis=1, keepdims=True)
    return probs


def attention_forward(q, k, v, heads: int, starts, row_block: int = 512):
    """Masked softmax attention per head, softmax in fp64.

    Scores S = q_n k_n^T / sqrt(d); key j is kept for query i iff
    starts[i] <= j <= i (causal within the document); P = softmax(S) row-wise
    (row maximum subtracted); ctx_n = P v_n.  Also returns the natural-log
    log-sum-exp of every score row, lse[n, i] = log sum_j exp(S_ij).

    Query rows are processed in blocks of ``row_block`` only to bound memory;
    keys outside [min start of the block, last row] carry weight exactly 0 and
    are not materialised.  Softmax in full precision follows the pages'
    attention_softmax_in_fp32 flag (page "Megatron-LM 3D parallelism guide",
    §3.2); the head split follows §2.1 of the same page.
    """
    T, h = q.shape
    d = h // heads
    scale = 1.0 / math.sqrt(d)
    ctx = np.zeros((T, h))
    lse = np.zeros((heads, T))
    for r0, r1 in _row_blocks(T, row_block):
        c0, c1 = int(starts[r0:r1].min()), r1
        allowed = _allowed(starts, r0, r1, c0, c1)
        for n in range(heads):
            sl = slice(n * d, (n + 1) * d)
            s = np.where(allowed, (q[r0:r1, sl] @ k[c0:c1, sl].T) * scale, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            ctx[r0:r1, sl] = (e / l) @ v[c0:c1, sl]
            lse[n, r0:r1] = (m + np.log(l))[:, 0]
    return ctx, lse


def attention_backward(q, k, v, dctx, heads: int, starts, row_block: int = 512):
    """Gradient of ``attention_forward`` w.r.t. q, k, v.

    With P the probabilities and dP = dctx_n v_n^T: dv_n = P^T dctx_n;
    the softmax Jacobian gives dS_i = P_i * (dP_i - <P_i, dP_i>);
    dq_n = dS k_n / sqrt(d), dk_n = dS^T q_n / sqrt(d).
    """
    T, h = q.shape
    d = h // heads
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros((T, h))
    dk = np.zeros((T, h))
    dv = np.zeros((T, h))
    for r0, r1 in _row_blocks(T, row_block):
        c0, c1 = int(starts[r0:r1].min()), r1
        allowed = _allowed(starts, r0, r1, c0, c1)
        for n in range(heads):
            sl = slice(n * d, (n + 1) * d)
            s = np.where(allowed, (q[r0:r1, sl] @ k[c0:c1, sl].T) * scale, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            do = dctx[r0:r1, sl]
            dv[c0:c1, sl] += p.T @ do
            dp = do @ v[c0:c1, sl].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[r0:r1, sl] = (ds @ k[c0:c1, sl]) * scale
            dk[c0:c1, sl] += (ds.T @ q[r0:r1, sl]) * scale
    return dq, dk, dv


# ---------------------------------------------------------------- whole layer
def _params64(params: Dict) -> Dict[str, np.ndarray]:
    return {k: to64(v) for k, v in params.items()
            if k not in ("x", "dy", "targets", "cu_seqlens", "emb")}


def _fwd_product(c, name, x, w, b, fp8: bool):
    """y = x W^T + b, or on FP8 codes (E4M3 x and W, per-tensor scales),
    whose codes are kept in c["fp8"][name] for the backward."""
    if not fp8:
        return linear(x, w, b)
    from . import fp8 as f8
    qx, sx = f8.quantize_per_tensor(x, "e4m3")
    qw, sw = f8.quantize_per_tensor(w, "e4m3")
    c.setdefault("fp8", {})[name] = {"qx": qx, "sx": sx, "qw": qw, "sw": sw}
    return f8.fp8_linear(qx, sx, qw, sw, b)


def layer_forward(params: Dict, x, heads: int, eps: float, starts,
                  fp8: bool = False) -> Dict[str, np.ndarray]:
    """Forward of the unsharded pre-LN layer; returns every intermediate.
    ``fp8``: the four linear maps on FP8 codes (see the module docstring)."""
    p = _params64(params)
    x = to64(x)
    h = x.shape[1]
    c: Dict[str, np.ndarray] = {"x": x}
    c["ln1"], c["mu1"], c["rstd1"] = layernorm(x, p["ln1_g"], p["ln1_b"], eps)
    wqkv = np.concatenate([p["wq"], p["wk"], p["wv"]], axis=0)
    c["qkv"] = _fwd_product(c, "qkv", c["ln1"], wqkv, p["bqkv"], fp8)
    q, k, v = c["qkv"][:, :h], c["qkv"][:, h:2 * h], c["qkv"][:, 2 * h:]
    c["ctx"], c["lse"] = attention_forward(q, k, v, heads, starts)
    c["y1"] = x + _fwd_product(c, "proj", c["ctx"], p["wo"], p["bo"], fp8)
    c["ln2"], c["mu2"], c["rstd2"] = layernorm(c["y1"], p["ln2_g"], p["ln2_b"], eps)
    if "w3" in p and fp8:
        f = p["w1"].shape[0]
        w13 = np.concatenate([p["w1"], p["w3"]], axis=0)
        u13 = _fwd_product(c, "fc1", c["ln2"], w13, None, fp8)
        c["u"], c["u3"] = u13[:, :f], u13[:, f:]
        c["g"] = silu(c["u"]) * c["u3"]
    elif "w3" in p:
        c["u"] = linear(c["ln2"], p["w1"])
        c["u3"] = linear(c["ln2"], p["w3"])
        c["g"] = silu(c["u"]) * c["u3"]
    else:
        c["u"] = _fwd_product(c, "fc1", c["ln2"], p["w1"], p["b1"], fp8)
        c["g"] = gelu_tanh(c["u"])
    c["y"] = c["y1"] + _fwd_product(c, "fc2", c["g"], p["w2"], p["b2"], fp8)
    return c


def _bwd_products(c, gr, name, dy, x, w):
    """(dy W, dy^T x): the data and weight gradients of y = x W^T, or on FP8
    codes: dy in E5M2 (codes kept in gr["fp8"][name]) with the forward's E4M3
    codes of W and x."""
    if "fp8" not in c:
        return dy @ w, dy.T @ x
    from . import fp8 as f8
    fw = c["fp8"][name]
    qd, sd = f8.quantize_per_tensor(dy, "e5m2")
    gr.setdefault("fp8", {})[name] = {"qdy": qd, "sdy": sd}
    return f8.fp8_dgrad(qd, sd, fw["qw"], fw["sw"]), f8.fp8_wgrad(qd, sd, fw["qx"], fw["sx"])


def layer_backward(params: Dict, cache: Dict[str, np.ndarray], dy, heads: int,
                   starts) -> Dict[str, np.ndarray]:
    """Backward of ``layer_forward`` for upstream gradient dy (chain rule);
    FP8 products when the forward ran with ``fp8``."""
    p = _params64(params)
    dy = to64(dy)
    c = cache
    h = dy.shape[1]
    gr: Dict[str, np.ndarray] = {}
    # MLP: y = y1 + g W2^T + b2
    dg, gr["dw2"] = _bwd_products(c, gr, "fc2", dy, c["g"], p["w2"])
    gr["db2"] = dy.sum(axis=0)
    if "w3" in p:
        du = dg * c["u3"] * silu_grad(c["u"])
        du3 = dg * silu(c["u"])
        gr["du"], gr["du3"] = du, du3
        if "fp8" in c:
            f = p["w1"].shape[0]
            w13 = np.concatenate([p["w1"], p["w3"]], axis=0)
            dln2, dw13 = _bwd_products(c, gr, "fc1", np.concatenate([du, du3], axis=1),
                                       c["ln2"], w13)
            gr["dw1"], gr["dw3"] = dw13[:f], dw13[f:]
        else:
            gr["dw1"] = du.T @ c["ln2"]
            gr["dw3"] = du3.T @ c["ln2"]
            dln2 = du @ p["w1"] + du3 @ p["w3"]
    else:
        du = dg * gelu_tanh_grad(c["u"])
        gr["du"] = du
        dln2, gr["dw1"] = _bwd_products(c, gr, "fc1", du, c["ln2"], p["w1"])
        gr["db1"] = du.sum(axis=0)
    gr["dln2"] = dln2
    dy1_ln, gr["dln2_g"], gr["dln2_b"] = layernorm_backward(dln2, c["y1"], p["ln2_g"],
                                                            c["mu2"], c["rstd2"])
    dy1 = dy + dy1_ln
    gr["dy1"] = dy1
    # attention block: y1 = x + ctx Wo^T + bo
    dctx, gr["dwo"] = _bwd_products(c, gr, "proj", dy1, c["ctx"], p["wo"])
    gr["dbo"] = dy1.sum(axis=0)
    gr["dctx"] = dctx
    q, k, v = c["qkv"][:, :h], c["qkv"][:, h:2 * h], c["qkv"][:, 2 * h:]
    dq, dk, dv = attention_backward(q, k, v, dctx, heads, starts)
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    gr["dqkv"] = dqkv
    wqkv = np.concatenate([p["wq"], p["wk"], p["wv"]], axis=0)
    dln1, dwqkv = _bwd_products(c, gr, "qkv", dqkv, c["ln1"], wqkv)
    gr["dwq"], gr["dwk"], gr["dwv"] = dwqkv[:h], dwqkv[h:2 * h], dwqkv[2 * h:]
    gr["dbqkv"] = dqkv.sum(axis=0)
    gr["dln1"] = dln1
    dx_ln, gr["dln1_g"], gr["dln1_b"] = layernorm_backward(dln1, c["x"], p["ln1_g"],
                                                           c["mu1"], c["rstd1"])
    gr["dx"] = dy1 + dx_ln
    return gr


# ------------------------------------------------------- vocab-parallel head
def vocab_ce_forward(y, emb, targets):
    """Logits z = y E^T (E [V, h]); mean token cross-entropy.

    loss = mean_t [ log sum_j exp(z_tj) - z_t,target_t ]  (row max subtracted
    before exp).  The vocabulary split across ranks (VocabParallelEmbedding,
    page "Megatron-LM: NVIDIA's large-model training framework", section
    "Tensor parallelism") changes nothing in this definition.
    Returns (loss, logits, lse[T]).
    """
    y = to64(y)
    emb = to64(emb)
    tg = np.asarray(targets, dtype=np.int64)
    z = y @ emb.T
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    loss = float(np.mean(lse - z[np.arange(z.shape[0]), tg]))
    return loss, z, lse


def vocab_ce_backward(y, emb, targets, logits, lse):
    """dz = (softmax(z) - onehot(target)) / T; dy = dz E; dE = dz^T y."""
    y = to64(y)
    emb = to64(emb)
    tg = np.asarray(targets, dtype=np.int64)
    T = logits.shape[0]
    dz = np.exp(logits - lse[:, None])
    dz[np.arange(T), tg] -= 1.0
    dz /= T
    return dz @ emb, dz.T @ y, dz


# ----------------------------------------------------------------- rank view
def rank_view(fwd: Dict[str, np.ndarray], grads: Optional[Dict[str, np.ndarray]],
              params: Dict, heads: int, tp: int, r: int) -> Dict[str, np.ndarray]:
    """The slices / partials of the unsharded result that rank r computes.

    Column-parallel weights (Wq, Wk, Wv, W1) are split by output rows and
    row-parallel ones (Wo, W2) by input columns (page "Megatron-LM 3D
    parallelism guide", §2.1): rank r owns heads [r*a/t, (r+1)*a/t), hidden
    columns [r*h/t, (r+1)*h/t) and FFN columns [r*f/t, (r+1)*f/t).  Its QKV
    output is packed [q_r | k_r | v_r].  Its row-parallel partial is the
    product of its input slice with its weight slice; the sum over ranks of
    these partials is the unsharded product.
    """
    p = _params64(params)
    h = p["wq"].shape[0]
    f = p["w1"].shape[0]
    hl, fl = h // tp, f // tp
    hc = slice(r * hl, (r + 1) * hl)
    fc = slice(r * fl, (r + 1) * fl)
    qkv_cols = np.r_[r * hl:(r + 1) * hl, h + r * hl:h + (r + 1) * hl,
                     2 * h + r * hl:2 * h + (r + 1) * hl]
    # operands of the partial products: the exact tensors, or with FP8 the
    # dequantized codes (whose scales belong to the whole tensor)
    f8 = fwd.get("fp8")
    g8 = grads.get("fp8") if grads is not None else None

    def opnd(exact, name, key):
        if f8 is None:
            return exact
        src = g8[name] if key == "qdy" else f8[name]
        return src[key] * float(src["sdy" if key == "qdy" else "s" + key[1]])
    wqkv = np.concatenate([p["wq"], p["wk"], p["wv"]], axis=0)
    v: Dict[str, np.ndarray] = {}
    v["qkv"] = fwd["qkv"][:, qkv_cols]
    v["ctx"] = fwd["ctx"][:, hc]
    v["lse"] = fwd["lse"][r * (heads // tp):(r + 1) * (heads // tp)]
    v["proj_partial"] = opnd(fwd["ctx"], "proj", "qx")[:, hc] @ opnd(p["wo"], "proj", "qw")[:, hc].T
    v["u"] = fwd["u"][:, fc]
    if "u3" in fwd:
        v["u3"] = fwd["u3"][:, fc]
    v["g"] = fwd["g"][:, fc]
    v["fc2_partial"] = opnd(fwd["g"], "fc2", "qx")[:, fc] @ opnd(p["w2"], "fc2", "qw")[:, fc].T
    if grads is not None:
        wqkv_r = opnd(wqkv, "qkv", "qw")[qkv_cols]
        v["du"] = grads["du"][:, fc]
        v["dw2"] = grads["dw2"][:, fc]
        v["dw1"] = grads["dw1"][fc]
        if "w3" in p:
            v["du3"] = grads["du3"][:, fc]
            v["dw3"] = grads["dw3"][fc]
            # the rank's gate and up rows of the one FFN input map [W1; W3]
            du13 = np.concatenate([grads["du"], grads["du3"]], axis=1)
            w13 = np.concatenate([p["w1"], p["w3"]], axis=0)
            rows = np.r_[r * fl:(r + 1) * fl, f + r * fl:f + (r + 1) * fl]
            v["fc1_dx_partial"] = (opnd(du13, "fc1", "qdy")[:, rows]
                                   @ opnd(w13, "fc1", "qw")[rows])
        else:
            v["fc1_dx_partial"] = (opnd(grads["du"], "fc1", "qdy")[:, fc]
                                   @ opnd(p["w1"], "fc1", "qw")[fc])
            v["db1"] = grads["db1"][fc]
        v["dctx"] = grads["dctx"][:, hc]
        v["dwo"] = grads["dwo"][:, hc]
        v["dqkv"] = grads["dqkv"][:, qkv_cols]
        v["dwqkv"] = np.concatenate([grads["dwq"][hc], grads["dwk"][hc], grads["dwv"][hc]], axis=0)
        v["dbqkv"] = grads["dbqkv"][qkv_cols]
        v["qkv_dx_partial"] = opnd(grads["dqkv"], "qkv", "qdy")[:, qkv_cols] @ wqkv_r
    return v
