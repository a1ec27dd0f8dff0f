"""FP8 (E4M3, per-tensor scale) quantization and forward linear maps on the
GPU against the fp64 oracle: the codes and scales bit for bit, the GEMMs
element-wise on sampled output rows at the 7B-style shard shapes."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from gpu_common import TOL, check, log, require_gpu

pytestmark = pytest.mark.gpu


def _bf16(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * std).to(torch.bfloat16)


def _quant_gpu(d, x):
    from tensor_transformer_layer_04_amd import mtp
    xc = x.cuda().contiguous()
    q = torch.empty(x.numel(), dtype=torch.uint8, device="cuda")
    s = torch.empty(2, dtype=torch.float32, device="cuda")
    mtp.mtp_quantize_fp8(d, xc, x.numel(), q, s)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("shape,std", [((2048, 4096), 1.0), ((6144, 4096), 0.02),
                                       ((1000, 24), 3.0), ((8, 16), 1e-3)])
def test_quantize_codes_bit_exact(shape, std):
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    d = mtp.make_desc(4096, 32, 11008, 2, 0, 2048, 1, mtp.MTP_BF16)
    x = _bf16(shape, 40 + shape[0], std)
    q, s = _quant_gpu(d, x)
    qo, so = ofp8.quantize_per_tensor(x.float().numpy())
    codes = ofp8.e4m3_encode(qo).reshape(-1)
    got = q.cpu().numpy()
    log(f"quantize {shape}: scale gpu {float(s[0])!r} oracle {float(so)!r}, "
        f"{int((got != codes).sum())} codes differ")
    assert float(s[0]) == float(so) and float(s[1]) == float(np.max(np.abs(x.float().numpy())))
    assert np.array_equal(got, codes)


def test_quantize_zero_tensor():
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    d = mtp.make_desc(256, 2, 512, 1, 0, 8, 1, mtp.MTP_BF16)
    q, s = _quant_gpu(d, torch.zeros(8, 256, dtype=torch.bfloat16))
    assert float(s[0]) == 1.0 and float(s[1]) == 0.0 and int(q.cpu().sum()) == 0


@pytest.mark.parametrize("T", [2048, 2000])
def test_fp8_linear_maps_7b_shard(T):
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    h, a, f, tp = 4096, 32, 11008, 2
    hl, fl = h // tp, f // tp
    d = mtp.make_desc(h, a, f, tp, 0, T, 1, mtp.MTP_BF16)
    tol = TOL["bf16"]
    rows = np.unique(np.concatenate([np.sort(np.random.default_rng(T).choice(T, 40, replace=False)),
                                     [0, T - 1]]))
    cases = {  # kind: (x shape, w shape, bias)
        "qkv": (mtp.MTP_QKV, (T, h), (3 * hl, h), True),
        "fc1": (mtp.MTP_FC1, (T, h), (fl, h), True),
        "proj": (mtp.MTP_PROJ, (T, hl), (h, hl), False),
        "fc2": (mtp.MTP_FC2, (T, fl), (h, fl), False),
    }
    report = {}
    for i, (name, (kind, xs, ws, has_b)) in enumerate(cases.items()):
        x, w = _bf16(xs, 60 + i), _bf16(ws, 70 + i, 0.02)
        b = _bf16((ws[0],), 80 + i, 0.1) if has_b else None
        qx, sx = _quant_gpu(d, x)
        qw, sw = _quant_gpu(d, w)
        y = torch.empty(T, ws[0], dtype=torch.bfloat16, device="cuda")
        u = torch.empty_like(y) if kind == mtp.MTP_FC1 else None
        mtp.mtp_linear_fwd_fp8(d, kind, qx, sx, qw, sw, None if b is None else b.cuda(), y, u)
        torch.cuda.synchronize()
        q_x, s_x = ofp8.quantize_per_tensor(x.float().numpy())
        q_w, s_w = ofp8.quantize_per_tensor(w.float().numpy())
        ref = ofp8.fp8_linear(q_x[rows], s_x, q_w, s_w, None if b is None else oracle.to64(b))
        if kind == mtp.MTP_FC1:
            check(f"{name}.u", u[rows].float().cpu(), ref, tol, report)
            ref = oracle.gelu_tanh(ref)
        check(f"{name}.y", y[rows].float().cpu(), ref, tol, report)
    log(f"fp8 linear T={T}: " + ", ".join(f"{k}={v:.2e}" for k, v in report.items()))


# ------------------------------------------------------------ FP8 step
def _amax_and_quant(d, fmt, shards):
    """GPU codes of a tensor given as its column shards (each [rows, c_i]):
    each shard's amax parts, then every shard's codes with all parts."""
    from tensor_transformer_layer_04_amd import mtp
    parts, out = [], []
    for x in shards:
        p = torch.empty(mtp.FP8_AMAX_PARTS, dtype=torch.float32, device="cuda")
        mtp.mtp_fp8_amax(d, x, x.numel(), p)
        parts.append(p)
    for x in shards:
        rows, cols = x.shape
        q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
        qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
        s = torch.empty(1, dtype=torch.float32, device="cuda")
        mtp.mtp_fp8_quantize(d, fmt, x, rows, cols, parts, q, qt, s)
        out.append((q, qt, s))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols,n_shards,std", [(300, 200, 2, 1.0), (2048, 5504, 1, 1e-4),
                                                    (77, 64, 3, 5.0), (0, 16, 1, 1.0)])
def test_fp8_quantize_shards_both_layouts(fmt, rows, cols, n_shards, std):
    """Codes of a tensor split into column shards, each scaled by the whole
    tensor's amax: row-major and transposed codes bit for bit against the
    oracle's quantization of the whole tensor, and the scale exactly."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    d = mtp.make_desc(4096, 32, 11008, 2, 0, 2048, 1, mtp.MTP_BF16)
    x = _bf16((rows, cols * n_shards), 90 + rows + cols, std)
    if rows:
        x[rows // 2, 3] = 7.0 * std   # one clear maximum, away from the first shard's edge
    shards = [x[:, i * cols:(i + 1) * cols].contiguous().cuda() for i in range(n_shards)]
    got = _amax_and_quant(d, mtp.MTP_FP8_E4M3 if fmt == "e4m3" else mtp.MTP_FP8_E5M2, shards)
    qo, so = ofp8.quantize_per_tensor(x.float().numpy(), fmt)
    codes = ofp8.fp8_encode(qo, fmt).reshape(rows, cols * n_shards)
    for i, (q, qt, s) in enumerate(got):
        ref = codes[:, i * cols:(i + 1) * cols]
        assert float(s[0]) == float(so), (float(s[0]), float(so))
        assert np.array_equal(q.cpu().numpy(), ref), f"shard {i}: row-major codes differ"
        assert np.array_equal(qt.cpu().numpy(), ref.T), f"shard {i}: transposed codes differ"


def _bf16_values_upto(amax):
    """Every bf16 value x with |x| <= amax (amax a positive bf16 value), both
    signs, as fp32."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[v <= np.float32(amax)]
    return np.concatenate([v, -v])


# amax per format: plain and all-ones / one-bit significands, the formats'
# maxima, tiny and huge tensors, and the two bf16 values around the scale
# 2^-60 where the convert kernel changes from multiplying by 1/s to dividing.
FP8_AMAX_SWEEP = {
    "e4m3": [1.0, 3.140625, 1.9921875, 1.0078125, 448.0, 57344.0, 9984.0, 0.0302734375, 2.0 ** -20,
             2.0 ** -100, 3.3895313892515355e38, 1.75 * 2.0 ** -52, 1.7421875 * 2.0 ** -52],
    "e5m2": [1.0, 3.140625, 1.9921875, 1.0078125, 448.0, 57344.0, 9984.0, 0.0302734375, 2.0 ** -20,
             2.0 ** -100, 3.3895313892515355e38, 1.75 * 2.0 ** -45, 1.7421875 * 2.0 ** -45],
}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_codes_of_every_bf16_value(fmt):
    """For each amax of the sweep, the tensor of every bf16 value up to it
    (both signs; 255 rows, a ragged count for the 128-row tiles and for the
    16-byte transposed stores): row-major and transposed codes and the
    scale bit for bit against the oracle."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    d = mtp.make_desc(4096, 32, 11008, 2, 0, 2048, 1, mtp.MTP_BF16)
    code = mtp.MTP_FP8_E4M3 if fmt == "e4m3" else mtp.MTP_FP8_E5M2
    cols = 256
    for amax in FP8_AMAX_SWEEP[fmt]:
        v = _bf16_values_upto(amax)
        x = np.zeros(((v.size + cols - 1) // cols) * cols, np.float32)
        x[:v.size] = v
        x = x.reshape(-1, cols)
        xt = torch.from_numpy(x).to(torch.bfloat16)
        assert torch.equal(xt.float(), torch.from_numpy(x)), "sweep values must be bf16"
        (q, qt, s), = _amax_and_quant(d, code, [xt.cuda()])
        qo, so = ofp8.quantize_per_tensor(x, fmt)
        ref = ofp8.fp8_encode(qo, fmt).reshape(x.shape)
        got, got_t = q.cpu().numpy(), qt.cpu().numpy()
        bad = np.argwhere(got != ref)
        log(f"{fmt} amax {amax!r}: {x.shape[0]} rows, scale {float(s[0])!r} / {float(so)!r}, "
            f"{len(bad)} codes differ" + (f"; first x={x[tuple(bad[0])]!r} got {got[tuple(bad[0])]:#04x} "
                                          f"want {ref[tuple(bad[0])]:#04x}" if len(bad) else ""))
        assert float(s[0]) == float(so)
        assert len(bad) == 0
        assert np.array_equal(got_t, ref.T)


# h, T, n: the fused paths (LayerNorm grid within the 1024 parts, one-pass
# sum + LayerNorm, fused backward), a LayerNorm grid of 1025 workgroups, and
# widths that take the separate kernels (then the parts come from a pass of
# their own over the output).
AMAX_LN_CASES = [(4096, 2048, 2), (4096, 4100, 2), (768, 77, 2), (12288, 9, 4), (512, 5, 1)]


@pytest.mark.parametrize("h,T,n", AMAX_LN_CASES)
def test_amax_parts_from_layernorm_kernels(h, T, n):
    """The amax parts that the LayerNorm forward, the partial sum + LayerNorm
    and the LayerNorm backward of summed partials write beside their bf16
    output: the maximum over the 1024 parts is the largest |value| stored,
    every slot is written (the buffer starts at 1e30), the codes and scale
    made from them equal those made from a separate amax pass bit for bit,
    and the outputs equal those of the calls without parts."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    d = mtp.make_desc(h, h // 64, 4 * h, 1, 0, T, 1, mtp.MTP_BF16)
    g = torch.Generator().manual_seed(700 + h + T)
    R = lambda *sh, std=1.0: (torch.randn(*sh, generator=g) * std).to(torch.bfloat16).cuda()
    x, res = R(T, h), R(T, h)
    parts = [R(T, h) for _ in range(n)]
    dys = [R(T, h, std=0.01) for _ in range(n)]
    gm, bt, bias = (1 + R(h, std=0.1).float()).to(torch.bfloat16), R(h, std=0.1), R(h, std=0.1)
    x[T // 2, 7] = 40.0   # a row whose LayerNorm output has one clear maximum
    E = lambda: torch.empty(T, h, dtype=torch.bfloat16, device="cuda")
    F = lambda k=T: torch.empty(k, dtype=torch.float32, device="cuda")
    P = lambda: torch.full((mtp.FP8_AMAX_PARTS,), 1e30, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(mtp.mtp_workspace_size(d, mtp.MTP_OP_LAYERNORM_BWD), 256),
                     dtype=torch.uint8, device="cuda")

    def outputs():
        """(name, output, parts) of the three producers with amax parts, and
        the same outputs of the calls without them."""
        res_ = []
        y0, y1, mu, rs = E(), E(), F(), F()
        mtp.mtp_layernorm(d, x, gm, bt, y0, mu, rs)
        p = P()
        mtp.mtp_layernorm(d, x, gm, bt, y1, mu, rs, amax_parts=p)
        res_.append(("layernorm", y1, y0, p))
        o0, o1, l0, l1 = E(), E(), E(), E()
        mtp.mtp_partial_sum_layernorm(d, parts, bias, res, o0, gm, bt, l0, mu, rs)
        p = P()
        mtp.mtp_partial_sum_layernorm(d, parts, bias, res, o1, gm, bt, l1, mu, rs, amax_parts=p)
        assert torch.equal(o0, o1)
        res_.append(("sum_layernorm", l1, l0, p))
        dx0, dx1, dg, db = E(), E(), F(h), F(h)
        mtp.mtp_layernorm_bwd_sum(d, dys, o0, gm, mu, rs, res, dx0, dg, db, 0, ws, ws.numel())
        p = P()
        mtp.mtp_layernorm_bwd_sum(d, dys, o0, gm, mu, rs, res, dx1, dg, db, 0, ws, ws.numel(),
                                  amax_parts=p)
        res_.append(("layernorm_bwd_sum", dx1, dx0, p))
        return res_

    for name, y, y_plain, p in outputs():
        assert torch.equal(y, y_plain), f"{name}: output changed by writing amax parts"
        ref = torch.empty(mtp.FP8_AMAX_PARTS, dtype=torch.float32, device="cuda")
        mtp.mtp_fp8_amax(d, y, y.numel(), ref)
        torch.cuda.synchronize()
        want = float(y.float().abs().max())
        log(f"amax parts {name} h={h} T={T}: fused {float(p.max())!r} separate "
            f"{float(ref.max())!r} max|y| {want!r}")
        assert float(p.max()) == want == float(ref.max())
        assert float(p.min()) >= 0.0
        for fmt in (mtp.MTP_FP8_E4M3, mtp.MTP_FP8_E5M2):
            codes = []
            for pp in (p, ref):
                q = torch.empty(T, h, dtype=torch.uint8, device="cuda")
                s = torch.empty(1, dtype=torch.float32, device="cuda")
                mtp.mtp_fp8_quantize(d, fmt, y, T, h, [pp], q, None, s)
                codes.append((q, s))
            torch.cuda.synchronize()
            assert torch.equal(codes[0][0], codes[1][0]) and torch.equal(codes[0][1], codes[1][1])


@pytest.mark.parametrize("T", [2048, 304])
def test_fp8_backward_gemms_7b_shard(T):
    """Data and weight gradients of the four linear maps from FP8 codes (E5M2
    gradient, the forward's E4M3 codes of W and x) at the 7B TP=2 shard
    shapes, against the oracle's FP8 products of the same codes: every
    element of the weight gradients, sampled rows of the data gradients."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    h, a, f, tp = 4096, 32, 11008, 2
    hl, fl = h // tp, f // tp
    d = mtp.make_desc(h, a, f, tp, 0, T, 1, mtp.MTP_BF16)
    tol = TOL["bf16"]
    rows = np.unique(np.concatenate([np.random.default_rng(T).choice(T, 24, replace=False),
                                     [0, T - 1]]))
    cases = {  # name: (kind, out, in)
        "qkv": (mtp.MTP_QKV, 3 * hl, h), "fc1": (mtp.MTP_FC1, fl, h),
        "proj": (mtp.MTP_PROJ, h, hl), "fc2": (mtp.MTP_FC2, h, fl)}
    report = {}
    for i, (name, (kind, out, inn)) in enumerate(cases.items()):
        dy = _bf16((T, out), 110 + i, 1e-3)
        w = _bf16((out, inn), 120 + i, 0.02)
        x = _bf16((T, inn), 130 + i)
        (dq, dqt, ds), = _amax_and_quant(d, mtp.MTP_FP8_E5M2, [dy.cuda()])
        (wq, wqt, wsc), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [w.cuda()])
        (xq, xqt, xs), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [x.cuda()])
        u = _bf16((T, inn), 140 + i) if kind == mtp.MTP_FC2 else None
        dx = torch.empty(T, inn, dtype=torch.bfloat16, device="cuda")
        dw = torch.empty(out, inn, dtype=torch.float32, device="cuda")
        mtp.mtp_linear_bwd_fp8(d, kind, dq, dqt, ds, wqt, wsc, xqt, xs,
                               None if u is None else u.cuda(), dx, dw)
        dw2 = torch.zeros(out, inn, dtype=torch.float32, device="cuda") + 1.0
        mtp.mtp_linear_bwd_fp8(d, kind, None, dqt, ds, None, None, xqt, xs, None, None, dw2, 1)
        torch.cuda.synchronize()
        q_dy, s_dy = ofp8.quantize_per_tensor(dy.float().numpy(), "e5m2")
        q_w, s_w = ofp8.quantize_per_tensor(w.float().numpy(), "e4m3")
        q_x, s_x = ofp8.quantize_per_tensor(x.float().numpy(), "e4m3")
        ref_dx = ofp8.fp8_dgrad(q_dy[rows], s_dy, q_w, s_w)
        if u is not None:
            ref_dx = ref_dx * oracle.gelu_tanh_grad(oracle.to64(u)[rows])
        ref_dw = ofp8.fp8_wgrad(q_dy, s_dy, q_x, s_x)
        check(f"{name}.dx", dx[rows].float().cpu(), ref_dx, tol, report)
        check(f"{name}.dw", dw.cpu(), ref_dw, 1e-4, report)
        check(f"{name}.dw_acc", dw2.cpu(), ref_dw + 1.0, 1e-4, report)
    log(f"fp8 backward GEMMs T={T}: " + ", ".join(f"{k}={v:.2e}" for k, v in report.items()))


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("T", [2048, 304, 16384])
def test_amax_parts_from_fp8_gemm_epilogues(T, act):
    """The FC1 forward (GeLU output g, or SiLU(gate) * up of the interleaved
    gate|up product) and the FC2 data gradient (du with the GeLU derivative,
    or the interleaved gate and up gradients) write the amax parts of their
    bf16 output when asked: the outputs are those of the calls without
    parts, the largest part is the largest |value| stored, every slot is
    written, and the codes made from the parts equal those of a separate
    amax pass bit for bit.  T = 16384 gives the FC1 GEMM more tiles than
    parts (the pass over the output then writes them)."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    h, a, f, tp = 4096, 32, 11008, 2
    fl = f // tp
    sw = act == "swiglu"
    ul = 2 * fl if sw else fl    # width of the FC1 product and of its gradient
    k_fc1, k_fc2 = ((mtp.MTP_FC1_SWIGLU, mtp.MTP_FC2_SWIGLU) if sw else
                    (mtp.MTP_FC1, mtp.MTP_FC2))
    d = mtp.make_desc(h, a, f, tp, 0, T, 1, mtp.MTP_BF16)
    x, w1 = _bf16((T, h), 150), _bf16((ul, h), 151, 0.02)
    b1 = None if sw else _bf16((fl,), 152, 0.1).cuda()
    dy, w2, u = _bf16((T, h), 153, 1e-3), _bf16((h, fl), 154, 0.02), _bf16((T, ul), 155)
    (xq, _, xs), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [x.cuda()])
    (w1q, _, w1s), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [w1.cuda()])
    (dq, _, ds), = _amax_and_quant(d, mtp.MTP_FP8_E5M2, [dy.cuda()])
    (_, w2qt, w2s), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [w2.cuda()])
    u = u.cuda()
    P = lambda: torch.full((mtp.FP8_AMAX_PARTS,), 1e30, dtype=torch.float32, device="cuda")
    E = lambda c: torch.empty(T, c, dtype=torch.bfloat16, device="cuda")
    g0, g1, u0, u1, p_g = E(fl), E(fl), E(ul), E(ul), P()
    mtp.mtp_linear_fwd_fp8(d, k_fc1, xq, xs, w1q, w1s, b1, g0, u0)
    mtp.mtp_linear_fwd_fp8(d, k_fc1, xq, xs, w1q, w1s, b1, g1, u1, amax_parts=p_g)
    du0, du1, p_du = E(ul), E(ul), P()
    mtp.mtp_linear_bwd_fp8(d, k_fc2, dq, None, ds, w2qt, w2s, None, None, u, du0, None)
    mtp.mtp_linear_bwd_fp8(d, k_fc2, dq, None, ds, w2qt, w2s, None, None, u, du1, None,
                           dx_amax_parts=p_du)
    torch.cuda.synchronize()
    assert torch.equal(g0, g1) and torch.equal(u0, u1) and torch.equal(du0, du1)
    for name, y, p, fmt in (("g", g1, p_g, mtp.MTP_FP8_E4M3), ("du", du1, p_du, mtp.MTP_FP8_E5M2)):
        cols = y.shape[1]
        ref = torch.empty(mtp.FP8_AMAX_PARTS, dtype=torch.float32, device="cuda")
        mtp.mtp_fp8_amax(d, y, y.numel(), ref)
        torch.cuda.synchronize()
        want = float(y.float().abs().max())
        log(f"fp8 GEMM amax parts {act} {name} T={T}: fused {float(p.max())!r} separate "
            f"{float(ref.max())!r} max|y| {want!r}")
        assert float(p.max()) == want == float(ref.max()) and float(p.min()) >= 0.0
        codes = []
        for pp in (p, ref):
            q = torch.empty(T, cols, dtype=torch.uint8, device="cuda")
            qt = torch.empty(cols, T, dtype=torch.uint8, device="cuda")
            s = torch.empty(1, dtype=torch.float32, device="cuda")
            mtp.mtp_fp8_quantize(d, fmt, y, T, cols, [pp], q, qt, s)
            codes.append((q, qt, s))
        torch.cuda.synchronize()
        assert all(torch.equal(a_, b_) for a_, b_ in zip(*codes))


def _gate_up(z):
    """(gate, up) halves of columns interleaved in groups of 4."""
    r = z.shape[0]
    v = z.reshape(r, -1, 2, 4)
    return v[:, :, 0].reshape(r, -1), v[:, :, 1].reshape(r, -1)


def _interleave(gate, up):
    r = gate.shape[0]
    return np.stack([gate.reshape(r, -1, 4), up.reshape(r, -1, 4)], 2).reshape(r, -1)


@pytest.mark.parametrize("T", [2048, 304])
def test_fp8_swiglu_maps_7b_shard(T):
    """The SwiGLU FFN on FP8 codes at the 7B TP=2 shard shapes (f_l = 5504;
    gate and up rows interleaved in groups of 4 under one scale), against
    the oracle's FP8 products of the same codes: the forward's interleaved
    pre-activation and SiLU(gate) * up, the FC2 data gradient's interleaved
    gate and up gradients (sampled rows), and the FC1 data gradient (sampled
    rows) and weight gradient (every element) over the interleaved width."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    h, a, f, tp = 4096, 32, 11008, 2
    fl = f // tp
    d = mtp.make_desc(h, a, f, tp, 0, T, 1, mtp.MTP_BF16)
    tol = TOL["bf16"]
    rows = np.unique(np.concatenate([np.random.default_rng(T + 7).choice(T, 24, replace=False),
                                     [0, T - 1]]))
    report = {}
    x, w13 = _bf16((T, h), 170), _bf16((2 * fl, h), 171, 0.02)
    dy, w2 = _bf16((T, h), 172, 1e-3), _bf16((h, fl), 173, 0.02)
    (xq, xqt, xs), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [x.cuda()])
    (wq, wqt, wsc), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [w13.cuda()])
    (dq, _, ds), = _amax_and_quant(d, mtp.MTP_FP8_E5M2, [dy.cuda()])
    (_, w2qt, w2s), = _amax_and_quant(d, mtp.MTP_FP8_E4M3, [w2.cuda()])
    u = torch.empty(T, 2 * fl, dtype=torch.bfloat16, device="cuda")
    g = torch.empty(T, fl, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_linear_fwd_fp8(d, mtp.MTP_FC1_SWIGLU, xq, xs, wq, wsc, None, g, u)
    du = torch.empty(T, 2 * fl, dtype=torch.bfloat16, device="cuda")
    mtp.mtp_linear_bwd_fp8(d, mtp.MTP_FC2_SWIGLU, dq, None, ds, w2qt, w2s, None, None, u, du,
                           None)
    torch.cuda.synchronize()
    q_x, s_x = ofp8.quantize_per_tensor(x.float().numpy(), "e4m3")
    q_w, s_w = ofp8.quantize_per_tensor(w13.float().numpy(), "e4m3")
    q_dy, s_dy = ofp8.quantize_per_tensor(dy.float().numpy(), "e5m2")
    q_w2, s_w2 = ofp8.quantize_per_tensor(w2.float().numpy(), "e4m3")
    uref = ofp8.fp8_linear(q_x[rows], s_x, q_w, s_w)
    check("fc1_swiglu.u", u[rows].float().cpu(), uref, tol, report)
    gt, up = _gate_up(uref)
    check("fc1_swiglu.g", g[rows].float().cpu(), oracle.silu(gt) * up, tol, report)
    # the derivative at the pre-activation the GPU stored (bf16)
    gt, up = _gate_up(oracle.to64(u[rows].cpu()))
    dg = ofp8.fp8_dgrad(q_dy[rows], s_dy, q_w2, s_w2)
    ref_du = _interleave(dg * up * oracle.silu_grad(gt), dg * oracle.silu(gt))
    check("fc2_swiglu.du", du[rows].float().cpu(), ref_du, tol, report)
    # FC1 backward over the interleaved width, from the codes of du
    (dq13, dqt13, ds13), = _amax_and_quant(d, mtp.MTP_FP8_E5M2, [du])
    dx = torch.empty(T, h, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(2 * fl, h, dtype=torch.float32, device="cuda")
    mtp.mtp_linear_bwd_fp8(d, mtp.MTP_FC1_SWIGLU, dq13, dqt13, ds13, wqt, wsc, xqt, xs, None, dx,
                           dw)
    torch.cuda.synchronize()
    q_du, s_du = ofp8.quantize_per_tensor(du.float().cpu().numpy(), "e5m2")
    check("fc1_swiglu.dx", dx[rows].float().cpu(), ofp8.fp8_dgrad(q_du[rows], s_du, q_w, s_w), tol,
          report)
    check("fc1_swiglu.dw", dw.cpu(), ofp8.fp8_wgrad(q_du, s_du, q_x, s_x), 1e-4, report)
    log(f"fp8 SwiGLU maps T={T}: " + ", ".join(f"{k}={v:.2e}" for k, v in report.items()))


@pytest.mark.parametrize("T,docs", [(2048, None), (304, None), (8192, None), (2048, [0, 700, 1500, 2048])])
def test_amax_parts_from_attention(T, docs):
    """The attention forward (ctx) and backward (dqkv) write the amax parts
    of their bf16 output when asked: outputs equal those of the calls
    without parts, the largest part is the largest |value| stored, every slot
    is written, and the codes made from the parts equal those of a separate
    amax pass bit for bit.  7B TP=2 shard heads (16 of d = 128); T = 8192
    gives the forward more workgroups than parts (the pass over ctx then
    writes them); the backward's 3 x 32 x 16 workgroups at T = 2048 share
    the 1024 slots; one case packs three documents."""
    require_gpu()
    from tensor_transformer_layer_04_amd import mtp
    h, a, f, tp = 4096, 32, 11008, 2
    hl, al = h // tp, a // tp
    d = mtp.make_desc(h, a, f, tp, 0, T, 1, mtp.MTP_BF16)
    qkv = (_bf16((T, 3 * hl), 160 + T) * 2).cuda()
    dctx = _bf16((T, hl), 161 + T, 0.05).cuda()
    cu = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    n = 0 if docs is None else len(docs) - 1
    P = lambda: torch.full((mtp.FP8_AMAX_PARTS,), 1e30, dtype=torch.float32, device="cuda")
    ctx0, ctx1 = (torch.empty(T, hl, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    lse0, lse1 = (torch.empty(al, T, dtype=torch.float32, device="cuda") for _ in range(2))
    p_ctx, p_dqkv = P(), P()
    mtp.mtp_attn_fwd(d, qkv, ctx0, lse0, cu, n)
    mtp.mtp_attn_fwd(d, qkv, ctx1, lse1, cu, n, ctx_amax_parts=p_ctx)
    wsb = mtp.mtp_workspace_size(d, mtp.MTP_OP_ATTN_BWD)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    g0, g1 = (torch.empty(T, 3 * hl, dtype=torch.bfloat16, device="cuda") for _ in range(2))
    mtp.mtp_attn_bwd(d, qkv, ctx0, lse0, dctx, g0, cu, n, ws, wsb)
    mtp.mtp_attn_bwd(d, qkv, ctx0, lse0, dctx, g1, cu, n, ws, wsb, dqkv_amax_parts=p_dqkv)
    torch.cuda.synchronize()
    assert torch.equal(ctx0, ctx1) and torch.equal(lse0, lse1) and torch.equal(g0, g1)
    for name, y, p, fmt in (("ctx", ctx1, p_ctx, mtp.MTP_FP8_E4M3),
                            ("dqkv", g1, p_dqkv, mtp.MTP_FP8_E5M2)):
        ref = torch.empty(mtp.FP8_AMAX_PARTS, dtype=torch.float32, device="cuda")
        mtp.mtp_fp8_amax(d, y, y.numel(), ref)
        torch.cuda.synchronize()
        want = float(y.float().abs().max())
        log(f"attention amax parts {name} T={T} docs={docs}: fused {float(p.max())!r} separate "
            f"{float(ref.max())!r} max|y| {want!r}")
        assert float(p.max()) == want == float(ref.max()) and float(p.min()) >= 0.0
        rows, cols = y.shape
        codes = []
        for pp in (p, ref):
            q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
            qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
            s = torch.empty(1, dtype=torch.float32, device="cuda")
            mtp.mtp_fp8_quantize(d, fmt, y, rows, cols, [pp], q, qt, s)
            codes.append((q, qt, s))
        torch.cuda.synchronize()
        assert all(torch.equal(a_, b_) for a_, b_ in zip(*codes))
