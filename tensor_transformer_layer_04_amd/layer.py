"""Tensor-parallel pre-LN transformer layer shards on one GPU.

``TPLayer`` sequences the libmtp calls for one or more rank shards of a
Megatron-style layer (page "Megatron-LM 3D parallelism guide", §2.1: the
Q/K/V and FC1 weights split by output columns, the output projection and
FC2 by input rows, per-rank partials summed).  All ranks' shards run one
after another on the same device and ``mtp_partial_sum`` stands in for the
tensor-parallel all-reduce.  Torch provides device memory and the stream;
every step of the layer runs in libmtp's kernels.

Forward (per step):
    ln1 = LN(x)                                   (replicated, computed once)
    per rank r: qkv_r = ln1 Wqkv_r^T + bqkv_r;  ctx_r, lse_r = attn(qkv_r)
                p_r = ctx_r Wo_r^T                (partial)
    y1 = sum_r p_r + bo + x
    ln2 = LN(y1)
    per rank r: u_r = ln2 W1_r^T + b1_r; g_r = GeLU(u_r); q_r = g_r W2_r^T
    y = sum_r q_r + b2 + y1
Backward mirrors it; the input gradient of each column-parallel map is the
sum of the ranks' partials (the input reached every rank).

Ranks that are not computed in this process can contribute their partials
through ``external`` buffers (e.g. precomputed by an earlier run), which is
how one rank's shard is timed with the full t-way sums charged to it.

Sequence parallelism (``cfg.sequence_parallel``; page "Megatron-LM: NVIDIA
large-model training framework", section "Sequence parallelism"): the
per-token work (LayerNorm, residual, bias, dropout) is split over the tokens
instead of replicated, rank r owning rows [r T/t, (r+1) T/t).  The sum of
the row-parallel partials becomes a reduce-scatter (rank r sums only its
rows), followed by an all-gather of the LayerNorm output before the next
column-parallel GEMM; in backward the column-dgrad partials are
reduce-scattered into the LayerNorm backward of each rank's rows and the
result all-gathered.  On one device the ranks' row blocks live in one
[T, h] buffer, so the all-gather moves nothing: a rank writes its rows and
the GEMMs read the whole buffer.  LayerNorm weight gradients and the
row-parallel bias gradients are each rank's column sums over its rows,
added over the computed ranks in rank order.

FP8 (``cfg.fp8``; the FP8 precision of page "Megatron-LM / Megatron Core
README digest", §0): the twelve GEMMs of the step run on FP8 codes with one
scale per tensor, E4M3 for the activations and weights the forward reads and
E5M2 for the gradients the backward reads, each GEMM's operands k-major (the
backward reads the transposed codes the quantization writes beside the
row-major ones).  A tensor split over the ranks (a weight shard, ctx_r, g_r,
du_r, dqkv_r) is scaled by the maximum over every rank's amax, as the ranks
of a tensor-parallel group would agree on it; the step therefore runs phase
by phase over the ranks (all ranks' amax, then their codes), and ranks not
computed here contribute their amax parts through ``external``.  With the
SwiGLU FFN the gate and up rows of W1|W3 are one tensor under one scale, and
so are their output gradients [du | du3], both in the interleaved order the
bf16 step uses.  With context-parallel attention, ctx and dqkv come out of
the chunks' block pairs and merges and take the amax pass.  With sequence
parallelism, ln1, ln2 and dy1 are written rank by rank on their row blocks;
each block's kernel writes amax parts of its own and the whole tensor is
scaled by the maximum over all blocks' parts (the other ranks' through
``external``).
"""
from __future__ import annotations

import bisect
import contextlib
from typing import Dict, List, Optional, Sequence

import torch

from . import mtp


def cp_block_pairs(chunks, cu_host=None):
    """The context-parallel block pairs (query chunk j, key chunk i < j) with
    work in them, in ring order (i = j-1, ..., 0) for each j.  ``chunks`` are
    consecutive (lo, hi) token ranges; ``cu_host`` the packed documents'
    offsets (None: one sequence from token 0, every pair has work).  A query sees only
    its own document's keys, and the earliest document start among a
    chunk's queries is that of its first token, so chunk i's keys are
    visible to some query of chunk j iff that start lies before the end of
    chunk i; the other pairs are not launched."""
    out = []
    for j, (q0, _) in enumerate(chunks):
        start = 0 if cu_host is None else cu_host[bisect.bisect_right(cu_host, q0) - 1]
        out += [(j, i) for i in range(j - 1, -1, -1) if start < chunks[i][1]]
    return out


def desc_for(cfg, rank: int) -> mtp.mtp_shard_desc:
    """The C descriptor of rank ``rank`` for a workload config."""
    T = cfg.tokens
    seq_len, mb = (T, 1) if cfg.varlen_tokens else (cfg.seq_len, cfg.micro_batch)
    return mtp.make_desc(cfg.hidden, cfg.heads, cfg.ffn, cfg.tp, rank, seq_len, mb,
                         mtp.MTP_F32 if cfg.dtype == "f32" else mtp.MTP_BF16,
                         vocab=cfg.vocab, ln_eps=cfg.eps)


def pack_rank_weights(full: Dict[str, torch.Tensor], cfg, rank: int,
                      device="cuda") -> Dict[str, torch.Tensor]:
    """Slice the unsharded weights into rank ``rank``'s shard.

    Column-parallel maps keep the rank's output rows (Wqkv_r stacks the
    rank's rows of Wq, Wk and Wv, so its output is [q_r | k_r | v_r]);
    row-parallel maps keep the rank's input columns.  Replicated tensors
    (LayerNorm affine, row-parallel biases) are copied as they are.
    """
    h, f, t = cfg.hidden, cfg.ffn, cfg.tp
    hl, fl = h // t, f // t
    hs = slice(rank * hl, (rank + 1) * hl)
    fs = slice(rank * fl, (rank + 1) * fl)

    def dev(x):
        return x.to(device).contiguous()
    w = {
        "wqkv": dev(torch.cat([full["wq"][hs], full["wk"][hs], full["wv"][hs]], 0)),
        "bqkv": dev(torch.cat([full["bqkv"][:h][hs], full["bqkv"][h:2 * h][hs],
                               full["bqkv"][2 * h:][hs]], 0)),
        "wo": dev(full["wo"][:, hs]),
        "w2": dev(full["w2"][:, fs]),
    }
    if getattr(cfg, "swiglu", False):
        # gate rows (W1) and up rows (W3) interleaved in groups of 4, the
        # layout MTP_FC1_SWIGLU takes
        w["w1"] = dev(swiglu_interleave(full["w1"][fs], full["w3"][fs]))
    else:
        w["w1"] = dev(full["w1"][fs])
        w["b1"] = dev(full["b1"][fs])
    if cfg.vocab:
        vl = cfg.vocab // t
        w["emb"] = dev(full["emb"][rank * vl:(rank + 1) * vl])
    return w


def swiglu_interleave(gate: torch.Tensor, up: torch.Tensor) -> torch.Tensor:
    """Rows (or, for a [T, f] activation, columns via .T) of gate and up
    interleaved in groups of 4: [g0..g3, u0..u3, g4..g7, u4..u7, ...]."""
    f = gate.shape[0]
    return torch.stack([gate.reshape(f // 4, 4, *gate.shape[1:]),
                        up.reshape(f // 4, 4, *up.shape[1:])], 1).reshape(2 * f, *gate.shape[1:])


def swiglu_split(x: torch.Tensor, dim: int = 0):
    """Inverse of ``swiglu_interleave`` along ``dim``: (gate, up)."""
    x = x.movedim(dim, 0)
    f2 = x.shape[0]
    v = x.reshape(f2 // 8, 2, 4, *x.shape[1:])
    gate = v[:, 0].reshape(f2 // 2, *x.shape[1:]).movedim(0, dim)
    up = v[:, 1].reshape(f2 // 2, *x.shape[1:]).movedim(0, dim)
    return gate, up


def replicated_params(full: Dict[str, torch.Tensor], device="cuda") -> Dict[str, torch.Tensor]:
    return {k: full[k].to(device).contiguous() for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "bo", "b2")}


class _Probed:
    """Optional timing probe: ``probe`` = {tag: [(start_event, end_event), ...]}
    for the tags present as keys; events are recorded on the given stream
    (default: the current one)."""

    probe: Optional[Dict[str, list]] = None
    device: torch.device

    @contextlib.contextmanager
    def _timed(self, tag: str, stream=None):
        pr = self.probe
        if pr is None or tag not in pr:
            yield
            return
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        yield
        b.record(st)
        pr[tag].append((a, b))


class TPLayer(_Probed):
    """One pre-LN layer, ``ranks`` of its ``cfg.tp`` shards computed here."""

    def __init__(self, cfg, full: Dict[str, torch.Tensor], ranks: Optional[Sequence[int]] = None,
                 device="cuda", cu_seqlens: Optional[torch.Tensor] = None, overlap: bool = True):
        self.cfg = cfg
        self.device = torch.device(device)
        self.ranks = list(range(cfg.tp)) if ranks is None else list(ranks)
        self.dt = cfg.torch_dtype
        self.T = cfg.tokens
        self.descs = {r: desc_for(cfg, r) for r in range(cfg.tp)}
        self.d0 = self.descs[self.ranks[0]]
        self.w = {r: pack_rank_weights(full, cfg, r, device) for r in self.ranks}
        self.rep = replicated_params(full, device)
        self.cu = None
        self.cu_host = None
        self.n_seqs = 0
        if cu_seqlens is not None and cfg.varlen_tokens:
            self.cu_host = [int(v) for v in cu_seqlens.cpu().tolist()]
            self.cu = cu_seqlens.to(device=self.device, dtype=torch.int32).contiguous()
            self.n_seqs = self.cu.numel() - 1
        # Weight and bias gradients are off the backward's critical path: with
        # ``overlap`` they run on a second stream (default priority) next to
        # the data gradients, joined back before backward() returns.
        self.side = torch.cuda.Stream(device=self.device) if overlap else None
        self.swiglu = bool(getattr(cfg, "swiglu", False))
        self.k_fc1 = mtp.MTP_FC1_SWIGLU if self.swiglu else mtp.MTP_FC1
        self.k_fc2 = mtp.MTP_FC2_SWIGLU if self.swiglu else mtp.MTP_FC2
        # Context parallelism: the attention of each rank's heads runs over
        # cp chunks of the token stream, block pair by block pair (the keys of
        # a chunk and of every earlier chunk), the partials merged through
        # their log-sum-exp; bf16, one sequence or packed documents.
        self.cp = int(getattr(cfg, "context_parallel", 1))
        if self.cp > 1:
            if cfg.dtype != "bf16" or cfg.micro_batch != 1:
                raise ValueError("context parallelism needs a bf16 shard with micro_batch 1")
            if self.T % self.cp:
                raise ValueError(f"context parallelism needs T ({self.T}) divisible by {self.cp}")
        self.sp = bool(getattr(cfg, "sequence_parallel", False)) and cfg.tp > 1
        if self.sp:
            # Each rank's row block must start on a 16-byte boundary of the
            # fp32 per-token statistics (the C ABI takes 16-byte aligned
            # pointers): T / tp a multiple of 4.
            if self.T % (4 * cfg.tp):
                raise ValueError(f"sequence parallelism needs T ({self.T}) divisible by "
                                 f"4 * tp ({4 * cfg.tp})")
            tr = self.T // cfg.tp
            self.rows = {r: slice(r * tr, (r + 1) * tr) for r in range(cfg.tp)}
            self.rdesc = {r: mtp.make_desc(cfg.hidden, cfg.heads, cfg.ffn, cfg.tp, r, tr, 1,
                                           mtp.MTP_F32 if cfg.dtype == "f32" else mtp.MTP_BF16,
                                           vocab=cfg.vocab, ln_eps=cfg.eps)
                          for r in range(cfg.tp)}
        self.fp8 = bool(getattr(cfg, "fp8", False))
        if self.fp8:
            if cfg.dtype != "bf16":
                raise ValueError("the FP8 step needs a bf16 layer")
            if self.T % 16:
                raise ValueError(f"the FP8 step needs T ({self.T}) divisible by 16")
        self._alloc()
        if self.fp8:
            self._alloc_fp8()

    # ------------------------------------------------------------ buffers
    def _alloc(self):
        cfg, T, dt, dev = self.cfg, self.T, self.dt, self.device
        h, t = cfg.hidden, cfg.tp
        hl, al, fl = h // t, cfg.heads // t, cfg.ffn // t
        E = lambda *s, d=dt: torch.empty(*s, dtype=d, device=dev)
        self.ln1, self.y1, self.ln2, self.y = E(T, h), E(T, h), E(T, h), E(T, h)
        self.mu1, self.rs1, self.mu2, self.rs2 = (E(T, d=torch.float32) for _ in range(4))
        self.a: Dict[int, Dict[str, torch.Tensor]] = {}
        # SwiGLU: the FC1 output (and its gradient) is the interleaved gate|up pair
        ul = 2 * fl if self.swiglu else fl
        for r in self.ranks:
            self.a[r] = {
                "qkv": E(T, 3 * hl), "ctx": E(T, hl), "lse": E(al, T, d=torch.float32),
                "p": E(T, h), "u": E(T, ul), "g": E(T, fl), "q": E(T, h),
                # backward
                "du": E(T, ul), "dln2": E(T, h), "dctx": E(T, hl), "dqkv": E(T, 3 * hl),
                "dln1": E(T, h),
            }
            if self.cp > 1:  # one partial attention result (ctx, lse) to merge
                self.a[r]["ctx_p"] = E(T, hl)
                self.a[r]["lse_p"] = E(al, T, d=torch.float32)
        self.dy1, self.dx = E(T, h), E(T, h)
        f32 = torch.float32
        self.grads: Dict[int, Dict[str, torch.Tensor]] = {}
        for r in self.ranks:
            self.grads[r] = {
                "dwqkv": E(3 * hl, h, d=f32), "dbqkv": E(3 * hl, d=f32), "dwo": E(h, hl, d=f32),
                "dw1": E(ul, h, d=f32), "dw2": E(h, fl, d=f32),
            }
            if not self.swiglu:
                self.grads[r]["db1"] = E(fl, d=f32)
        self.rgrads = {k: E(h, d=f32) for k in ("dln1_g", "dln1_b", "dln2_g", "dln2_b", "dbo", "db2")}
        d = self.d0
        ws = max(
            mtp.mtp_workspace_size(d, mtp.MTP_OP_LAYERNORM_BWD),
            mtp.mtp_workspace_size(d, mtp.MTP_OP_COL_LINEAR_BWD, mtp.MTP_QKV),
            mtp.mtp_workspace_size(d, mtp.MTP_OP_COL_LINEAR_BWD, mtp.MTP_FC1),
            mtp.mtp_workspace_size(d, mtp.MTP_OP_ROW_LINEAR_BWD, mtp.MTP_PROJ),
            mtp.mtp_workspace_size(d, mtp.MTP_OP_ATTN_BWD),
            256)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.ws_bytes = ws
        # the side stream gets a workspace of its own
        self.ws_side = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.owns_bias = self.ranks[0]  # rank whose call produces row-parallel bias grads
        self.probe = None

    def _alloc_fp8(self):
        """Codes (row-major q and transposed qt, uint8), scale and amax parts
        of every tensor the FP8 GEMMs read."""
        cfg, T, dev = self.cfg, self.T, self.device
        h, t = cfg.hidden, cfg.tp
        hl, fl = h // t, cfg.ffn // t
        # SwiGLU: gate and up rows (and their output gradients) are one
        # tensor under one scale, in the interleaved order of the bf16 step
        ul = 2 * fl if self.swiglu else fl

        def slot(rows, cols):
            return {"q": torch.empty(rows, cols, dtype=torch.uint8, device=dev),
                    "qt": torch.empty(cols, rows, dtype=torch.uint8, device=dev),
                    "s": torch.empty(4, dtype=torch.float32, device=dev),
                    "amax": torch.zeros(mtp.FP8_AMAX_PARTS, dtype=torch.float32, device=dev),
                    "rows": rows, "cols": cols}
        # replicated inputs (one quantization serves every rank)
        self.q8 = {k: slot(T, h) for k in ("ln1", "ln2", "dy", "dy1")}
        shapes = {"ctx": (T, hl), "g": (T, fl), "du": (T, ul), "dqkv": (T, 3 * hl),
                  "wqkv": (3 * hl, h), "wo": (h, hl), "w1": (ul, h), "w2": (h, fl)}
        self.r8 = {r: {k: slot(*sh) for k, sh in shapes.items()} for r in self.ranks}
        # sequence parallelism: ln1, ln2 and dy1 are written rank by rank on
        # their row blocks, each block with amax parts of its own
        if self.sp:
            self.p8 = {k: {r: torch.zeros(mtp.FP8_AMAX_PARTS, dtype=torch.float32, device=dev)
                           for r in self.ranks} for k in ("ln1", "ln2", "dy1")}

    def _quant_shared(self, name, x, fmt, amax_written=False):
        """amax and codes of a tensor every rank holds whole (amax_written:
        the kernel that produced x already wrote its amax parts)."""
        sl = self.q8[name]
        if not amax_written:
            mtp.mtp_fp8_amax(self.d0, x, x.numel(), sl["amax"])
        mtp.mtp_fp8_quantize(self.d0, fmt, x, sl["rows"], sl["cols"], [sl["amax"]], sl["q"],
                             sl["qt"], sl["s"])

    def _quant_rows(self, name, x, fmt, ext):
        """Codes of a tensor that every rank holds whole but whose row blocks
        the ranks produced (sequence parallelism), scaled by the maximum over
        the blocks' amax parts (this layer's ranks and ``ext``'s)."""
        sl = self.q8[name]
        parts = [self.p8[name][r] for r in self.ranks] + list(ext.get("fp8_" + name, []))
        mtp.mtp_fp8_quantize(self.d0, fmt, x, sl["rows"], sl["cols"], parts, sl["q"], sl["qt"],
                             sl["s"])

    def _quant_split(self, name, xs, fmt, ext, amax_written=False):
        """amax of every computed rank's shard xs[r], then its codes with the
        scale of the whole tensor (this layer's ranks and ``ext``'s;
        amax_written: the kernels that produced the shards wrote their amax
        parts)."""
        if not amax_written:
            for r in self.ranks:
                mtp.mtp_fp8_amax(self.descs[r], xs[r], xs[r].numel(), self.r8[r][name]["amax"])
        parts = [self.r8[r][name]["amax"] for r in self.ranks] + list(ext.get("fp8_" + name, []))
        for r in self.ranks:
            sl = self.r8[r][name]
            mtp.mtp_fp8_quantize(self.descs[r], fmt, xs[r], sl["rows"], sl["cols"], parts, sl["q"],
                                 sl["qt"], sl["s"])

    def adopt_rows(self, other: "TPLayer"):
        """Sequence parallelism: share ``other``'s token-sharded buffers, whose
        row blocks of the ranks not computed here stay resident (the
        all-gathered activations and gradients of those ranks)."""
        for k in ("ln1", "mu1", "rs1", "y1", "ln2", "mu2", "rs2", "y", "dy1", "dx"):
            setattr(self, k, getattr(other, k))

    # ------------------------------------------------------------ forward
    def forward(self, x: torch.Tensor, external: Optional[Dict[str, List[torch.Tensor]]] = None):
        """Forward of the computed ranks; returns y (valid when every rank's
        partials are available, computed or external)."""
        ext = external or {}
        if self.fp8:
            return self._forward_fp8(x, ext)
        d0, rep = self.d0, self.rep
        self.x = x
        T = self._timed
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("ln1"):
                    mtp.mtp_layernorm(self.rdesc[r], x[s], rep["ln1_g"], rep["ln1_b"],
                                      self.ln1[s], self.mu1[s], self.rs1[s])
        else:
            with T("ln1"):
                mtp.mtp_layernorm(d0, x, rep["ln1_g"], rep["ln1_b"], self.ln1, self.mu1, self.rs1)
        for r in self.ranks:
            d, w, a = self.descs[r], self.w[r], self.a[r]
            with T("qkv_fwd"):
                mtp.mtp_col_linear_fwd(d, mtp.MTP_QKV, self.ln1, w["wqkv"], w["bqkv"], a["qkv"],
                                       None)
            with T("attn_fwd"):
                if self.cp > 1:
                    self._attn_fwd_cp(d, a)
                else:
                    mtp.mtp_attn_fwd(d, a["qkv"], a["ctx"], a["lse"], self.cu, self.n_seqs)
            with T("proj_fwd"):
                mtp.mtp_row_linear_fwd(d, mtp.MTP_PROJ, a["ctx"], w["wo"], a["p"])
        parts = [self.a[r]["p"] for r in self.ranks] + list(ext.get("proj", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("sum_proj_ln2"):
                    mtp.mtp_partial_sum_layernorm(self.rdesc[r], [q[s] for q in parts], rep["bo"],
                                                  x[s], self.y1[s], rep["ln2_g"], rep["ln2_b"],
                                                  self.ln2[s], self.mu2[s], self.rs2[s])
        else:
            with T("sum_proj_ln2"):
                mtp.mtp_partial_sum_layernorm(d0, parts, rep["bo"], x, self.y1, rep["ln2_g"],
                                              rep["ln2_b"], self.ln2, self.mu2, self.rs2)
        for r in self.ranks:
            d, w, a = self.descs[r], self.w[r], self.a[r]
            with T("fc1_fwd"):
                mtp.mtp_col_linear_fwd(d, self.k_fc1, self.ln2, w["w1"], w.get("b1"), a["g"],
                                       a["u"])
            with T("fc2_fwd"):
                mtp.mtp_row_linear_fwd(d, self.k_fc2, a["g"], w["w2"], a["q"])
        parts = [self.a[r]["q"] for r in self.ranks] + list(ext.get("fc2", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("sum_fc2"):
                    mtp.mtp_partial_sum(self.rdesc[r], [q[s] for q in parts], rep["b2"],
                                        self.y1[s], self.y[s])
        else:
            with T("sum_fc2"):
                mtp.mtp_partial_sum(d0, parts, rep["b2"], self.y1, self.y)
        return self.y

    # ----------------------------------------------------------- backward
    def backward(self, dy: torch.Tensor, external: Optional[Dict[str, List[torch.Tensor]]] = None):
        ext = external or {}
        if self.fp8:
            return self._backward_fp8(dy, ext)
        d0, rep, ws, wsb = self.d0, self.rep, self.ws, self.ws_bytes
        T = self._timed
        main = torch.cuda.current_stream(self.device)
        side = self.side
        wss = self.ws_side if side is not None else ws

        def fork():
            """Point the side stream past everything issued on main so far."""
            if side is not None:
                side.wait_stream(main)

        def on_side():
            return torch.cuda.stream(side) if side is not None else contextlib.nullcontext()

        # Each linear map's backward is issued as two calls: the data gradient
        # on the main stream and the weight + bias gradients on the side one.
        fork()
        for r in self.ranks:
            d, w, a, g = self.descs[r], self.w[r], self.a[r], self.grads[r]
            db2 = self.rgrads["db2"] if (r == self.owns_bias and not self.sp) else None
            with T("fc2_dgrad"):
                mtp.mtp_row_linear_bwd(d, self.k_fc2, dy, a["g"], w["w2"], a["u"], a["du"], None,
                                       None, 0, ws, wsb)
            with on_side(), T("fc2_wgrad", side):
                mtp.mtp_row_linear_bwd(d, self.k_fc2, dy, a["g"], w["w2"], None, None, g["dw2"],
                                       db2, 0, wss, wsb)
            if self.sp:
                # row-parallel bias: this rank's column sums of dy over its rows
                s = self.rows[r]
                with on_side(), T("fc2_bias", side):
                    mtp.mtp_row_linear_bwd(self.rdesc[r], self.k_fc2, dy[s], a["g"][s], w["w2"],
                                           None, None, None, self.rgrads["db2"],
                                           int(r != self.ranks[0]), wss, wsb)
            # FC1's weight gradient needs only du: it is queued as soon as
            # du exists, beside FC1's data gradient.
            fork()
            with on_side(), T("fc1_wgrad", side):
                mtp.mtp_col_linear_bwd(d, self.k_fc1, a["du"], self.ln2, w["w1"], None, g["dw1"],
                                       g.get("db1"), 0, wss, wsb)
            with T("fc1_dgrad"):
                mtp.mtp_col_linear_bwd(d, self.k_fc1, a["du"], self.ln2, w["w1"], a["dln2"], None,
                                       None, 0, ws, wsb)
        parts = [self.a[r]["dln2"] for r in self.ranks] + list(ext.get("fc1_dx", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("ln2_bwd"):
                    mtp.mtp_layernorm_bwd_sum(self.rdesc[r], [q[s] for q in parts], self.y1[s],
                                              rep["ln2_g"], self.mu2[s], self.rs2[s], dy[s],
                                              self.dy1[s], self.rgrads["dln2_g"],
                                              self.rgrads["dln2_b"], int(r != self.ranks[0]), ws,
                                              wsb)
        else:
            with T("ln2_bwd"):
                mtp.mtp_layernorm_bwd_sum(d0, parts, self.y1, rep["ln2_g"], self.mu2, self.rs2, dy,
                                          self.dy1, self.rgrads["dln2_g"], self.rgrads["dln2_b"], 0,
                                          ws, wsb)
        fork()
        for r in self.ranks:
            d, w, a, g = self.descs[r], self.w[r], self.a[r], self.grads[r]
            dbo = self.rgrads["dbo"] if (r == self.owns_bias and not self.sp) else None
            with T("proj_dgrad"):
                mtp.mtp_row_linear_bwd(d, mtp.MTP_PROJ, self.dy1, a["ctx"], w["wo"], None,
                                       a["dctx"], None, None, 0, ws, wsb)
            with on_side(), T("proj_wgrad", side):
                mtp.mtp_row_linear_bwd(d, mtp.MTP_PROJ, self.dy1, a["ctx"], w["wo"], None, None,
                                       g["dwo"], dbo, 0, wss, wsb)
            if self.sp:
                s = self.rows[r]
                with on_side(), T("proj_bias", side):
                    mtp.mtp_row_linear_bwd(self.rdesc[r], mtp.MTP_PROJ, self.dy1[s], a["ctx"][s],
                                           w["wo"], None, None, None, self.rgrads["dbo"],
                                           int(r != self.ranks[0]), wss, wsb)
            with T("attn_bwd"):
                if self.cp > 1:
                    self._attn_bwd_cp(d, a, ws, wsb)
                else:
                    mtp.mtp_attn_bwd(d, a["qkv"], a["ctx"], a["lse"], a["dctx"], a["dqkv"],
                                     self.cu, self.n_seqs, ws, wsb)
            with T("qkv_dgrad"):
                mtp.mtp_col_linear_bwd(d, mtp.MTP_QKV, a["dqkv"], self.ln1, w["wqkv"], a["dln1"],
                                       None, None, 0, ws, wsb)
            fork()
            with on_side(), T("qkv_wgrad", side):
                mtp.mtp_col_linear_bwd(d, mtp.MTP_QKV, a["dqkv"], self.ln1, w["wqkv"], None,
                                       g["dwqkv"], None, 0, wss, wsb)
        parts = [self.a[r]["dln1"] for r in self.ranks] + list(ext.get("qkv_dx", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("ln1_bwd"):
                    mtp.mtp_layernorm_bwd_sum(self.rdesc[r], [q[s] for q in parts], self.x[s],
                                              rep["ln1_g"], self.mu1[s], self.rs1[s], self.dy1[s],
                                              self.dx[s], self.rgrads["dln1_g"],
                                              self.rgrads["dln1_b"], int(r != self.ranks[0]), ws,
                                              wsb)
        else:
            with T("ln1_bwd"):
                mtp.mtp_layernorm_bwd_sum(d0, parts, self.x, rep["ln1_g"], self.mu1, self.rs1,
                                          self.dy1, self.dx, self.rgrads["dln1_g"],
                                          self.rgrads["dln1_b"], 0, ws, wsb)
        self._qkv_bias_grad()
        if side is not None:
            main.wait_stream(side)
        return self.dx

    def _qkv_bias_grad(self):
        """QKV bias gradients (column sums of dqkv) on the main stream after the
        LN1 backward: there they run beside the QKV weight gradient, the last
        kernel of the second stream, instead of after it at the end of the
        step."""
        for r in self.ranks:
            with self._timed("qkv_bias"):
                mtp.mtp_col_linear_bwd(self.descs[r], mtp.MTP_QKV, self.a[r]["dqkv"], self.ln1,
                                       self.w[r]["wqkv"], None, None, self.grads[r]["dbqkv"], 0,
                                       self.ws, self.ws_bytes)

    # ------------------------------------------------------------- FP8 step
    def _forward_fp8(self, x, ext):
        d0, rep, T = self.d0, self.rep, self._timed
        E4, q8, r8 = mtp.MTP_FP8_E4M3, self.q8, self.r8
        self.x = x
        # The weights' codes (made once per optimizer update; with gradient
        # accumulation they serve every micro-batch until the next one), on
        # the second stream, which has no other work in the forward, beside
        # LN1 and its codes; each GEMM waits for its weight's codes only.
        side = self.side
        ready = {}
        if side is not None:
            side.wait_stream(torch.cuda.current_stream(self.device))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("ln1"):
                    mtp.mtp_layernorm(self.rdesc[r], x[s], rep["ln1_g"], rep["ln1_b"], self.ln1[s],
                                      self.mu1[s], self.rs1[s], amax_parts=self.p8["ln1"][r])
        else:
            with T("ln1"):
                mtp.mtp_layernorm(d0, x, rep["ln1_g"], rep["ln1_b"], self.ln1, self.mu1, self.rs1,
                                  amax_parts=q8["ln1"]["amax"])
        for name in ("wqkv", "wo", "w1", "w2"):
            with (torch.cuda.stream(side) if side is not None else contextlib.nullcontext()), \
                    T("quant_w", side):
                self._quant_split(name, {r: self.w[r][name] for r in self.ranks}, E4, ext)
            if side is not None:
                ready[name] = torch.cuda.Event()
                ready[name].record(side)

        def wait_w(name):
            if name in ready:
                torch.cuda.current_stream(self.device).wait_event(ready[name])
        with T("quant"):
            if self.sp:
                self._quant_rows("ln1", self.ln1, E4, ext)
            else:
                self._quant_shared("ln1", self.ln1, E4, amax_written=True)
        wait_w("wqkv")
        for r in self.ranks:
            d, w, a, c = self.descs[r], self.w[r], self.a[r], r8[r]
            with T("qkv_fwd"):
                mtp.mtp_linear_fwd_fp8(d, mtp.MTP_QKV, q8["ln1"]["q"], q8["ln1"]["s"],
                                       c["wqkv"]["q"], c["wqkv"]["s"], w["bqkv"], a["qkv"], None)
        for r in self.ranks:
            a = self.a[r]
            with T("attn_fwd"):
                if self.cp > 1:
                    # the chunks' block pairs and merges: ctx's amax in a pass of its own
                    self._attn_fwd_cp(self.descs[r], a)
                else:
                    mtp.mtp_attn_fwd(self.descs[r], a["qkv"], a["ctx"], a["lse"], self.cu,
                                     self.n_seqs, ctx_amax_parts=r8[r]["ctx"]["amax"])
        with T("quant"):
            self._quant_split("ctx", {r: self.a[r]["ctx"] for r in self.ranks}, E4, ext,
                              amax_written=self.cp == 1)
        wait_w("wo")
        for r in self.ranks:
            c = r8[r]
            with T("proj_fwd"):
                mtp.mtp_linear_fwd_fp8(self.descs[r], mtp.MTP_PROJ, c["ctx"]["q"], c["ctx"]["s"],
                                       c["wo"]["q"], c["wo"]["s"], None, self.a[r]["p"], None)
        parts = [self.a[r]["p"] for r in self.ranks] + list(ext.get("proj", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("sum_proj_ln2"):
                    mtp.mtp_partial_sum_layernorm(self.rdesc[r], [q[s] for q in parts], rep["bo"],
                                                  x[s], self.y1[s], rep["ln2_g"], rep["ln2_b"],
                                                  self.ln2[s], self.mu2[s], self.rs2[s],
                                                  amax_parts=self.p8["ln2"][r])
            with T("quant"):
                self._quant_rows("ln2", self.ln2, E4, ext)
        else:
            with T("sum_proj_ln2"):
                mtp.mtp_partial_sum_layernorm(d0, parts, rep["bo"], x, self.y1, rep["ln2_g"],
                                              rep["ln2_b"], self.ln2, self.mu2, self.rs2,
                                              amax_parts=q8["ln2"]["amax"])
            with T("quant"):
                self._quant_shared("ln2", self.ln2, E4, amax_written=True)
        wait_w("w1")
        for r in self.ranks:
            w, a, c = self.w[r], self.a[r], r8[r]
            with T("fc1_fwd"):
                mtp.mtp_linear_fwd_fp8(self.descs[r], self.k_fc1, q8["ln2"]["q"], q8["ln2"]["s"],
                                       c["w1"]["q"], c["w1"]["s"], w.get("b1"), a["g"], a["u"],
                                       amax_parts=c["g"]["amax"])
        with T("quant"):
            self._quant_split("g", {r: self.a[r]["g"] for r in self.ranks}, E4, ext,
                              amax_written=True)
        wait_w("w2")
        for r in self.ranks:
            c = r8[r]
            with T("fc2_fwd"):
                mtp.mtp_linear_fwd_fp8(self.descs[r], self.k_fc2, c["g"]["q"], c["g"]["s"],
                                       c["w2"]["q"], c["w2"]["s"], None, self.a[r]["q"], None)
        parts = [self.a[r]["q"] for r in self.ranks] + list(ext.get("fc2", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("sum_fc2"):
                    mtp.mtp_partial_sum(self.rdesc[r], [q[s] for q in parts], rep["b2"],
                                        self.y1[s], self.y[s])
        else:
            with T("sum_fc2"):
                mtp.mtp_partial_sum(d0, parts, rep["b2"], self.y1, self.y)
        return self.y

    def _backward_fp8(self, dy, ext):
        d0, rep, ws, wsb = self.d0, self.rep, self.ws, self.ws_bytes
        T = self._timed
        E5, q8, r8 = mtp.MTP_FP8_E5M2, self.q8, self.r8
        main = torch.cuda.current_stream(self.device)
        side = self.side
        wss = self.ws_side if side is not None else ws

        def fork():
            if side is not None:
                side.wait_stream(main)

        def on_side():
            return torch.cuda.stream(side) if side is not None else contextlib.nullcontext()

        self.dy_seen = dy
        # FC2: du = (dy W2) * GeLU'(u) (SwiGLU: the interleaved gate and up
        # gradients); dW2 = dy^T g
        with T("quant"):
            self._quant_shared("dy", dy, E5)
        fork()
        for r in self.ranks:
            d, w, a, g, c = self.descs[r], self.w[r], self.a[r], self.grads[r], r8[r]
            with T("fc2_dgrad"):
                mtp.mtp_linear_bwd_fp8(d, self.k_fc2, q8["dy"]["q"], None, q8["dy"]["s"],
                                       c["w2"]["qt"], c["w2"]["s"], None, None, a["u"], a["du"],
                                       None, dx_amax_parts=c["du"]["amax"])
            with on_side(), T("fc2_wgrad", side):
                mtp.mtp_linear_bwd_fp8(d, self.k_fc2, None, q8["dy"]["qt"], q8["dy"]["s"], None,
                                       None, c["g"]["qt"], c["g"]["s"], None, None, g["dw2"])
            if self.sp:
                # row-parallel bias: this rank's column sums of dy over its rows
                s = self.rows[r]
                with on_side(), T("fc2_bias", side):
                    mtp.mtp_row_linear_bwd(self.rdesc[r], mtp.MTP_FC2, dy[s], a["g"][s], w["w2"],
                                           None, None, None, self.rgrads["db2"],
                                           int(r != self.ranks[0]), wss, wsb)
            elif r == self.owns_bias:
                with on_side(), T("fc2_bias", side):
                    mtp.mtp_row_linear_bwd(d, mtp.MTP_FC2, dy, a["g"], w["w2"], None, None, None,
                                           self.rgrads["db2"], 0, wss, wsb)
        # FC1: dln2_r = du_r W1_r; dW1 = du^T ln2
        with T("quant"):
            self._quant_split("du", {r: self.a[r]["du"] for r in self.ranks}, E5, ext,
                              amax_written=True)
        fork()
        for r in self.ranks:
            d, w, a, g, c = self.descs[r], self.w[r], self.a[r], self.grads[r], r8[r]
            with on_side(), T("fc1_wgrad", side):
                mtp.mtp_linear_bwd_fp8(d, self.k_fc1, None, c["du"]["qt"], c["du"]["s"], None,
                                       None, q8["ln2"]["qt"], q8["ln2"]["s"], None, None, g["dw1"])
                if not self.swiglu:
                    mtp.mtp_col_linear_bwd(d, mtp.MTP_FC1, a["du"], self.ln2, w["w1"], None, None,
                                           g["db1"], 0, wss, wsb)
            with T("fc1_dgrad"):
                mtp.mtp_linear_bwd_fp8(d, self.k_fc1, c["du"]["q"], None, c["du"]["s"],
                                       c["w1"]["qt"], c["w1"]["s"], None, None, None, a["dln2"],
                                       None)
        parts = [self.a[r]["dln2"] for r in self.ranks] + list(ext.get("fc1_dx", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("ln2_bwd"):
                    mtp.mtp_layernorm_bwd_sum(self.rdesc[r], [q[s] for q in parts], self.y1[s],
                                              rep["ln2_g"], self.mu2[s], self.rs2[s], dy[s],
                                              self.dy1[s], self.rgrads["dln2_g"],
                                              self.rgrads["dln2_b"], int(r != self.ranks[0]), ws,
                                              wsb, amax_parts=self.p8["dy1"][r])
        else:
            with T("ln2_bwd"):
                mtp.mtp_layernorm_bwd_sum(d0, parts, self.y1, rep["ln2_g"], self.mu2, self.rs2,
                                          dy, self.dy1, self.rgrads["dln2_g"],
                                          self.rgrads["dln2_b"], 0, ws, wsb,
                                          amax_parts=q8["dy1"]["amax"])
        # PROJ: dctx_r = dy1 Wo_r; dWo_r = dy1^T ctx_r; then attention
        with T("quant"):
            if self.sp:
                self._quant_rows("dy1", self.dy1, E5, ext)
            else:
                self._quant_shared("dy1", self.dy1, E5, amax_written=True)
        fork()
        for r in self.ranks:
            d, w, a, g, c = self.descs[r], self.w[r], self.a[r], self.grads[r], r8[r]
            with T("proj_dgrad"):
                mtp.mtp_linear_bwd_fp8(d, mtp.MTP_PROJ, q8["dy1"]["q"], None, q8["dy1"]["s"],
                                       c["wo"]["qt"], c["wo"]["s"], None, None, None, a["dctx"],
                                       None)
            with on_side(), T("proj_wgrad", side):
                mtp.mtp_linear_bwd_fp8(d, mtp.MTP_PROJ, None, q8["dy1"]["qt"], q8["dy1"]["s"],
                                       None, None, c["ctx"]["qt"], c["ctx"]["s"], None, None,
                                       g["dwo"])
                if self.sp:
                    s = self.rows[r]
                    mtp.mtp_row_linear_bwd(self.rdesc[r], mtp.MTP_PROJ, self.dy1[s], a["ctx"][s],
                                           w["wo"], None, None, None, self.rgrads["dbo"],
                                           int(r != self.ranks[0]), wss, wsb)
                elif r == self.owns_bias:
                    mtp.mtp_row_linear_bwd(d, mtp.MTP_PROJ, self.dy1, a["ctx"], w["wo"], None,
                                           None, None, self.rgrads["dbo"], 0, wss, wsb)
            with T("attn_bwd"):
                if self.cp > 1:
                    self._attn_bwd_cp(d, a, ws, wsb)
                else:
                    mtp.mtp_attn_bwd(d, a["qkv"], a["ctx"], a["lse"], a["dctx"], a["dqkv"],
                                     self.cu, self.n_seqs, ws, wsb,
                                     dqkv_amax_parts=c["dqkv"]["amax"])
        # QKV: dln1_r = dqkv_r Wqkv_r; dWqkv_r = dqkv_r^T ln1
        with T("quant"):
            self._quant_split("dqkv", {r: self.a[r]["dqkv"] for r in self.ranks}, E5, ext,
                              amax_written=self.cp == 1)
        fork()
        for r in self.ranks:
            d, w, a, g, c = self.descs[r], self.w[r], self.a[r], self.grads[r], r8[r]
            with T("qkv_dgrad"):
                mtp.mtp_linear_bwd_fp8(d, mtp.MTP_QKV, c["dqkv"]["q"], None, c["dqkv"]["s"],
                                       c["wqkv"]["qt"], c["wqkv"]["s"], None, None, None,
                                       a["dln1"], None)
            with on_side(), T("qkv_wgrad", side):
                mtp.mtp_linear_bwd_fp8(d, mtp.MTP_QKV, None, c["dqkv"]["qt"], c["dqkv"]["s"],
                                       None, None, q8["ln1"]["qt"], q8["ln1"]["s"], None, None,
                                       g["dwqkv"])
        parts = [self.a[r]["dln1"] for r in self.ranks] + list(ext.get("qkv_dx", []))
        if self.sp:
            for r in self.ranks:
                s = self.rows[r]
                with T("ln1_bwd"):
                    mtp.mtp_layernorm_bwd_sum(self.rdesc[r], [q[s] for q in parts], self.x[s],
                                              rep["ln1_g"], self.mu1[s], self.rs1[s], self.dy1[s],
                                              self.dx[s], self.rgrads["dln1_g"],
                                              self.rgrads["dln1_b"], int(r != self.ranks[0]), ws,
                                              wsb)
        else:
            with T("ln1_bwd"):
                mtp.mtp_layernorm_bwd_sum(d0, parts, self.x, rep["ln1_g"], self.mu1, self.rs1,
                                          self.dy1, self.dx, self.rgrads["dln1_g"],
                                          self.rgrads["dln1_b"], 0, ws, wsb)
        self._qkv_bias_grad()
        if side is not None:
            main.wait_stream(side)
        return self.dx

    # ------------------------------------------------ context parallelism
    def _chunks(self):
        L = self.T // self.cp
        return [(c * L, (c + 1) * L) for c in range(self.cp)]

    def cp_pairs(self):
        return cp_block_pairs(self._chunks(), self.cu_host)

    def _attn_fwd_cp(self, d, a):
        """Chunk j (a context-parallel rank) attends to its own keys (the
        diagonal block), then, ring step by ring step, to the keys of the
        earlier chunks its documents reach; each partial is merged into
        (ctx, lse) of j's rows."""
        ch = self._chunks()
        cu, n = self.cu, self.n_seqs
        for (q0, q1) in ch:
            mtp.mtp_attn_fwd_block(d, a["qkv"], q0, q1, q0, q1, a["ctx"], a["lse"], cu, n)
        for j, i in self.cp_pairs():
            (q0, q1), (k0, k1) = ch[j], ch[i]
            mtp.mtp_attn_fwd_block(d, a["qkv"], q0, q1, k0, k1, a["ctx_p"], a["lse_p"], cu, n)
            mtp.mtp_attn_merge(d, a["ctx"], a["lse"], a["ctx_p"], a["lse_p"], q0, q1)

    def _attn_bwd_cp(self, d, a, ws, wsb):
        """Backward of every block pair with the merged ctx and lse: the
        diagonal pairs first (they write each chunk's dQ rows and dK/dV rows),
        then the pairs below the diagonal, which add into them."""
        ch = self._chunks()
        cu, n = self.cu, self.n_seqs
        for (q0, q1) in ch:
            mtp.mtp_attn_bwd_block(d, a["qkv"], a["ctx"], a["lse"], a["dctx"], a["dqkv"], q0, q1,
                                   q0, q1, 0, ws, wsb, cu, n)
        for j, i in self.cp_pairs():
            (q0, q1), (k0, k1) = ch[j], ch[i]
            mtp.mtp_attn_bwd_block(d, a["qkv"], a["ctx"], a["lse"], a["dctx"], a["dqkv"],
                                   q0, q1, k0, k1, 1, ws, wsb, cu, n)

    def partials(self) -> Dict[str, List[torch.Tensor]]:
        """This object's partial outputs, to be passed as ``external`` to a
        layer that computes the remaining ranks."""
        out = {
            "proj": [self.a[r]["p"].clone() for r in self.ranks],
            "fc2": [self.a[r]["q"].clone() for r in self.ranks],
            "fc1_dx": [self.a[r]["dln2"].clone() for r in self.ranks],
            "qkv_dx": [self.a[r]["dln1"].clone() for r in self.ranks],
        }
        if self.fp8:  # the amax parts of the tensors split over the ranks
            for k in ("ctx", "g", "du", "dqkv", "wqkv", "wo", "w1", "w2"):
                out["fp8_" + k] = [self.r8[r][k]["amax"].clone() for r in self.ranks]
            if self.sp:  # and of the row blocks each rank wrote
                for k in ("ln1", "ln2", "dy1"):
                    out["fp8_" + k] = [self.p8[k][r].clone() for r in self.ranks]
        return out


class VocabHead(_Probed):
    """Vocab-parallel output head with cross-entropy from per-shard stats.

    Rank r holds rows [r*V/t, (r+1)*V/t) of the output embedding
    (VocabParallelEmbedding, page "Megatron-LM: NVIDIA large-model training
    framework", section "Tensor parallelism").  Each shard computes its fp32
    logits, their max / sum-exp / target logit; the combine gives the loss
    per token; the backward writes dlogits and the shard's partial of dy.
    """

    def __init__(self, cfg, full: Dict[str, torch.Tensor], ranks: Optional[Sequence[int]] = None,
                 device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.ranks = list(range(cfg.tp)) if ranks is None else list(ranks)
        self.descs = {r: desc_for(cfg, r) for r in range(cfg.tp)}
        self.d0 = self.descs[self.ranks[0]]
        T, h, vl = cfg.tokens, cfg.hidden, cfg.vocab // cfg.tp
        vl_rows = slice(0, 0)
        self.emb = {r: full["emb"][r * vl:(r + 1) * vl].to(device).contiguous() for r in self.ranks}
        self.targets = full["targets"].to(device=device, dtype=torch.int32).contiguous()
        f32, dt = torch.float32, cfg.torch_dtype
        E = lambda *s, d=dt: torch.empty(*s, dtype=d, device=self.device)
        self.logits = {r: E(T, vl, d=f32) for r in self.ranks}
        self.stats = {r: (E(T, d=f32), E(T, d=f32), E(T, d=f32)) for r in self.ranks}
        self.dlogits = {r: E(T, vl) for r in self.ranks}
        self.dy_part = {r: E(T, h) for r in self.ranks}
        self.demb = {r: E(vl, h, d=f32) for r in self.ranks}
        self.M, self.S, self.loss = E(T, d=f32), E(T, d=f32), E(T, d=f32)
        self.loss_mean = E(1, d=f32)
        self.dy = E(T, h)
        self.probe = None
        del vl_rows

    def forward(self, y: torch.Tensor, external_stats: Sequence = ()):
        self.y = y
        T = self._timed
        for r in self.ranks:
            d = self.descs[r]
            with T("vocab_fwd"):
                mtp.mtp_col_linear_fwd(d, mtp.MTP_VOCAB, y, self.emb[r], None, self.logits[r],
                                       None)
            m, s, z = self.stats[r]
            with T("ce_stats"):
                mtp.mtp_vocab_ce_stats(d, self.logits[r], self.targets, m, s, z)
        stats = [self.stats[r] for r in self.ranks] + list(external_stats)
        with T("ce_combine"):
            mtp.mtp_vocab_ce_combine(self.d0, [s[0] for s in stats], [s[1] for s in stats],
                                     [s[2] for s in stats], self.M, self.S, self.loss,
                                     self.loss_mean)
        return self.loss_mean

    def backward(self, external_dy: Sequence[torch.Tensor] = ()):
        T = self._timed
        n_tok = self.cfg.tokens
        for r in self.ranks:
            d = self.descs[r]
            with T("ce_bwd"):
                mtp.mtp_vocab_ce_bwd(d, self.logits[r], self.targets, self.M, self.S,
                                     1.0 / max(n_tok, 1), self.dlogits[r])
            with T("vocab_bwd"):
                mtp.mtp_col_linear_bwd(d, mtp.MTP_VOCAB, self.dlogits[r], self.y, self.emb[r],
                                       self.dy_part[r], self.demb[r], None, 0, None, 0)
        parts = [self.dy_part[r] for r in self.ranks] + list(external_dy)
        with T("sum_vocab_dy"):
            mtp.mtp_partial_sum(self.d0, parts, None, None, self.dy)
        return self.dy

    def partials(self):
        """This object's per-rank stats and dy partials, to be passed as
        ``external_stats`` / ``external_dy`` to a head that computes the
        remaining ranks."""
        return ([tuple(t.clone() for t in self.stats[r]) for r in self.ranks],
                [self.dy_part[r].clone() for r in self.ranks])
