"""ctypes binding of libmtp (include/mtp.h): argument marshalling only.

Every function here has the name of the C entry point it wraps and takes
the same arguments in the same order; tensors may be passed as torch tensors
(their ``data_ptr()`` is used) or as raw integer device addresses.  The
``stream`` argument defaults to torch's current HIP stream.  A non-zero
status raises ``MtpError``.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmtp.so")

MTP_OK, MTP_ERR_INVALID_ARG, MTP_ERR_UNSUPPORTED, MTP_ERR_WORKSPACE, MTP_ERR_HIP = range(5)
MTP_F32, MTP_BF16 = 0, 1
MTP_QKV, MTP_PROJ, MTP_FC1, MTP_FC2, MTP_VOCAB, MTP_FC1_SWIGLU, MTP_FC2_SWIGLU = range(7)
MTP_FP8_E4M3, MTP_FP8_E5M2 = 0, 1
FP8_AMAX_PARTS = 1024  # fp32 partial maxima written by mtp_fp8_amax
(MTP_OP_LAYERNORM_BWD, MTP_OP_COL_LINEAR_BWD, MTP_OP_ROW_LINEAR_BWD, MTP_OP_ATTN_BWD,
 MTP_OP_VOCAB_CE) = range(5)


class MtpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} -> {status}: {mtp_status_string(status)}")


class mtp_shard_desc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("tp_size", ctypes.c_int32), ("tp_rank", ctypes.c_int32),
        ("seq_len", ctypes.c_int32), ("micro_batch", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
    ]


_lib: Optional[ctypes.CDLL] = None

_VP = ctypes.c_void_p
_FP = ctypes.c_void_p  # float* passed as an address
_SIGS = {
    "mtp_version": (ctypes.c_int, []),
    "mtp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mtp_workspace_size": (ctypes.c_size_t, [_VP, ctypes.c_int, ctypes.c_int]),
    "mtp_layernorm": (ctypes.c_int, [_VP] + [_VP] * 7 + [_VP]),
    "mtp_layernorm_bwd": (ctypes.c_int, [_VP] + [_VP] * 9 + [ctypes.c_int, _VP, ctypes.c_size_t, _VP]),
    "mtp_col_linear_fwd": (ctypes.c_int, [_VP, ctypes.c_int] + [_VP] * 5 + [_VP]),
    "mtp_col_linear_bwd": (ctypes.c_int, [_VP, ctypes.c_int] + [_VP] * 6
                           + [ctypes.c_int, _VP, ctypes.c_size_t, _VP]),
    "mtp_row_linear_fwd": (ctypes.c_int, [_VP, ctypes.c_int] + [_VP] * 3 + [_VP]),
    "mtp_row_linear_bwd": (ctypes.c_int, [_VP, ctypes.c_int] + [_VP] * 7
                           + [ctypes.c_int, _VP, ctypes.c_size_t, _VP]),
    "mtp_attn_fwd": (ctypes.c_int, [_VP] + [_VP] * 4 + [ctypes.c_int32, _VP, _VP]),
    "mtp_attn_bwd": (ctypes.c_int, [_VP] + [_VP] * 6
                     + [ctypes.c_int32, _VP, ctypes.c_size_t, _VP, _VP]),
    "mtp_attn_bwd_noalloc": (ctypes.c_int, [_VP] + [_VP] * 6 + [ctypes.c_int32, _VP]),
    "mtp_quantize_fp8": (ctypes.c_int, [_VP, _VP, ctypes.c_int64, _VP, _VP, _VP]),
    "mtp_linear_fwd_fp8": (ctypes.c_int, [_VP, ctypes.c_int] + [_VP] * 8 + [_VP]),
    "mtp_fp8_amax": (ctypes.c_int, [_VP, _VP, ctypes.c_int64, _VP, _VP]),
    "mtp_fp8_quantize": (ctypes.c_int, [_VP, ctypes.c_int, _VP, ctypes.c_int64, ctypes.c_int64,
                                        _VP, ctypes.c_int32, _VP, _VP, _VP, _VP]),
    "mtp_linear_bwd_fp8": (ctypes.c_int, [_VP, ctypes.c_int] + [_VP] * 10
                           + [ctypes.c_int, _VP, _VP]),
    "mtp_attn_fwd_block": (ctypes.c_int, [_VP, _VP] + [ctypes.c_int64] * 4
                           + [_VP, _VP, _VP, ctypes.c_int32, _VP]),
    "mtp_attn_merge": (ctypes.c_int, [_VP] + [_VP] * 4 + [ctypes.c_int64] * 2 + [_VP]),
    "mtp_attn_bwd_block": (ctypes.c_int, [_VP] + [_VP] * 5 + [ctypes.c_int64] * 4
                           + [ctypes.c_int, _VP, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]),
    "mtp_partial_sum": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, _VP, _VP, _VP]),
    "mtp_partial_sum_layernorm": (ctypes.c_int, [_VP, _VP, ctypes.c_int32] + [_VP] * 9 + [_VP]),
    "mtp_layernorm_bwd_sum": (ctypes.c_int, [_VP, _VP, ctypes.c_int32] + [_VP] * 8
                              + [ctypes.c_int, _VP, ctypes.c_size_t, _VP, _VP]),
    "mtp_vocab_ce_stats": (ctypes.c_int, [_VP] + [_VP] * 5 + [_VP]),
    "mtp_vocab_ce_combine": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int32] + [_VP] * 4 + [_VP]),
    "mtp_vocab_ce_bwd": (ctypes.c_int, [_VP] + [_VP] * 4 + [ctypes.c_float, _VP, _VP]),
}


def lib() -> ctypes.CDLL:
    """Load libmtp.so (built in-tree).  Fails loudly when it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m tensor_transformer_layer_04_amd.build` "
                "(there is no fallback implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def exported_names() -> Sequence[str]:
    return list(_SIGS)


def _addr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[_addr(t) for t in ts])
    return arr


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != MTP_OK:
        raise MtpError(name, st)
    return st


def make_desc(hidden, heads, ffn, tp_size, tp_rank, seq_len, micro_batch=1, dtype=MTP_BF16,
              vocab=0, ln_eps=1e-5) -> mtp_shard_desc:
    return mtp_shard_desc(hidden, heads, ffn, vocab, tp_size, tp_rank, seq_len, micro_batch,
                          dtype, ln_eps)


def mtp_version() -> int:
    return lib().mtp_version()


def mtp_status_string(status: int) -> str:
    return lib().mtp_status_string(status).decode()


def mtp_workspace_size(desc, op, kind=0) -> int:
    return lib().mtp_workspace_size(ctypes.byref(desc), op, kind)


def mtp_layernorm(desc, x, gamma, beta, y, mean, rstd, amax_parts=None, stream=None):
    return _call("mtp_layernorm", ctypes.byref(desc), _addr(x), _addr(gamma), _addr(beta),
                 _addr(y), _addr(mean), _addr(rstd), _addr(amax_parts), _stream(stream))


def mtp_layernorm_bwd(desc, dy, x, gamma, mean, rstd, dres, dx, dgamma, dbeta, accumulate, ws,
                      ws_bytes, stream=None):
    return _call("mtp_layernorm_bwd", ctypes.byref(desc), _addr(dy), _addr(x), _addr(gamma),
                 _addr(mean), _addr(rstd), _addr(dres), _addr(dx), _addr(dgamma), _addr(dbeta),
                 int(accumulate), _addr(ws), ws_bytes, _stream(stream))


def mtp_col_linear_fwd(desc, kind, x, w, b, y, preact, stream=None):
    return _call("mtp_col_linear_fwd", ctypes.byref(desc), kind, _addr(x), _addr(w), _addr(b),
                 _addr(y), _addr(preact), _stream(stream))


def mtp_col_linear_bwd(desc, kind, dy, x, w, dx_partial, dw, db, accumulate, ws, ws_bytes,
                       stream=None):
    return _call("mtp_col_linear_bwd", ctypes.byref(desc), kind, _addr(dy), _addr(x), _addr(w),
                 _addr(dx_partial), _addr(dw), _addr(db), int(accumulate), _addr(ws), ws_bytes,
                 _stream(stream))


def mtp_row_linear_fwd(desc, kind, x_local, w, partial, stream=None):
    return _call("mtp_row_linear_fwd", ctypes.byref(desc), kind, _addr(x_local), _addr(w),
                 _addr(partial), _stream(stream))


def mtp_row_linear_bwd(desc, kind, dy, x_local, w, gelu_preact, dx_local, dw, db, accumulate, ws,
                       ws_bytes, stream=None):
    return _call("mtp_row_linear_bwd", ctypes.byref(desc), kind, _addr(dy), _addr(x_local),
                 _addr(w), _addr(gelu_preact), _addr(dx_local), _addr(dw), _addr(db),
                 int(accumulate), _addr(ws), ws_bytes, _stream(stream))


def mtp_attn_fwd(desc, qkv, ctx, lse, cu_seqlens=None, n_seqs=0, ctx_amax_parts=None,
                 stream=None):
    return _call("mtp_attn_fwd", ctypes.byref(desc), _addr(qkv), _addr(ctx), _addr(lse),
                 _addr(cu_seqlens), int(n_seqs), _addr(ctx_amax_parts), _stream(stream))


def mtp_attn_bwd(desc, qkv, ctx, lse, dctx, dqkv, cu_seqlens, n_seqs, ws, ws_bytes,
                 dqkv_amax_parts=None, stream=None):
    return _call("mtp_attn_bwd", ctypes.byref(desc), _addr(qkv), _addr(ctx), _addr(lse),
                 _addr(dctx), _addr(dqkv), _addr(cu_seqlens), int(n_seqs), _addr(ws), ws_bytes,
                 _addr(dqkv_amax_parts), _stream(stream))


def mtp_attn_bwd_noalloc(desc, qkv, ctx, lse, dctx, dqkv, cu_seqlens, n_seqs, stream=None):
    return _call("mtp_attn_bwd_noalloc", ctypes.byref(desc), _addr(qkv), _addr(ctx), _addr(lse),
                 _addr(dctx), _addr(dqkv), _addr(cu_seqlens), int(n_seqs), _stream(stream))


def mtp_quantize_fp8(desc, x, n, q, scale, stream=None):
    return _call("mtp_quantize_fp8", ctypes.byref(desc), _addr(x), int(n), _addr(q), _addr(scale),
                 _stream(stream))


def mtp_linear_fwd_fp8(desc, kind, x8, x_scale, w8, w_scale, b, y, preact, amax_parts=None,
                       stream=None):
    return _call("mtp_linear_fwd_fp8", ctypes.byref(desc), kind, _addr(x8), _addr(x_scale),
                 _addr(w8), _addr(w_scale), _addr(b), _addr(y), _addr(preact),
                 _addr(amax_parts), _stream(stream))


def mtp_fp8_amax(desc, x, n, amax_parts, stream=None):
    return _call("mtp_fp8_amax", ctypes.byref(desc), _addr(x), int(n), _addr(amax_parts),
                 _stream(stream))


def mtp_fp8_quantize(desc, fmt, x, rows, cols, amax_parts, q, q_t, scale, stream=None):
    """``amax_parts``: a sequence of device tensors (one per shard)."""
    arr = (ctypes.c_void_p * len(amax_parts))(*[_addr(a) for a in amax_parts])
    return _call("mtp_fp8_quantize", ctypes.byref(desc), int(fmt), _addr(x), int(rows), int(cols),
                 arr, len(amax_parts), _addr(q), _addr(q_t), _addr(scale), _stream(stream))


def mtp_linear_bwd_fp8(desc, kind, dy8, dy8_t, dy_scale, w8_t, w_scale, x8_t, x_scale, preact,
                       dx, dw, accumulate=0, dx_amax_parts=None, stream=None):
    return _call("mtp_linear_bwd_fp8", ctypes.byref(desc), kind, _addr(dy8), _addr(dy8_t),
                 _addr(dy_scale), _addr(w8_t), _addr(w_scale), _addr(x8_t), _addr(x_scale),
                 _addr(preact), _addr(dx), _addr(dw), int(accumulate), _addr(dx_amax_parts),
                 _stream(stream))


def mtp_attn_fwd_block(desc, qkv, q_lo, q_hi, k_lo, k_hi, ctx, lse, cu_seqlens=None, n_seqs=0,
                       stream=None):
    return _call("mtp_attn_fwd_block", ctypes.byref(desc), _addr(qkv), q_lo, q_hi, k_lo, k_hi,
                 _addr(ctx), _addr(lse), _addr(cu_seqlens), int(n_seqs), _stream(stream))


def mtp_attn_merge(desc, ctx, lse, ctx_part, lse_part, row_lo, row_hi, stream=None):
    return _call("mtp_attn_merge", ctypes.byref(desc), _addr(ctx), _addr(lse), _addr(ctx_part),
                 _addr(lse_part), row_lo, row_hi, _stream(stream))


def mtp_attn_bwd_block(desc, qkv, ctx, lse, dctx, dqkv, q_lo, q_hi, k_lo, k_hi, accumulate, ws,
                       ws_bytes, cu_seqlens=None, n_seqs=0, stream=None):
    return _call("mtp_attn_bwd_block", ctypes.byref(desc), _addr(qkv), _addr(ctx), _addr(lse),
                 _addr(dctx), _addr(dqkv), q_lo, q_hi, k_lo, k_hi, accumulate,
                 _addr(cu_seqlens), int(n_seqs), _addr(ws), ws_bytes, _stream(stream))


def mtp_partial_sum(desc, partials, bias, residual, out, stream=None):
    arr = _ptr_array(partials)
    return _call("mtp_partial_sum", ctypes.byref(desc), arr, len(partials), _addr(bias),
                 _addr(residual), _addr(out), _stream(stream))


def mtp_partial_sum_layernorm(desc, partials, bias, residual, out, gamma, beta, ln_out, mean,
                              rstd, amax_parts=None, stream=None):
    arr = _ptr_array(partials)
    return _call("mtp_partial_sum_layernorm", ctypes.byref(desc), arr, len(partials), _addr(bias),
                 _addr(residual), _addr(out), _addr(gamma), _addr(beta), _addr(ln_out),
                 _addr(mean), _addr(rstd), _addr(amax_parts), _stream(stream))


def mtp_layernorm_bwd_sum(desc, dy_partials, x, gamma, mean, rstd, dres, dx, dgamma, dbeta,
                          accumulate, ws, ws_bytes, amax_parts=None, stream=None):
    arr = _ptr_array(dy_partials)
    return _call("mtp_layernorm_bwd_sum", ctypes.byref(desc), arr, len(dy_partials), _addr(x),
                 _addr(gamma), _addr(mean), _addr(rstd), _addr(dres), _addr(dx), _addr(dgamma),
                 _addr(dbeta), int(accumulate), _addr(ws), ws_bytes, _addr(amax_parts),
                 _stream(stream))


def mtp_vocab_ce_stats(desc, logits, targets, m, s, z_tgt, stream=None):
    return _call("mtp_vocab_ce_stats", ctypes.byref(desc), _addr(logits), _addr(targets), _addr(m),
                 _addr(s), _addr(z_tgt), _stream(stream))


def mtp_vocab_ce_combine(desc, m_list, s_list, zt_list, M, S, loss, loss_mean, stream=None):
    n = len(m_list)
    return _call("mtp_vocab_ce_combine", ctypes.byref(desc), _ptr_array(m_list),
                 _ptr_array(s_list), _ptr_array(zt_list), n, _addr(M), _addr(S), _addr(loss),
                 _addr(loss_mean), _stream(stream))


def mtp_vocab_ce_bwd(desc, logits, targets, M, S, dloss_scale, dlogits, stream=None):
    return _call("mtp_vocab_ce_bwd", ctypes.byref(desc), _addr(logits), _addr(targets), _addr(M),
                 _addr(S), float(dloss_scale), _addr(dlogits), _stream(stream))
