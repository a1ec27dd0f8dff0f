"""Seeded synthetic workloads for one pre-LN GPT transformer layer.

This module only draws random numbers and records shapes.  It holds none of
the layer's arithmetic, so both the fp64 CPU oracle and the HIP path can take
their inputs from it without sharing any computation.

Shapes follow the pages' statement of the problem: hidden size, attention
heads, FFN size, tensor-parallel size, sequence length and micro-batch
(page "Megatron-LM: NVIDIA's large-model training framework", section
"GPT model definition" with hidden 4096 / 32 heads / ffn 11008 / seq 2048;
page "Megatron-LM 3D parallelism guide", §3.2 for hidden 12288 under TP 8;
page "Megatron-LM / Megatron Core README digest", §5 "Benchmark" for vocab
131072 at sequence length 4096).

Generation recipe (fixed order, one ``torch.Generator`` seeded with
``cfg.seed``, values drawn in float32 then rounded to the config dtype with
round-to-nearest-even):

1. varlen configs only: document lengths, integer-uniform in
   ``[doc_min, doc_max]``, drawn until they cover ``tokens``; the last one is
   truncated to fit (it may end shorter than ``doc_min``);
2. ``x`` ~ N(0, 1), shape [T, h];
3. ``dy`` ~ N(0, 1), shape [T, h] (not drawn for vocab-head configs, whose
   upstream gradient comes from the cross-entropy head);
4. ``wq, wk, wv, wo`` ~ N(0, 0.02), shape [h, h];
5. ``w1`` ~ N(0, 0.02), shape [f, h]; ``w2`` ~ N(0, 0.02), shape [h, f];
6. vocab configs: ``emb`` ~ N(0, 0.02), shape [V, h], then ``targets``
   integer-uniform over [0, V), shape [T].

Biases are zero, LayerNorm gamma is one and beta zero (``zeros``/``ones``),
unless ``affine_random`` is set: then, after everything above, the biases
bqkv, bo, b1, b2 and LayerNorm betas are drawn ~ N(0, 0.1) and the gammas
~ 1 + N(0, 0.1), in that order, so that tests exercise every affine term.
Weights use the nn.Linear convention W[out, in] so a linear map is x @ W.T.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

__all__ = ["LayerConfig", "CONFIGS", "PARITY_CASES", "generate", "get_config"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int
    heads: int
    ffn: int
    tp: int
    seq_len: int
    micro_batch: int = 1
    dtype: str = "bf16"          # "f32" or "bf16": storage type of weights/activations
    vocab: int = 0               # 0: no vocab-parallel head
    varlen_tokens: int = 0       # >0: packed variable-length batch of this many tokens
    doc_min: int = 0
    doc_max: int = 0
    eps: float = 1e-5
    seed: int = 0
    affine_random: bool = False  # draw non-trivial biases / LayerNorm affine
    sequence_parallel: bool = False  # per-token work on T/tp row blocks per rank
    swiglu: bool = False         # SwiGLU FFN (gate w1, up w3), no FFN-input bias b1
    context_parallel: int = 1    # attention over this many sequence chunks, pair by pair
    fp8: bool = False            # the four linear maps and their gradients on FP8 codes
    description: str = ""

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def tokens(self) -> int:
        return self.varlen_tokens if self.varlen_tokens else self.seq_len * self.micro_batch

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads the method is measured on.
CONFIGS: Dict[str, LayerConfig] = {
    "tiny_tp2": LayerConfig(
        "tiny_tp2", hidden=256, heads=4, ffn=1024, tp=2, seq_len=128, dtype="f32",
        description="tiny pre-LN GPT layer, TP=2 (both shards), fp32"),
    "7b_tp2": LayerConfig(
        "7b_tp2", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        description="7B-style layer, one TP=2 rank shard, bf16"),
    "wide_tp8": LayerConfig(
        "wide_tp8", hidden=12288, heads=96, ffn=49152, tp=8, seq_len=2048, dtype="bf16",
        description="wide layer, TP=8, all 8 shards in sequence, bf16"),
    "bench_tp4_vocab": LayerConfig(
        "bench_tp4_vocab", hidden=8192, heads=64, ffn=32768, tp=4, seq_len=4096, dtype="bf16",
        vocab=131072, description="benchmark-shaped layer + vocab-parallel CE head, TP=4, bf16"),
    "7b_tp2_sp": LayerConfig(
        "7b_tp2_sp", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        sequence_parallel=True,
        description="7B-style layer, one TP=2 rank shard with sequence parallelism, bf16"),
    "7b_tp2_swiglu": LayerConfig(
        "7b_tp2_swiglu", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        swiglu=True,
        description="7B-style layer with a SwiGLU FFN (gate and up 11008 wide, no FFN-input "
                    "bias), one TP=2 rank shard, bf16"),
    "7b_tp2_cp2": LayerConfig(
        "7b_tp2_cp2", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        context_parallel=2,
        description="7B-style layer, one TP=2 rank shard, attention as 2 context-parallel "
                    "chunks merged by log-sum-exp, bf16"),
    "7b_tp2_fp8": LayerConfig(
        "7b_tp2_fp8", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        fp8=True,
        description="7B-style layer, one TP=2 rank shard, its twelve GEMMs on FP8 codes (E4M3 "
                    "activations and weights, E5M2 gradients, per-tensor scales), bf16 elsewhere"),
    "7b_tp2_swiglu_fp8": LayerConfig(
        "7b_tp2_swiglu_fp8", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        swiglu=True, fp8=True,
        description="7B-style layer with a SwiGLU FFN, one TP=2 rank shard, its twelve GEMMs on "
                    "FP8 codes (gate and up under one scale), bf16 elsewhere"),
    "7b_tp2_sp_fp8": LayerConfig(
        "7b_tp2_sp_fp8", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        sequence_parallel=True, fp8=True,
        description="7B-style layer, one TP=2 rank shard with sequence parallelism, its twelve "
                    "GEMMs on FP8 codes, bf16 elsewhere"),
    "7b_tp2_cp2_fp8": LayerConfig(
        "7b_tp2_cp2_fp8", hidden=4096, heads=32, ffn=11008, tp=2, seq_len=2048, dtype="bf16",
        context_parallel=2, fp8=True,
        description="7B-style layer, one TP=2 rank shard, 2-chunk context-parallel attention, its "
                    "twelve GEMMs on FP8 codes, bf16 elsewhere"),
    "varlen_tp1": LayerConfig(
        "varlen_tp1", hidden=4096, heads=32, ffn=11008, tp=1, seq_len=16384, dtype="bf16",
        varlen_tokens=16384, doc_min=256, doc_max=4096,
        description="packed variable-length batch, TP=1, bf16"),
    "varlen_tp1_fp8": LayerConfig(
        "varlen_tp1_fp8", hidden=4096, heads=32, ffn=11008, tp=1, seq_len=16384, dtype="bf16",
        varlen_tokens=16384, doc_min=256, doc_max=4096, fp8=True,
        description="packed variable-length batch, TP=1, its twelve GEMMs on FP8 codes, bf16 "
                    "elsewhere"),
    "varlen_tp1_cp4": LayerConfig(
        "varlen_tp1_cp4", hidden=4096, heads=32, ffn=11008, tp=1, seq_len=16384, dtype="bf16",
        varlen_tokens=16384, doc_min=256, doc_max=4096, context_parallel=4,
        description="the packed variable-length batch, TP=1, attention as 4 context-parallel "
                    "chunks of 4096 tokens (block pairs only where a document crosses), bf16"),
}

# Scaled-down cases with the same structure that the oracle finishes in
# seconds; token counts and FFN widths are chosen to leave ragged tails
# against 32/64/128/256-wide tiles.
PARITY_CASES: Dict[str, LayerConfig] = {
    "small_bf16_tp2": LayerConfig(
        "small_bf16_tp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=300, dtype="bf16",
        affine_random=True),
    "small_bf16_d64_tp4": LayerConfig(
        "small_bf16_d64_tp4", hidden=512, heads=8, ffn=2080, tp=4, seq_len=200, dtype="bf16",
        affine_random=True),
    "small_bf16_mb2": LayerConfig(
        "small_bf16_mb2", hidden=256, heads=2, ffn=768, tp=2, seq_len=136, micro_batch=2,
        dtype="bf16"),
    "small_varlen_tp1": LayerConfig(
        "small_varlen_tp1", hidden=256, heads=2, ffn=1024, tp=1, seq_len=1000, dtype="bf16",
        varlen_tokens=1000, doc_min=1, doc_max=300, affine_random=True),
    "small_vocab_tp4": LayerConfig(
        "small_vocab_tp4", hidden=512, heads=4, ffn=1024, tp=4, seq_len=264, dtype="bf16",
        vocab=8192),
    "small_f32_tp4": LayerConfig(
        "small_f32_tp4", hidden=256, heads=4, ffn=1024, tp=4, seq_len=77, dtype="f32",
        affine_random=True),
    "small_bf16_tp2_sp": LayerConfig(
        "small_bf16_tp2_sp", hidden=512, heads=4, ffn=1376, tp=2, seq_len=304, dtype="bf16",
        affine_random=True, sequence_parallel=True),
    "small_f32_tp4_sp": LayerConfig(
        "small_f32_tp4_sp", hidden=256, heads=4, ffn=1024, tp=4, seq_len=80, dtype="f32",
        affine_random=True, sequence_parallel=True),
    "tiny_swiglu_tp2": LayerConfig(
        "tiny_swiglu_tp2", hidden=256, heads=4, ffn=1024, tp=2, seq_len=128, dtype="f32",
        swiglu=True, affine_random=True),
    "small_bf16_swiglu_tp2": LayerConfig(
        "small_bf16_swiglu_tp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=300, dtype="bf16",
        swiglu=True, affine_random=True),
    "small_bf16_swiglu_sp_tp4": LayerConfig(
        "small_bf16_swiglu_sp_tp4", hidden=512, heads=8, ffn=2080, tp=4, seq_len=208,
        dtype="bf16", swiglu=True, sequence_parallel=True),
    "small_bf16_tp2_cp2": LayerConfig(
        "small_bf16_tp2_cp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=300, dtype="bf16",
        affine_random=True, context_parallel=2),
    "small_bf16_d64_cp4": LayerConfig(
        "small_bf16_d64_cp4", hidden=512, heads=8, ffn=2080, tp=4, seq_len=264, dtype="bf16",
        context_parallel=4),
    # packed documents over context-parallel chunks of 250 and 320 tokens:
    # chunk edges fall inside documents and inside 64-row tiles
    "small_varlen_cp4": LayerConfig(
        "small_varlen_cp4", hidden=256, heads=2, ffn=1024, tp=1, seq_len=1000, dtype="bf16",
        varlen_tokens=1000, doc_min=1, doc_max=300, context_parallel=4, affine_random=True),
    "small_varlen_d64_tp2_cp3": LayerConfig(
        "small_varlen_d64_tp2_cp3", hidden=512, heads=8, ffn=1376, tp=2, seq_len=960,
        dtype="bf16", varlen_tokens=960, doc_min=1, doc_max=400, context_parallel=3),
    # FP8 layer steps: token counts and reduction widths multiples of 16
    # (the FP8 GEMMs' 16-byte k chunks), ragged against the tiles otherwise
    "small_fp8_tp2": LayerConfig(
        "small_fp8_tp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=304, dtype="bf16",
        affine_random=True, fp8=True),
    "small_fp8_d64_tp4": LayerConfig(
        "small_fp8_d64_tp4", hidden=512, heads=8, ffn=2176, tp=4, seq_len=208, dtype="bf16",
        fp8=True),
    # the FP8 step over packed documents (block-diagonal causal attention)
    "small_fp8_varlen_tp2": LayerConfig(
        "small_fp8_varlen_tp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=304, dtype="bf16",
        varlen_tokens=304, doc_min=1, doc_max=150, affine_random=True, fp8=True),
    # the FP8 step with the SwiGLU FFN (gate|up one tensor under one scale)
    "small_fp8_swiglu_tp2": LayerConfig(
        "small_fp8_swiglu_tp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=304, dtype="bf16",
        swiglu=True, affine_random=True, fp8=True),
    "small_fp8_swiglu_d64_tp4": LayerConfig(
        "small_fp8_swiglu_d64_tp4", hidden=512, heads=8, ffn=2176, tp=4, seq_len=208,
        dtype="bf16", swiglu=True, fp8=True),
    # the FP8 step with context-parallel attention (chunks of 152 and 208
    # tokens; packed documents cross the chunk edges in the second case)
    "small_fp8_tp2_cp2": LayerConfig(
        "small_fp8_tp2_cp2", hidden=512, heads=4, ffn=1376, tp=2, seq_len=304, dtype="bf16",
        affine_random=True, fp8=True, context_parallel=2),
    "small_fp8_varlen_d64_cp3": LayerConfig(
        "small_fp8_varlen_d64_cp3", hidden=512, heads=8, ffn=1376, tp=2, seq_len=624,
        dtype="bf16", varlen_tokens=624, doc_min=1, doc_max=300, fp8=True, context_parallel=3),
    # the FP8 step over eight tensor-parallel shards (every split tensor's
    # scale merges eight ranks' amax parts)
    "small_fp8_tp8": LayerConfig(
        "small_fp8_tp8", hidden=1024, heads=8, ffn=4096, tp=8, seq_len=208, dtype="bf16",
        affine_random=True, fp8=True),
    # the FP8 step over two micro-batch sequences of 136 tokens (T = 272)
    "small_fp8_mb2": LayerConfig(
        "small_fp8_mb2", hidden=256, heads=2, ffn=768, tp=2, seq_len=136, micro_batch=2,
        dtype="bf16", affine_random=True, fp8=True),
    # the FP8 step with sequence parallelism (LayerNorm and the sums on row
    # blocks of 152 and 52 tokens)
    "small_fp8_tp2_sp": LayerConfig(
        "small_fp8_tp2_sp", hidden=512, heads=4, ffn=1376, tp=2, seq_len=304, dtype="bf16",
        affine_random=True, sequence_parallel=True, fp8=True),
    "small_fp8_swiglu_sp_tp4": LayerConfig(
        "small_fp8_swiglu_sp_tp4", hidden=512, heads=8, ffn=2176, tp=4, seq_len=208,
        dtype="bf16", swiglu=True, sequence_parallel=True, fp8=True),
    "one_token_bf16": LayerConfig(
        "one_token_bf16", hidden=256, heads=2, ffn=512, tp=2, seq_len=1, dtype="bf16"),
}


def get_config(name: str) -> LayerConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    return PARITY_CASES[name]


def _doc_lengths(cfg: LayerConfig, g: torch.Generator) -> List[int]:
    lens: List[int] = []
    total = 0
    while total < cfg.varlen_tokens:
        n = int(torch.randint(cfg.doc_min, cfg.doc_max + 1, (1,), generator=g).item())
        n = min(n, cfg.varlen_tokens - total)
        lens.append(n)
        total += n
    return lens


def generate(cfg: LayerConfig, device: str = "cpu") -> Dict[str, object]:
    """Draw every input of one layer step for ``cfg`` (see module docstring).

    Returns a dict of tensors in the config dtype (targets and cu_seqlens are
    int32).  ``cu_seqlens`` is always present: for fixed-length batches it
    marks the micro-batch sequence boundaries.
    """
    g = torch.Generator().manual_seed(cfg.seed)
    T, h, f = cfg.tokens, cfg.hidden, cfg.ffn
    dt = cfg.torch_dtype
    out: Dict[str, object] = {}
    if cfg.varlen_tokens:
        lens = _doc_lengths(cfg, g)
    else:
        lens = [cfg.seq_len] * cfg.micro_batch
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)

    def normal(shape, std):
        t = torch.randn(*shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dt)

    out["x"] = normal((T, h), 1.0)
    if not cfg.vocab:
        out["dy"] = normal((T, h), 1.0)
    for name in ("wq", "wk", "wv", "wo"):
        out[name] = normal((h, h), 0.02)
    out["w1"] = normal((f, h), 0.02)
    out["w2"] = normal((h, f), 0.02)
    if cfg.swiglu:
        out["w3"] = normal((f, h), 0.02)
    if cfg.vocab:
        out["emb"] = normal((cfg.vocab, h), 0.02)
        out["targets"] = torch.randint(0, cfg.vocab, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    if cfg.affine_random:
        out["bqkv"] = normal((3 * h,), 0.1)
        out["bo"] = normal((h,), 0.1)
        out["b1"] = normal((f,), 0.1)
        out["b2"] = normal((h,), 0.1)
        out["ln1_b"] = normal((h,), 0.1)
        out["ln2_b"] = normal((h,), 0.1)
        out["ln1_g"] = (1.0 + torch.randn(h, generator=g) * 0.1).to(dt)
        out["ln2_g"] = (1.0 + torch.randn(h, generator=g) * 0.1).to(dt)
    else:
        out["bqkv"] = torch.zeros(3 * h, dtype=dt)
        out["bo"] = torch.zeros(h, dtype=dt)
        out["b1"] = torch.zeros(f, dtype=dt)
        out["b2"] = torch.zeros(h, dtype=dt)
        out["ln1_b"] = torch.zeros(h, dtype=dt)
        out["ln2_b"] = torch.zeros(h, dtype=dt)
        out["ln1_g"] = torch.ones(h, dtype=dt)
        out["ln2_g"] = torch.ones(h, dtype=dt)
    if cfg.swiglu:
        del out["b1"]  # the SwiGLU variant has no bias on the FFN input
    if device != "cpu":
        out = {k: v.to(device) for k, v in out.items()}
    return out
