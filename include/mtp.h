/*
 * mtp.h -- C ABI of libmtp: one tensor-parallel rank's shard of a pre-LN GPT
 * transformer layer, forward and backward, on one AMD MI355X (gfx950).
 *
 * The method (page "Megatron-LM 3D parallelism guide", §2.1 "Tensor
 * parallelism"): the Q/K/V projection weights are split by output columns
 * across the t ranks of a tensor-parallel group and every rank receives the
 * whole input ("column parallel", no exchange in forward); the attention
 * output projection is split by input rows, so each rank produces a partial
 * of the full output and the partials are summed ("row parallel").  The MLP
 * uses the same column/row pair.  The problem is stated by hidden size,
 * attention heads, TP size and rank, sequence length and micro-batch (page
 * "Megatron-LM: NVIDIA large-model training framework", sections
 * "Configuration example", "Launching training" and "GPT model definition").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - T = seq_len * micro_batch tokens; h hidden; a heads; d = h/a head
 *    size; t = tp_size; h_l = h/t, a_l = a/t, f_l = ffn/t, V_l = vocab/t.
 *  - Activations are token-major, row-major [T, features], element type
 *    `desc->dtype` (fp32 or bf16).  Weights use the nn.Linear convention
 *    W[out, in] (y = x W^T) in `desc->dtype`.  Weight and bias gradients are
 *    fp32.  Statistics (LayerNorm mean/rstd, attention log-sum-exp,
 *    cross-entropy max/sum) are fp32.
 *  - Rank r's QKV output is [T, 3*h_l] = [q_r | k_r | v_r]; inside each
 *    block head n (local) owns columns n*d .. n*d+d-1.  The caller packs the
 *    rank's weight shard accordingly: Wqkv_r = [Wq rows r*h_l..; Wk rows
 *    r*h_l..; Wv rows r*h_l..], shape [3*h_l, h].
 *  - Every pointer argument is caller-owned device memory, 16-byte aligned,
 *    contiguous with the documented shape, unless documented as a host
 *    pointer.  The library allocates nothing and keeps no state between
 *    calls; scratch memory is passed as `ws`/`ws_bytes`, sized by
 *    mtp_workspace_size().
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and never synchronises.
 *  - Return value: MTP_OK, or an error code.  Arguments are validated before
 *    any device work is enqueued, so an error return means nothing was
 *    launched, except MTP_ERR_HIP (a launch failed; earlier kernels of the
 *    same call may have been enqueued).  No call aborts the process.
 *  - Size limit: the kernels address the GEMM operands (activations,
 *    weights, their gradients and FP8 codes) and the attention inputs,
 *    statistics and workspace through 32-bit buffer offsets, so each such
 *    tensor must span less than 2 GiB.  A call whose tensors exceed that
 *    returns MTP_ERR_UNSUPPORTED before anything is enqueued.
 *  - T = 0 is valid: the call is a no-op except that non-accumulating
 *    gradient outputs (dgamma/dbeta, dw, db) are set to zero.
 */
#ifndef MTP_H
#define MTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_VERSION 1

enum mtp_status {
    MTP_OK = 0,
    MTP_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad rank, divisibility  */
    MTP_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, dtype, ...)  */
    MTP_ERR_WORKSPACE = 3,    /* ws too small or NULL where needed                 */
    MTP_ERR_HIP = 4           /* a HIP launch reported an error                    */
};

typedef enum { MTP_F32 = 0, MTP_BF16 = 1 } mtp_dtype;

/* Which of the layer's linear maps a call computes. */
typedef enum {
    MTP_QKV = 0,   /* column parallel: [T,h] -> [T,3h_l], bias [3h_l]            */
    MTP_PROJ = 1,  /* row parallel:    [T,h_l] -> partial [T,h]                   */
    MTP_FC1 = 2,   /* column parallel: [T,h] -> [T,f_l], GeLU-tanh applied         */
    MTP_FC2 = 3,   /* row parallel:    [T,f_l] -> partial [T,h]                   */
    MTP_VOCAB = 4, /* column parallel vocab head: [T,h] -> fp32 logits [T,V_l]   */
    /* SwiGLU FFN without a bias on its input (page "Megatron-LM 3D
     * parallelism guide", §3.3: --swiglu --disable-bias-linear):          */
    MTP_FC1_SWIGLU = 5, /* column parallel: [T,h] -> gate|up [T,2f_l] -> SiLU(gate)*up [T,f_l] */
    MTP_FC2_SWIGLU = 6  /* row parallel: [T,f_l] -> partial [T,h] (as MTP_FC2)  */
} mtp_linear_kind;

/* Operation ids for mtp_workspace_size(). */
typedef enum {
    MTP_OP_LAYERNORM_BWD = 0,
    MTP_OP_COL_LINEAR_BWD = 1,
    MTP_OP_ROW_LINEAR_BWD = 2,
    MTP_OP_ATTN_BWD = 3,
    MTP_OP_VOCAB_CE = 4
} mtp_op;

/* FP8 formats (see the FP8 section below). */
typedef enum { MTP_FP8_E4M3 = 0, MTP_FP8_E5M2 = 1 } mtp_fp8_format;

/*
 * The problem statement of one shard.  Divisibility follows the pages
 * (page "Megatron-LM 3D parallelism guide", §3.2: hidden size and head
 * count must divide by the TP size, e.g. 12288/8 = 1536 per rank while a TP
 * size of 5 is rejected).  Additionally d must be 64 or 128, f_l and V_l
 * multiples of 8 (MTP_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
    int32_t hidden;       /* h                                                   */
    int32_t heads;        /* a                                                   */
    int32_t ffn;          /* f (MLP inner size, unsharded)                        */
    int32_t vocab;        /* V (unsharded), 0 if the layer has no vocab head      */
    int32_t tp_size;      /* t >= 1                                              */
    int32_t tp_rank;      /* r in [0, t)                                         */
    int32_t seq_len;      /* s >= 0                                              */
    int32_t micro_batch;  /* b >= 1; T = b*s                                     */
    int32_t dtype;        /* mtp_dtype of weights and activations                */
    float ln_eps;         /* LayerNorm epsilon (> 0), e.g. 1e-5                   */
} mtp_shard_desc;

/* ---------------------------------------------------------------- LayerNorm
 * y = gamma * (x - mean) * rstd + beta per token, mean and population
 * variance over h, rstd = 1/sqrt(var + eps).  The pages name a fused
 * LayerNorm kernel (page "Megatron-LM 3D parallelism guide", §4.2).  Under
 * the column/row split each rank holds the whole [T,h] input, so the
 * statistics are computed locally with no exchange.
 *   x, y: [T,h] dtype.  gamma, beta: [h] dtype.  mean, rstd: [T] fp32 (out).
 *   amax_parts: nullable, 1024 fp32 (out); when given, receives partial
 *   maxima of |y| as stored, in the form mtp_fp8_amax writes (each part the
 *   maximum over some of y's elements, unused parts 0, so the largest part
 *   is y's amax), for mtp_fp8_quantize of y without a separate amax pass;
 *   bf16 only (MTP_ERR_UNSUPPORTED for an fp32 shard).
 */
int mtp_layernorm(const mtp_shard_desc* desc, const void* x, const void* gamma,
                  const void* beta, void* y, float* mean, float* rstd, float* amax_parts,
                  void* stream);

/* LayerNorm backward.  dy: [T,h] gradient w.r.t. y; x, gamma, mean, rstd as
 * saved by mtp_layernorm.  dres: nullable [T,h] residual-branch gradient that
 * is added to dx (dx = dres + dLN/dx . dy).  dx: [T,h] dtype.  dgamma, dbeta:
 * [h] fp32, overwritten, or incremented when accumulate != 0.  Needs
 * ws_bytes >= mtp_workspace_size(desc, MTP_OP_LAYERNORM_BWD, 0).           */
int mtp_layernorm_bwd(const mtp_shard_desc* desc, const void* dy, const void* x,
                      const void* gamma, const float* mean, const float* rstd,
                      const void* dres, void* dx, float* dgamma, float* dbeta,
                      int accumulate, void* ws, size_t ws_bytes, void* stream);

/* LayerNorm backward of a gradient that arrives as tensor-parallel partials
 * (the column-parallel input gradient of page "Megatron-LM 3D parallelism
 * guide", §2.1: the input reached every rank, so its gradient is the sum of
 * the ranks' partials), in one pass where the width allows:
 *   dy = sum_{i<n} dy_partials[i], accumulated in fp32 in the order
 *   i = 0..n-1 and rounded to dtype exactly as mtp_partial_sum would store
 *   it (a single partial is used as is); then everything as
 *   mtp_layernorm_bwd(dy, ...).  The sum itself is not stored.
 * dy_partials: HOST array of n_partials (1..16) device pointers, [T,h] dtype.
 * amax_parts: nullable, as in mtp_layernorm, of dx.
 * Other arguments, workspace and errors as mtp_layernorm_bwd.                */
int mtp_layernorm_bwd_sum(const mtp_shard_desc* desc, const void* const* dy_partials,
                          int32_t n_partials, const void* x, const void* gamma,
                          const float* mean, const float* rstd, const void* dres, void* dx,
                          float* dgamma, float* dbeta, int accumulate, void* ws,
                          size_t ws_bytes, float* amax_parts, void* stream);

/* ----------------------------------------------- column-parallel linear
 * ColumnParallelLinear with the output left sharded (page "Megatron-LM:
 * NVIDIA large-model training framework", section "Tensor parallelism":
 * gather_output=False; page "Megatron-LM 3D parallelism guide", §2.1).
 *   kind MTP_QKV:   x [T,h], w [3h_l,h], b [3h_l] nullable, y [T,3h_l];
 *                   preact must be NULL.
 *   kind MTP_FC1:   x [T,h], w [f_l,h], b [f_l] nullable; preact [T,f_l]
 *                   receives u = x w^T + b and y [T,f_l] receives GeLU_tanh(u).
 *   kind MTP_VOCAB: x [T,h], w = vocab shard [V_l,h], b [V_l] nullable,
 *                   y = fp32 logits [T,V_l]; preact must be NULL.
 *   kind MTP_FC1_SWIGLU: x [T,h]; w [2f_l,h] holds the rank's gate rows
 *                   (of W1) and up rows (of W3) interleaved in groups of 4:
 *                   rows 8j..8j+3 = gate rows 4j..4j+3, rows 8j+4..8j+7 = up
 *                   rows 4j..4j+3.  b must be NULL.  preact [T,2f_l] receives
 *                   x w^T in that interleaved column order and y [T,f_l]
 *                   receives SiLU(gate) * up, SiLU(z) = z / (1 + e^-z).
 */
int mtp_col_linear_fwd(const mtp_shard_desc* desc, int kind, const void* x, const void* w,
                       const void* b, void* y, void* preact, void* stream);

/* Backward of the column-parallel linear map (pre-activation gradient in):
 *   dy [T,out_l] is the gradient w.r.t. x w^T + b (for MTP_FC1: w.r.t. u,
 *   i.e. GeLU' already applied, see mtp_row_linear_bwd); dtype for QKV and
 *   FC1, dtype for VOCAB (the dlogits written by mtp_vocab_ce_bwd).
 *   dx_partial [T,h] dtype (out): this rank's partial of the input gradient.
 *     The input fed every rank, so the full gradient is the sum of all ranks'
 *     partials (mtp_partial_sum).  Nullable (skipped).
 *   For MTP_FC1_SWIGLU, out_l = 2 f_l in the interleaved order of the
 *   forward's w and preact, dw comes out in that order and db must be NULL.
 *   dw [out_l,h] fp32, db [out_l] fp32, both nullable (skipped): overwritten,
 *     or incremented when accumulate != 0.  Each of dx_partial, dw, db is an
 *     independent product, so one map's backward may be split over calls.
 * Needs ws_bytes >= mtp_workspace_size(desc, MTP_OP_COL_LINEAR_BWD, kind)
 * when db != NULL.                                                           */
int mtp_col_linear_bwd(const mtp_shard_desc* desc, int kind, const void* dy, const void* x,
                       const void* w, void* dx_partial, float* dw, float* db, int accumulate,
                       void* ws, size_t ws_bytes, void* stream);

/* -------------------------------------------------- row-parallel linear
 * RowParallelLinear with an already-sharded input (input_is_parallel=True,
 * same snippet); the output is this rank's partial of the full product.  The
 * pages sum the partials with an all-reduce; here mtp_partial_sum does it.
 *   kind MTP_PROJ: x_local [T,h_l], w [h,h_l];  kind MTP_FC2 and
 *   MTP_FC2_SWIGLU: x_local [T,f_l], w [h,f_l].  partial [T,h] dtype.  No bias: the row-parallel bias
 *   is added once, after the sum (mtp_partial_sum).                          */
int mtp_row_linear_fwd(const mtp_shard_desc* desc, int kind, const void* x_local,
                       const void* w, void* partial, void* stream);

/* Backward of the row-parallel map.
 *   dy [T,h] dtype: gradient w.r.t. the summed output (identical on ranks).
 *   x_local, w: as in forward.
 *   gelu_preact: nullable [T,f_l] (MTP_FC2 only).  When given, x_local was
 *     GeLU_tanh(gelu_preact) and dx_local receives the gradient w.r.t. the
 *     pre-activation, (dy w) * GeLU_tanh'(gelu_preact), ready for
 *     mtp_col_linear_bwd(MTP_FC1).  Otherwise dx_local = dy w.
 *   For MTP_FC2_SWIGLU, gelu_preact is instead the interleaved gate|up
 *     preact [T,2f_l] of mtp_col_linear_fwd(MTP_FC1_SWIGLU); when given,
 *     dx_local [T,2f_l] receives, in the same interleaved order, the
 *     gradients w.r.t. gate, (dy w) * up * SiLU'(gate), and w.r.t. up,
 *     (dy w) * SiLU(gate), ready for mtp_col_linear_bwd(MTP_FC1_SWIGLU).
 *   dx_local [T,in_l] dtype (out), nullable.
 *   dw [h,in_l] fp32 nullable; db [h] fp32 nullable (the row-parallel bias
 *     belongs to one rank: pass it on exactly one).  accumulate as above.
 * Needs ws_bytes >= mtp_workspace_size(desc, MTP_OP_ROW_LINEAR_BWD, kind)
 * when db != NULL.                                                           */
int mtp_row_linear_bwd(const mtp_shard_desc* desc, int kind, const void* dy,
                       const void* x_local, const void* w, const void* gelu_preact,
                       void* dx_local, float* dw, float* db, int accumulate,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- attention
 * Softmax attention over the rank's a_l local heads (the head split of page
 * "Megatron-LM 3D parallelism guide", §2.1; softmax in fp32 as the
 * attention_softmax_in_fp32 flag of §3.2 asks).  Per head n:
 *   S = q_n k_n^T / sqrt(d); key j is visible to query i iff start(i) <= j <= i
 *   where start(i) is the first token of i's sequence; P = softmax(S);
 *   ctx_n = P v_n.
 * Sequences: when cu_seqlens is NULL, the T tokens are micro_batch sequences
 * of seq_len tokens each.  Otherwise cu_seqlens is a device int32 array of
 * n_seqs+1 non-decreasing offsets [0, ..., T] of packed variable-length
 * documents (block-diagonal causal mask); the library trusts its contents
 * (it cannot read device memory before launch).
 *   qkv [T,3h_l] dtype (layout above); ctx [T,h_l] dtype (out);
 *   lse [a_l,T] fp32 (out): natural-log log-sum-exp of each score row;
 *   ctx_amax_parts: nullable, bf16 only (else MTP_ERR_UNSUPPORTED): 1024
 *   fp32 (out) receiving partial maxima of |ctx| as stored in the form
 *   mtp_fp8_amax writes, for mtp_fp8_quantize of ctx without an amax pass.
 */
int mtp_attn_fwd(const mtp_shard_desc* desc, const void* qkv, void* ctx, float* lse,
                 const int32_t* cu_seqlens, int32_t n_seqs, float* ctx_amax_parts,
                 void* stream);

/* Attention backward: given qkv, ctx and lse from mtp_attn_fwd and dctx
 * [T,h_l], writes dqkv [T,3h_l] dtype = [dq | dk | dv] in the qkv layout.
 * Needs ws_bytes >= mtp_workspace_size(desc, MTP_OP_ATTN_BWD, 0) (= two fp32
 * values per local head and token: D = rowsum(dctx * ctx) and the
 * log-sum-exp in base 2).  dqkv_amax_parts: nullable, bf16 only, as
 * ctx_amax_parts of mtp_attn_fwd, of dqkv.                                  */
int mtp_attn_bwd(const mtp_shard_desc* desc, const void* qkv, const void* ctx,
                 const float* lse, const void* dctx, void* dqkv,
                 const int32_t* cu_seqlens, int32_t n_seqs, void* ws, size_t ws_bytes,
                 float* dqkv_amax_parts, void* stream);

/* The same attention backward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): it takes no workspace.  Its two fp32 rows per local
 * head and token live in a fixed 16 MiB device buffer of the library, one
 * per GPU, held until the process ends; the call itself allocates nothing.
 * Needs 8 * a_l * T <= 16 MiB (a_l * T <= 2^21), else MTP_ERR_WORKSPACE
 * before any launch.  The buffer's device address is looked up on the first
 * call on each device (the current device, which must be the stream's).
 * Every call on one GPU shares that buffer and keeps the previous call's
 * contents (nothing in it needs clearing: the call writes every row it
 * reads), so calls that overlap in time on one GPU, on different streams or
 * from different host threads, race; serialise them.  Results are
 * bit-identical to mtp_attn_bwd's (which alone offers the optional amax
 * parts of dqkv).                                                            */
int mtp_attn_bwd_noalloc(const mtp_shard_desc* desc, const void* qkv, const void* ctx,
                         const float* lse, const void* dctx, void* dqkv,
                         const int32_t* cu_seqlens, int32_t n_seqs, void* stream);

/* ---------------------------------------------------------- FP8 GEMMs
 * Forward linear maps with E4M3 operands and one fp32 scale per tensor (FP8
 * among the training precisions of page "Megatron-LM / Megatron Core README
 * digest", §0, and the --enable-fp8 flag of page "Megatron-LM 3D parallelism
 * guide", §5.1; reading: OCP E4M3 without infinities, s = amax / 448), on
 * the FP8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).  bf16 shards
 * only, else MTP_ERR_UNSUPPORTED.
 *
 * mtp_quantize_fp8: x holds n values of the shard dtype, n % 8 == 0; scale
 *   points to 2 fp32 values in device memory: scale[1] receives amax = max
 *   |x|, scale[0] s = amax / 448 (1 when amax is 0); q[i] receives the E4M3
 *   code of round-to-nearest-even(clamp(x[i] / s, -448, 448)), the quotient
 *   correctly rounded in fp32.                                               */
int mtp_quantize_fp8(const mtp_shard_desc* desc, const void* x, int64_t n, uint8_t* q,
                     float* scale, void* stream);

/* mtp_linear_fwd_fp8: y = (x8 w8^T) * x_scale[0] * w_scale[0] (+ b), with x8,
 *   w8 the codes and scales of mtp_quantize_fp8 of the layouts of
 *   mtp_col_linear_fwd / mtp_row_linear_fwd: kind MTP_QKV (x8 [T,h], w8
 *   [3h_l,h], b nullable, y [T,3h_l]), MTP_FC1 (w8 [f_l,h]; preact [T,f_l]
 *   receives u, y GeLU_tanh(u)), MTP_FC1_SWIGLU (w8 [2f_l,h], the codes of
 *   the interleaved gate|up rows of mtp_col_linear_fwd(MTP_FC1_SWIGLU) under
 *   one scale; b NULL; preact [T,2f_l] receives the interleaved gate|up
 *   product, y [T,f_l] SiLU(gate) * up; f_l % 4 == 0), MTP_PROJ (x8 [T,h_l],
 *   w8 [h,h_l], y the partial [T,h], b NULL) or MTP_FC2 / MTP_FC2_SWIGLU (x8
 *   [T,f_l], w8 [h,f_l], b NULL).  y and preact in the shard dtype; the inner
 *   width must be a multiple of 16 (else MTP_ERR_UNSUPPORTED).  amax_parts:
 *   nullable, MTP_FC1 and MTP_FC1_SWIGLU only (else MTP_ERR_INVALID_ARG):
 *   1024 fp32 (out) receiving partial maxima of |y| as stored in the form
 *   mtp_fp8_amax writes, for mtp_fp8_quantize of y without a separate amax
 *   pass.                                                                    */
int mtp_linear_fwd_fp8(const mtp_shard_desc* desc, int kind, const uint8_t* x8,
                       const float* x_scale, const uint8_t* w8, const float* w_scale,
                       const void* b, void* y, void* preact, float* amax_parts, void* stream);

/* FP8 training step: per-tensor scales shared by every shard of a tensor
 * (the ranks of a tensor-parallel group agree on the maximum of their
 * shards' amax), E4M3 codes for activations and weights and E5M2 codes for
 * gradients (reading of the FP8 precision named in README digest §0 and the
 * --enable-fp8 flag of guide §5.1, which give no recipe).  Every FP8 GEMM
 * reads both operands k-major, so the backward takes the transposed codes
 * that mtp_fp8_quantize writes beside the row-major ones.
 *
 * mtp_fp8_amax: amax_parts [1024] fp32 (out) receives partial maxima of |x|
 *   over the n values of x (dtype bf16, n % 8 == 0; 0 where a part saw no
 *   value): max |x| is their maximum.  No atomics; the result is the same
 *   on every call.
 * mtp_fp8_quantize: the codes of x [rows, cols] (bf16, row-major, cols % 8
 *   == 0) in format fmt with s = amax / max_fmt (448 for E4M3, 57344 for
 *   E5M2; 1 when amax is 0), amax the maximum over the n_parts arrays of 1024
 *   partial maxima in amax_parts (a HOST array of device pointers: one per
 *   shard of the tensor, 1 <= n_parts <= 16).  Codes are
 *   round-to-nearest-even(clamp(fl32(x / s), -max, max)).  q [rows, cols]
 *   and/or q_t [cols, rows] (the transpose; nullable, not both NULL) receive
 *   them; scale [1] fp32 (out) receives s.  With n = 0 or rows = 0, x, q
 *   and q_t may be NULL.
 * mtp_linear_bwd_fp8: the gradients of one of the linear maps of kind
 *   (QKV, FC1, FC1_SWIGLU, PROJ, FC2, FC2_SWIGLU; out x in = 3h_l x h,
 *   f_l x h, 2f_l x h (the interleaved gate|up rows), h x h_l, h x f_l,
 *   h x f_l) from FP8 codes:
 *   dx [T, in] dtype (nullable) = (dy8 [T, out] E5M2) (w8_t [in, out] E4M3,
 *     the transposed codes of W)^T * dy_scale * w_scale, times
 *     GeLU_tanh'(preact) for FC2 with preact = u [T, f_l] (the FFN's du);
 *     for FC2_SWIGLU with preact = the interleaved gate|up product
 *     [T, 2f_l], dx [T, 2f_l] instead receives in that order the gradients
 *     w.r.t. gate and up as mtp_row_linear_bwd(MTP_FC2_SWIGLU) defines
 *     them, ready for quantization as one E5M2 tensor;
 *     needs out % 16 == 0;
 *   dw [out, in] fp32 (nullable; += when accumulate) = (dy8_t [out, T] E5M2,
 *     the transposed codes of dy) (x8_t [in, T] E4M3, those of the forward
 *     input)^T * dy_scale * x_scale; needs T % 16 == 0;
 *   dx_amax_parts: nullable, only with dx and preact (FC2's du, or the
 *     interleaved [dgate | dup] of FC2_SWIGLU; else MTP_ERR_INVALID_ARG):
 *     partial maxima of |dx| as in mtp_linear_fwd_fp8.
 *   Scales are [1] fp32 device values as written by mtp_fp8_quantize.     */
int mtp_fp8_amax(const mtp_shard_desc* desc, const void* x, int64_t n, float* amax_parts,
                 void* stream);
int mtp_fp8_quantize(const mtp_shard_desc* desc, int fmt, const void* x, int64_t rows,
                     int64_t cols, const float* const* amax_parts, int32_t n_parts, uint8_t* q,
                     uint8_t* q_t, float* scale, void* stream);
int mtp_linear_bwd_fp8(const mtp_shard_desc* desc, int kind, const uint8_t* dy8,
                       const uint8_t* dy8_t, const float* dy_scale, const uint8_t* w8_t,
                       const float* w_scale, const uint8_t* x8_t, const float* x_scale,
                       const void* preact, void* dx, float* dw, int accumulate,
                       float* dx_amax_parts, void* stream);

/* ------------------------------------------ context-parallel attention
 * The sequence split into chunks whose attention runs block pair by block
 * pair, each partial result merged through its log-sum-exp (context
 * parallelism, named among the parallel strategies in §4 of page
 * "Megatron-LM / Megatron Core README digest"; the pages give no algorithm,
 * the chunked, log-sum-exp merged form is the plain reading of splitting
 * the sequence dimension of attention; here all chunks are computed on one
 * device, one pair per call).  bf16 shards, micro_batch 1, else
 * MTP_ERR_UNSUPPORTED.  The tokens are one sequence when cu_seqlens is NULL,
 * else the packed documents of cu_seqlens (n_seqs+1 device offsets, as for
 * mtp_attn_fwd; the chunks need not align with the documents): a query then
 * sees only the keys of its own document, and a query with no visible key
 * in a block gets ctx 0 and lse -inf from mtp_attn_fwd_block, which
 * mtp_attn_merge treats as an empty part.
 *
 * mtp_attn_fwd_block: queries at rows [q_lo, q_hi) of qkv attend to the keys
 *   at rows [k_lo, k_hi) with the causal mask of their absolute positions:
 *   either the diagonal block (q_lo == k_lo, q_hi == k_hi) or a block whose
 *   keys all precede the queries (k_hi <= q_lo), else MTP_ERR_INVALID_ARG.
 *   Writes rows [q_lo, q_hi) of ctx [T,h_l] and columns [q_lo, q_hi) of lse
 *   [a_l,T] (natural log of each row's sum of exp(score)) and nothing else. */
int mtp_attn_fwd_block(const mtp_shard_desc* desc, const void* qkv, int64_t q_lo, int64_t q_hi,
                       int64_t k_lo, int64_t k_hi, void* ctx, float* lse,
                       const int32_t* cu_seqlens, int32_t n_seqs, void* stream);

/* mtp_attn_merge: rows [row_lo, row_hi) of (ctx, lse) become the attention
 *   over the union of the key sets of (ctx, lse) and (ctx_part, lse_part),
 *   two results of mtp_attn_fwd_block for the same queries and disjoint keys:
 *   lse = log(e^lse + e^lse_part), ctx = (e^lse ctx + e^lse_part ctx_part) /
 *   e^lse_new, per row and head.  In place on (ctx, lse).  A row whose
 *   lse_part is -inf is left unchanged.                                     */
int mtp_attn_merge(const mtp_shard_desc* desc, void* ctx, float* lse, const void* ctx_part,
                   const float* lse_part, int64_t row_lo, int64_t row_hi, void* stream);

/* mtp_attn_bwd_block: the backward of one block pair given the merged ctx and
 *   lse of the queries (the whole rows' softmax): writes (accumulate == 0) or
 *   adds to (accumulate != 0) the dQ columns of dqkv at the query rows and
 *   the dK, dV columns at the key rows; q_hi - q_lo must equal k_hi - k_lo.
 *   Needs the workspace of mtp_attn_bwd.                                    */
int mtp_attn_bwd_block(const mtp_shard_desc* desc, const void* qkv, const void* ctx,
                       const float* lse, const void* dctx, void* dqkv, int64_t q_lo,
                       int64_t q_hi, int64_t k_lo, int64_t k_hi, int accumulate,
                       const int32_t* cu_seqlens, int32_t n_seqs, void* ws, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------ partial sum
 * The sum that the pages perform with a tensor-parallel all-reduce (page
 * "Megatron-LM 3D parallelism guide", §2.1: the row-split output projection's
 * per-rank shards are summed into the complete output).  Here all partials
 * are on one device:
 *   out = sum_{i<n} partials[i] + bias + residual, accumulated in fp32 in
 *   the fixed order i = 0..n-1, then bias, then residual.
 * partials: HOST array of n_partials (1..16) device pointers, each [T,h]
 * dtype.  bias [h] and residual [T,h] are nullable.  out [T,h] dtype (may
 * alias residual or partials[i]).                                            */
int mtp_partial_sum(const mtp_shard_desc* desc, const void* const* partials,
                    int32_t n_partials, const void* bias, const void* residual, void* out,
                    void* stream);

/* The partial sum followed by the LayerNorm of its result (the sum that
 * completes the row-parallel projection, §2.1 of page "Megatron-LM 3D
 * parallelism guide", feeding the next pre-LN LayerNorm; the same page, §4.2,
 * fuses LayerNorm with its neighbours), in one pass where the width allows:
 *   out = exactly what mtp_partial_sum(partials, n_partials, bias, residual)
 *   stores; then ln_out, mean, rstd = exactly what mtp_layernorm(out, gamma,
 *   beta, amax_parts) writes.  Arguments as those two calls; out may alias
 *   residual or a partial.                                                   */
int mtp_partial_sum_layernorm(const mtp_shard_desc* desc, const void* const* partials,
                              int32_t n_partials, const void* bias, const void* residual,
                              void* out, const void* gamma, const void* beta, void* ln_out,
                              float* mean, float* rstd, float* amax_parts, void* stream);

/* ------------------------------------------------- vocab-parallel CE head
 * Cross-entropy over a vocabulary split across ranks (VocabParallelEmbedding,
 * page "Megatron-LM: NVIDIA large-model training framework", section
 * "Tensor parallelism"; vocab 131072 at seq 4096 in page "Megatron-LM /
 * Megatron Core README digest", §5).  Rank r owns ids [r*V_l, (r+1)*V_l).
 *
 * Stats of one shard: for every token, m = max_j z_j, s = sum_j exp(z_j - m)
 * over the shard's logits, and z_tgt = the target's logit if this shard owns
 * the target id, else 0.  logits [T,V_l] fp32; targets [T] int32 global ids
 * in [0, V) (checked on device: an out-of-range id yields NaN loss).
 * m, s, z_tgt: [T] fp32 (out).                                               */
int mtp_vocab_ce_stats(const mtp_shard_desc* desc, const float* logits,
                       const int32_t* targets, float* m, float* s, float* z_tgt,
                       void* stream);

/* Combine the t shards' stats: M = max_r m_r, S = sum_r s_r exp(m_r - M),
 * loss_t = log S + M - sum_r z_tgt_r; loss_mean = mean_t loss_t.
 * m, s, z_tgt: HOST arrays of n_ranks device pointers ([T] fp32 each).
 * M, S, loss: [T] fp32 (out); loss_mean: [1] fp32 (out, nullable).           */
int mtp_vocab_ce_combine(const mtp_shard_desc* desc, const float* const* m,
                         const float* const* s, const float* const* z_tgt, int32_t n_ranks,
                         float* M, float* S, float* loss, float* loss_mean, void* stream);

/* Gradient of dloss_scale * sum_t loss_t w.r.t. this shard's logits:
 * dlogits = dloss_scale * (exp(z - M)/S - [j == target]).  For the mean
 * loss pass dloss_scale = 1/T.  dlogits [T,V_l] dtype (out).  A token whose
 * target id lies outside [0, V) gets a NaN row (its loss is NaN too).      */
int mtp_vocab_ce_bwd(const mtp_shard_desc* desc, const float* logits, const int32_t* targets,
                     const float* M, const float* S, float dloss_scale, void* dlogits,
                     void* stream);

/* ------------------------------------------------------------- utilities */
/* Bytes of `ws` that operation `op` needs for this shard; `kind` selects
 * the linear map for MTP_OP_COL_LINEAR_BWD / MTP_OP_ROW_LINEAR_BWD.
 * Returns 0 when none is needed, and 0 for an invalid desc.                 */
size_t mtp_workspace_size(const mtp_shard_desc* desc, int op, int kind);

/* Static string for a status code. */
const char* mtp_status_string(int status);

/* MTP_VERSION of the built library. */
int mtp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MTP_H */
