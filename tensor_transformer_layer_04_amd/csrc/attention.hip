// Softmax attention over the rank's local heads, forward and backward.
//
// The head split needs no exchange between ranks (page "Megatron-LM 3D
// parallelism guide", §2.1): each rank attends over its own a_l heads.  The
// softmax runs in fp32 (the attention_softmax_in_fp32 flag, §3.2 of the same
// page).  Key j is visible to query i iff start(i) <= j <= i, start(i) being
// the first token of i's sequence (fixed-length micro-batch or packed
// variable-length documents given by cu_seqlens).
//
// This file holds the fp32 path (plain SIMT kernels, one query or key per
// workgroup), the backward preprocess D = rowsum(dO * O) shared by both
// paths, and the launchers.  The bf16 path is the MFMA kernels of
// attention_fwd.hip and attention_bwd.hip.
#include "common.h"
#include "kernels.h"

namespace mtp {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
  const void* qkv; int64_t ld;      // [T, 3*hl]
  void* ctx;                        // [T, hl]
  float* lse;                       // [heads, T] natural log
  const void* dctx;                 // [T, hl]
  void* dqkv;                       // [T, 3*hl]
  float* delta;                     // [heads, T]
  float* amax;                      // amax parts of dqkv, zeroed here (nullable)
  const int32_t* cu; int n_seqs;
  int T; int seq_len; int heads; int hl;
  float scale;                      // 1/sqrt(D)
  float scale_log2;                 // log2(e)/sqrt(D)
};

__device__ __forceinline__ int seq_index(const AttnParams& p, int i) {
  int lo = 0, hi = p.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}
__device__ __forceinline__ int seq_start(const AttnParams& p, int i) {
  if (!p.cu) return (i / p.seq_len) * p.seq_len;
  return p.cu[seq_index(p, i)];
}
__device__ __forceinline__ int seq_end(const AttnParams& p, int i) {
  if (!p.cu) return min(p.T, (i / p.seq_len + 1) * p.seq_len);
  return p.cu[seq_index(p, i) + 1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// -------------------------------------------------- backward preprocess
// delta[n][i] = sum_d dctx[i, n*D + d] * ctx[i, n*D + d]  (= rowsum(P * dP)),
// and (bf16 path) lse2[n][i] = lse[n][i] * log2(e) right after delta in the
// workspace, so the MFMA passes get exp(S - lse) as exp2(S*scale*log2e - lse2).
// Rows [row_lo, row_lo + rows) only: the query rows of the block being
// differentiated (all T rows for the whole attention).
template <typename T>
__global__ void __launch_bounds__(256) attn_delta_kernel(AttnParams p, int D, int row_lo,
                                                         int rows) {
  const int per_row = D / 8;                 // threads per (token, head)
  const int pairs_per_block = 256 / per_row;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * pairs_per_block + threadIdx.x / per_row;
  const int c = threadIdx.x % per_row;
  // the backward kernel that follows raises these slots to the partial
  // maxima of |dqkv|
  if (p.amax && blockIdx.x == 0)
    for (int k = threadIdx.x; k < kAmaxParts; k += 256) p.amax[k] = 0.0f;
  float acc = 0.0f;
  int64_t i = 0;
  int n = 0;
  if (pair < static_cast<int64_t>(rows) * p.heads) {
    i = row_lo + pair / p.heads;
    n = static_cast<int>(pair % p.heads);
    float a[8], b[8];
    load8(static_cast<const T*>(p.dctx) + i * p.hl + n * D + c * 8, a);
    load8(static_cast<const T*>(p.ctx) + i * p.hl + n * D + c * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += a[e] * b[e];
  }
  for (int o = per_row / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (c == 0 && pair < static_cast<int64_t>(rows) * p.heads) {
    const int64_t at = static_cast<int64_t>(n) * p.T + i;
    p.delta[at] = acc;
    if (sizeof(T) == 2) p.delta[static_cast<int64_t>(p.heads) * p.T + at] = p.lse[at] * kLog2e;
  }
}

// row max and sum, pass 2 accumulates P v in chunks of 64 keys via LDS.
__global__ void __launch_bounds__(64) attn_fwd_f32(AttnParams p, int D) {
  __shared__ float pr[64];
  const int T = p.T;
  const int i = blockIdx.x / p.heads, n = blockIdx.x % p.heads;
  const int lane = threadIdx.x;
  const float* qkv = static_cast<const float*>(p.qkv);
  const float* q = qkv + static_cast<int64_t>(i) * p.ld + n * D;
  const float* kb = qkv + p.hl + n * D;
  const float* vb = qkv + 2 * p.hl + n * D;
  const int j_lo = seq_start(p, i), j_hi = i + 1;
  float m = -INFINITY;
  for (int j = j_lo + lane; j < j_hi; j += 64) {
    const float* k = kb + static_cast<int64_t>(j) * p.ld;
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = fmaf(q[d], k[d], s);
    m = fmaxf(m, s * p.scale);
  }
  m = warp_max(m);
  float l = 0.0f;
  for (int j = j_lo + lane; j < j_hi; j += 64) {
    const float* k = kb + static_cast<int64_t>(j) * p.ld;
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = fmaf(q[d], k[d], s);
    l += __expf(s * p.scale - m);
  }
  l = warp_sum(l);
  float acc0 = 0.0f, acc1 = 0.0f;  // d = lane, lane + 64
  for (int c0 = j_lo; c0 < j_hi; c0 += 64) {
    const int j = c0 + lane;
    float pj = 0.0f;
    if (j < j_hi) {
      const float* k = kb + static_cast<int64_t>(j) * p.ld;
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = fmaf(q[d], k[d], s);
      pj = __expf(s * p.scale - m) / l;
    }
    __syncthreads();
    pr[lane] = pj;
    __syncthreads();
    const int cn = min(64, j_hi - c0);
    for (int jj = 0; jj < cn; ++jj) {
      const float* v = vb + static_cast<int64_t>(c0 + jj) * p.ld;
      if (lane < D) acc0 = fmaf(pr[jj], v[lane], acc0);
      if (lane + 64 < D) acc1 = fmaf(pr[jj], v[lane + 64], acc1);
    }
  }
  float* out = static_cast<float*>(p.ctx) + static_cast<int64_t>(i) * p.hl + n * D;
  if (lane < D) out[lane] = acc0;
  if (lane + 64 < D) out[lane + 64] = acc1;
  if (lane == 0) p.lse[static_cast<int64_t>(n) * T + i] = m + __logf(l);
}

// dQ: one wave per (query, head); dS for 64 keys at a time via LDS.
__global__ void __launch_bounds__(64) attn_dq_f32(AttnParams p, int D) {
  __shared__ float dsh[64];
  const int T = p.T;
  const int i = blockIdx.x / p.heads, n = blockIdx.x % p.heads;
  const int lane = threadIdx.x;
  const float* qkv = static_cast<const float*>(p.qkv);
  const float* q = qkv + static_cast<int64_t>(i) * p.ld + n * D;
  const float* kb = qkv + p.hl + n * D;
  const float* vb = qkv + 2 * p.hl + n * D;
  const float* dO = static_cast<const float*>(p.dctx) + static_cast<int64_t>(i) * p.hl + n * D;
  const float lse = p.lse[static_cast<int64_t>(n) * T + i];
  const float dl = p.delta[static_cast<int64_t>(n) * T + i];
  const int j_lo = seq_start(p, i), j_hi = i + 1;
  float acc0 = 0.0f, acc1 = 0.0f;
  for (int c0 = j_lo; c0 < j_hi; c0 += 64) {
    const int j = c0 + lane;
    float ds = 0.0f;
    if (j < j_hi) {
      const float* k = kb + static_cast<int64_t>(j) * p.ld;
      const float* v = vb + static_cast<int64_t>(j) * p.ld;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) { s = fmaf(q[d], k[d], s); dp = fmaf(dO[d], v[d], dp); }
      const float pe = __expf(s * p.scale - lse);
      ds = pe * (dp - dl);
    }
    __syncthreads();
    dsh[lane] = ds;
    __syncthreads();
    const int cn = min(64, j_hi - c0);
    for (int jj = 0; jj < cn; ++jj) {
      const float* k = kb + static_cast<int64_t>(c0 + jj) * p.ld;
      if (lane < D) acc0 = fmaf(dsh[jj], k[lane], acc0);
      if (lane + 64 < D) acc1 = fmaf(dsh[jj], k[lane + 64], acc1);
    }
  }
  float* out = static_cast<float*>(p.dqkv) + static_cast<int64_t>(i) * p.ld + n * D;
  if (lane < D) out[lane] = acc0 * p.scale;
  if (lane + 64 < D) out[lane + 64] = acc1 * p.scale;
}

// dK, dV: one wave per (key, head); P and dS for 64 queries at a time.
__global__ void __launch_bounds__(64) attn_dkv_f32(AttnParams p, int D) {
  __shared__ float psh[64], dsh[64];
  const int T = p.T;
  const int j = blockIdx.x / p.heads, n = blockIdx.x % p.heads;
  const int lane = threadIdx.x;
  const float* qkv = static_cast<const float*>(p.qkv);
  const float* k = qkv + static_cast<int64_t>(j) * p.ld + p.hl + n * D;
  const float* v = qkv + static_cast<int64_t>(j) * p.ld + 2 * p.hl + n * D;
  const float* qb = qkv + n * D;
  const float* dob = static_cast<const float*>(p.dctx) + n * D;
  const int i_lo = j, i_hi = seq_end(p, j);
  float dk0 = 0.0f, dk1 = 0.0f, dv0 = 0.0f, dv1 = 0.0f;
  for (int c0 = i_lo; c0 < i_hi; c0 += 64) {
    const int i = c0 + lane;
    float pe = 0.0f, ds = 0.0f;
    if (i < i_hi) {
      const float* q = qb + static_cast<int64_t>(i) * p.ld;
      const float* dO = dob + static_cast<int64_t>(i) * p.hl;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) { s = fmaf(q[d], k[d], s); dp = fmaf(dO[d], v[d], dp); }
      pe = __expf(s * p.scale - p.lse[static_cast<int64_t>(n) * T + i]);
      ds = pe * (dp - p.delta[static_cast<int64_t>(n) * T + i]);
    }
    __syncthreads();
    psh[lane] = pe;
    dsh[lane] = ds;
    __syncthreads();
    const int cn = min(64, i_hi - c0);
    for (int ii = 0; ii < cn; ++ii) {
      const float* q = qb + static_cast<int64_t>(c0 + ii) * p.ld;
      const float* dO = dob + static_cast<int64_t>(c0 + ii) * p.hl;
      if (lane < D) { dv0 = fmaf(psh[ii], dO[lane], dv0); dk0 = fmaf(dsh[ii], q[lane], dk0); }
      if (lane + 64 < D) { dv1 = fmaf(psh[ii], dO[lane + 64], dv1); dk1 = fmaf(dsh[ii], q[lane + 64], dk1); }
    }
  }
  float* out = static_cast<float*>(p.dqkv) + static_cast<int64_t>(j) * p.ld + n * D;
  if (lane < D) { out[p.hl + lane] = dk0 * p.scale; out[2 * p.hl + lane] = dv0; }
  if (lane + 64 < D) { out[p.hl + lane + 64] = dk1 * p.scale; out[2 * p.hl + lane + 64] = dv1; }
}

// Merge of two partial attention results of the same queries over disjoint
// key sets (their union is the keys the query sees): with weights
// w = e^(lse - max(lse_a, lse_b)), ctx = (w_a ctx_a + w_b ctx_b) / (w_a + w_b)
// and lse = max + log(w_a + w_b) (natural log).  One thread per (row, head)
// reads both partials of its row and head before writing either output, so
// the accumulated pair may be updated in place.
__global__ void __launch_bounds__(256) attn_merge_kernel(bf16_t* ctx, float* lse,
                                                         const bf16_t* ctx_p, const float* lse_p,
                                                         int T, int hl, int heads, int D,
                                                         int row_lo, int rows) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(rows) * heads) return;
  const int r = row_lo + static_cast<int>(idx / heads), h = static_cast<int>(idx % heads);
  const int64_t li = static_cast<int64_t>(h) * T + r;
  const float la = lse[li], lb = lse_p[li];
  // an empty part (no visible key: lse -inf, ctx 0) leaves the row as it is
  if (lb == -INFINITY) return;
  const float m = fmaxf(la, lb);
  const float wa = __expf(la - m), wb = __expf(lb - m);
  const float inv = 1.0f / (wa + wb);
  bf16_t* o = ctx + static_cast<int64_t>(r) * hl + h * D;
  const bf16_t* q = ctx_p + static_cast<int64_t>(r) * hl + h * D;
  for (int c = 0; c < D; c += 8) {
    float a[8], b[8];
    load8(o + c, a);
    load8(q + c, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (wa * a[e] + wb * b[e]) * inv;
    store8(o + c, a);
  }
  lse[li] = m + __logf(wa + wb);
}

AttnParams make_params(const AttnDesc& a) {
  AttnParams p{};
  p.qkv = a.qkv; p.ld = 3LL * a.heads * a.head_dim;
  p.ctx = a.ctx; p.lse = a.lse; p.dctx = a.dctx; p.dqkv = a.dqkv; p.delta = a.delta;
  p.amax = a.amax;
  p.cu = a.cu_seqlens; p.n_seqs = a.n_seqs;
  p.T = static_cast<int>(a.T); p.seq_len = a.seq_len; p.heads = a.heads;
  p.hl = a.heads * a.head_dim;
  p.scale = 1.0f / sqrtf(static_cast<float>(a.head_dim));
  p.scale_log2 = p.scale * kLog2e;
  return p;
}

}  // namespace

hipError_t attn_fwd(bool bf16, const AttnDesc& a, hipStream_t s) {
  if (a.amax && !bf16) return hipErrorInvalidValue;
  if (a.T == 0 || a.heads == 0) return a.amax ? fp8_amax(a.ctx, 0, a.amax, s) : hipSuccess;
  const AttnParams p = make_params(a);
  if (bf16) {
    return attn_fwd_bf16_mfma(a, s);
  } else {
    hipLaunchKernelGGL(attn_fwd_f32, dim3(static_cast<unsigned>(a.T * a.heads)), dim3(64), 0, s,
                       p, a.head_dim);
  }
  return hipGetLastError();
}

hipError_t attn_merge(const AttnDesc& a, const void* ctx_part, const float* lse_part,
                      int64_t row_lo, int64_t row_hi, hipStream_t s) {
  const int64_t rows = row_hi - row_lo;
  if (rows <= 0 || a.heads == 0) return hipSuccess;
  const int64_t n = rows * a.heads;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, static_cast<bf16_t*>(a.ctx), a.lse,
                     static_cast<const bf16_t*>(ctx_part), lse_part, static_cast<int>(a.T),
                     a.heads * a.head_dim, a.heads, a.head_dim, static_cast<int>(row_lo),
                     static_cast<int>(rows));
  return hipGetLastError();
}

hipError_t attn_bwd(bool bf16, const AttnDesc& a, hipStream_t s) {
  if (a.amax && (!bf16 || a.accumulate)) return hipErrorInvalidValue;
  if (a.T == 0 || a.heads == 0) return a.amax ? fp8_amax(a.dqkv, 0, a.amax, s) : hipSuccess;
  const AttnParams p = make_params(a);
  const int per_row = a.head_dim / 8;
  // D and lse*log2(e) are read only at the query rows of the range
  const int row_lo = static_cast<int>(a.q_lo);
  const int rows = static_cast<int>((a.q_hi < 0 ? a.T : a.q_hi) - a.q_lo);
  if (rows <= 0) return a.amax ? fp8_amax(a.dqkv, 0, a.amax, s) : hipSuccess;
  const int64_t pairs = static_cast<int64_t>(rows) * a.heads;
  const int pairs_per_block = 256 / per_row;
  const dim3 dgrid(static_cast<unsigned>((pairs + pairs_per_block - 1) / pairs_per_block));
  if (bf16)
    hipLaunchKernelGGL(attn_delta_kernel<bf16_t>, dgrid, dim3(256), 0, s, p, a.head_dim, row_lo,
                       rows);
  else
    hipLaunchKernelGGL(attn_delta_kernel<float>, dgrid, dim3(256), 0, s, p, a.head_dim, row_lo,
                       rows);
  if (bf16) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return attn_bwd_bf16_mfma(a, s);
  } else {
    const dim3 grid(static_cast<unsigned>(a.T * a.heads));
    hipLaunchKernelGGL(attn_dkv_f32, grid, dim3(64), 0, s, p, a.head_dim);
    hipLaunchKernelGGL(attn_dq_f32, grid, dim3(64), 0, s, p, a.head_dim);
  }
  return hipGetLastError();
}

}  // namespace mtp
