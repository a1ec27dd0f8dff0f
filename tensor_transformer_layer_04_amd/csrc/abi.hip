// C ABI of libmtp (declared in include/mtp.h): argument validation, then
// dispatch to the kernels.  Validation completes before anything is
// enqueued; no entry point allocates memory or keeps state.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"
#include "mtp.h"

namespace {

using mtp::GemmDesc;

struct Shard {
  int64_t T;
  int h, a, d, t, r, hl, al, fl;
  int64_t V, Vl;
  bool bf16;
  int esize;
  float eps;
};

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned(p); }

int check_desc(const mtp_shard_desc* desc, Shard* s) {
  if (!desc) return MTP_ERR_INVALID_ARG;
  const mtp_shard_desc& d = *desc;
  if (d.hidden <= 0 || d.heads <= 0 || d.ffn < 0 || d.vocab < 0 || d.tp_size < 1 ||
      d.tp_rank < 0 || d.tp_rank >= d.tp_size || d.seq_len < 0 || d.micro_batch < 1)
    return MTP_ERR_INVALID_ARG;
  if (!(d.ln_eps > 0.0f) || !isfinite(d.ln_eps)) return MTP_ERR_INVALID_ARG;
  if (d.dtype != MTP_F32 && d.dtype != MTP_BF16) return MTP_ERR_UNSUPPORTED;
  if (d.hidden % d.heads != 0) return MTP_ERR_INVALID_ARG;
  // hidden and heads must split evenly over the TP ranks; so must the FFN
  // and the vocabulary.
  if (d.heads % d.tp_size != 0 || d.hidden % d.tp_size != 0) return MTP_ERR_INVALID_ARG;
  if (d.ffn % d.tp_size != 0 || d.vocab % d.tp_size != 0) return MTP_ERR_INVALID_ARG;
  const int hd = d.hidden / d.heads;
  if (hd != 64 && hd != 128) return MTP_ERR_UNSUPPORTED;
  if ((d.ffn / d.tp_size) % 8 != 0 || (d.vocab / d.tp_size) % 8 != 0) return MTP_ERR_UNSUPPORTED;
  if (d.hidden > 16384) return MTP_ERR_UNSUPPORTED;
  const int64_t T = static_cast<int64_t>(d.seq_len) * d.micro_batch;
  if (T > (static_cast<int64_t>(1) << 30)) return MTP_ERR_UNSUPPORTED;
  s->T = T;
  s->h = d.hidden; s->a = d.heads; s->d = hd; s->t = d.tp_size; s->r = d.tp_rank;
  s->hl = d.hidden / d.tp_size; s->al = d.heads / d.tp_size; s->fl = d.ffn / d.tp_size;
  s->V = d.vocab; s->Vl = d.vocab / d.tp_size;
  s->bf16 = d.dtype == MTP_BF16;
  s->esize = s->bf16 ? 2 : 4;
  s->eps = d.ln_eps;
  return MTP_OK;
}

// Operands that the kernels address through 32-bit buffer resources (the
// GEMM operands, the attention inputs, statistics and workspace) must each
// span less than 2 GiB.  Each entry point checks the ones it touches before
// it enqueues anything, so an over-large shard returns MTP_ERR_UNSUPPORTED
// with nothing launched.
constexpr int64_t kMaxBufferBytes = int64_t{1} << 31;
bool fits(int64_t rows, int64_t cols, int64_t esize) {
  return rows * cols * esize < kMaxBufferBytes;
}
bool attn_fits(const Shard& s) {
  return fits(s.T, 3LL * s.hl, s.esize) && fits(s.T, s.hl, s.esize) && fits(s.T, s.al, 4);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MTP_OK : MTP_ERR_HIP; }

hipError_t gemm(const Shard& s, const GemmDesc& g, hipStream_t st) {
  return s.bf16 ? mtp::gemm_bf16(g, st) : mtp::gemm_f32(g, st);
}

// Output width of a column-parallel kind, 0 for anything else.
int64_t col_out(const Shard& s, int kind) {
  switch (kind) {
    case MTP_QKV: return 3LL * s.hl;
    case MTP_FC1: return s.fl;
    case MTP_FC1_SWIGLU: return 2LL * s.fl;
    case MTP_VOCAB: return s.Vl;
    default: return 0;
  }
}
// Input width of a row-parallel kind, 0 for anything else.
int64_t row_in(const Shard& s, int kind) {
  switch (kind) {
    case MTP_PROJ: return s.hl;
    case MTP_FC2: return s.fl;
    case MTP_FC2_SWIGLU: return s.fl;
    default: return 0;
  }
}

// A (query rows, key rows) block of the context-parallel entry points: the
// diagonal block of one chunk, or keys entirely before the queries.  The
// path is the bf16 MFMA one, over one sequence (micro_batch 1).
int check_block(const Shard& s, const mtp_shard_desc* desc, int64_t q_lo, int64_t q_hi,
                int64_t k_lo, int64_t k_hi) {
  if (!s.bf16 || desc->micro_batch != 1) return MTP_ERR_UNSUPPORTED;
  if (q_lo < 0 || q_hi > s.T || q_lo >= q_hi || k_lo < 0 || k_hi > s.T || k_lo >= k_hi)
    return MTP_ERR_INVALID_ARG;
  const bool diagonal = q_lo == k_lo && q_hi == k_hi;
  const bool before = k_hi <= q_lo;
  return (diagonal || before) ? MTP_OK : MTP_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

int mtp_version(void) { return MTP_VERSION; }

const char* mtp_status_string(int status) {
  switch (status) {
    case MTP_OK: return "MTP_OK";
    case MTP_ERR_INVALID_ARG: return "MTP_ERR_INVALID_ARG: invalid argument";
    case MTP_ERR_UNSUPPORTED: return "MTP_ERR_UNSUPPORTED: valid but unsupported shape or dtype";
    case MTP_ERR_WORKSPACE: return "MTP_ERR_WORKSPACE: workspace missing or too small";
    case MTP_ERR_HIP: return "MTP_ERR_HIP: a HIP launch failed";
    default: return "unknown mtp status";
  }
}

size_t mtp_workspace_size(const mtp_shard_desc* desc, int op, int kind) {
  Shard s;
  if (check_desc(desc, &s) != MTP_OK) return 0;
  switch (op) {
    case MTP_OP_LAYERNORM_BWD: return mtp::layernorm_bwd_ws_bytes(s.T, s.h, s.bf16);
    case MTP_OP_COL_LINEAR_BWD: {
      const int64_t n = col_out(s, kind);
      return n > 0 ? mtp::column_sum_ws_bytes(s.T, n) : 0;
    }
    case MTP_OP_ROW_LINEAR_BWD:
      return row_in(s, kind) > 0 ? mtp::column_sum_ws_bytes(s.T, s.h) : 0;
    case MTP_OP_ATTN_BWD: return static_cast<size_t>(s.al) * s.T * sizeof(float) * 2;
    default: return 0;
  }
}

int mtp_layernorm(const mtp_shard_desc* desc, const void* x, const void* gamma, const void* beta,
                  void* y, float* mean, float* rstd, float* amax_parts, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(x) || !ok_ptr(gamma) || !ok_ptr(beta) || !ok_ptr(y) || !ok_ptr(mean) ||
      !ok_ptr(rstd) || !ok_opt(amax_parts))
    return MTP_ERR_INVALID_ARG;
  if (amax_parts && !s.bf16) return MTP_ERR_UNSUPPORTED;
  return hip_status(mtp::layernorm_fwd(s.bf16, x, gamma, beta, y, mean, rstd, s.T, s.h, s.eps,
                                       amax_parts, static_cast<hipStream_t>(stream)));
}

int mtp_layernorm_bwd(const mtp_shard_desc* desc, const void* dy, const void* x, const void* gamma,
                      const float* mean, const float* rstd, const void* dres, void* dx,
                      float* dgamma, float* dbeta, int accumulate, void* ws, size_t ws_bytes,
                      void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(dy) || !ok_ptr(x) || !ok_ptr(gamma) || !ok_ptr(mean) || !ok_ptr(rstd) ||
      !ok_opt(dres) || !ok_ptr(dx) || !ok_ptr(dgamma) || !ok_ptr(dbeta))
    return MTP_ERR_INVALID_ARG;
  const size_t need = mtp::layernorm_bwd_ws_bytes(s.T, s.h, s.bf16);
  if (need > 0 && (ws == nullptr || !aligned(ws) || ws_bytes < need)) return MTP_ERR_WORKSPACE;
  return hip_status(mtp::layernorm_bwd(s.bf16, dy, x, gamma, mean, rstd, dres, dx, dgamma, dbeta,
                                       accumulate != 0, s.T, s.h, ws,
                                       static_cast<hipStream_t>(stream)));
}

int mtp_layernorm_bwd_sum(const mtp_shard_desc* desc, const void* const* dy_partials,
                          int32_t n_partials, const void* x, const void* gamma,
                          const float* mean, const float* rstd, const void* dres, void* dx,
                          float* dgamma, float* dbeta, int accumulate, void* ws,
                          size_t ws_bytes, float* amax_parts, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!dy_partials || n_partials < 1 || n_partials > mtp::kMaxPartials) return MTP_ERR_INVALID_ARG;
  for (int i = 0; i < n_partials; ++i)
    if (!ok_ptr(dy_partials[i])) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(x) || !ok_ptr(gamma) || !ok_ptr(mean) || !ok_ptr(rstd) || !ok_opt(dres) ||
      !ok_ptr(dx) || !ok_ptr(dgamma) || !ok_ptr(dbeta) || !ok_opt(amax_parts))
    return MTP_ERR_INVALID_ARG;
  if (amax_parts && !s.bf16) return MTP_ERR_UNSUPPORTED;
  const size_t need = mtp::layernorm_bwd_ws_bytes(s.T, s.h, s.bf16);
  if (need > 0 && (ws == nullptr || !aligned(ws) || ws_bytes < need)) return MTP_ERR_WORKSPACE;
  return hip_status(mtp::layernorm_bwd_sum(s.bf16, dy_partials, n_partials, x, gamma, mean, rstd,
                                           dres, dx, dgamma, dbeta, accumulate != 0, s.T, s.h,
                                           ws, amax_parts, static_cast<hipStream_t>(stream)));
}

int mtp_col_linear_fwd(const mtp_shard_desc* desc, int kind, const void* x, const void* w,
                       const void* b, void* y, void* preact, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  const int64_t n = col_out(s, kind);
  if (n <= 0) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(x) || !ok_ptr(w) || !ok_opt(b) || !ok_ptr(y)) return MTP_ERR_INVALID_ARG;
  const bool swiglu = kind == MTP_FC1_SWIGLU;
  if ((kind == MTP_FC1 || swiglu) ? !ok_ptr(preact) : preact != nullptr) return MTP_ERR_INVALID_ARG;
  if (swiglu && b != nullptr) return MTP_ERR_INVALID_ARG;
  if (!fits(s.T, s.h, s.esize) || !fits(n, s.h, s.esize)) return MTP_ERR_UNSUPPORTED;
  GemmDesc g{};
  g.A = x; g.lda = s.h; g.a_kmajor = true;
  g.B = w; g.ldb = s.h; g.b_kmajor = true;
  g.M = static_cast<int>(s.T); g.N = static_cast<int>(n); g.K = s.h;
  g.C = y; g.ldc = swiglu ? s.fl : n; g.bias = b;
  g.aux = preact; g.ld_aux = n;
  g.epi = kind == MTP_FC1 ? mtp::kEpiGelu : swiglu ? mtp::kEpiSwiGLU
        : kind == MTP_VOCAB ? mtp::kEpiF32 : mtp::kEpiStore;
 
  return hip_status(gemm(s, g, static_cast<hipStream_t>(stream)));
}

int mtp_col_linear_bwd(const mtp_shard_desc* desc, int kind, const void* dy, const void* x,
                       const void* w, void* dx_partial, float* dw, float* db, int accumulate,
                       void* ws, size_t ws_bytes, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  const int64_t n = col_out(s, kind);
  if (n <= 0) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(dy) || !ok_ptr(x) || !ok_ptr(w) || !ok_opt(dx_partial) || !ok_opt(dw) || !ok_opt(db))
    return MTP_ERR_INVALID_ARG;
  if (kind == MTP_FC1_SWIGLU && db != nullptr) return MTP_ERR_INVALID_ARG;
  if (!fits(s.T, n, s.esize) || !fits(n, s.h, s.esize) || !fits(s.T, s.h, s.esize))
    return MTP_ERR_UNSUPPORTED;
  if (db) {
    const size_t need = mtp::column_sum_ws_bytes(s.T, n);
    if (need > 0 && (ws == nullptr || !aligned(ws) || ws_bytes < need)) return MTP_ERR_WORKSPACE;
  }
  hipStream_t str = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (dx_partial) {
    GemmDesc g{};
    g.A = dy; g.lda = n; g.a_kmajor = true;
    g.B = w; g.ldb = s.h; g.b_kmajor = false;
    g.M = static_cast<int>(s.T); g.N = s.h; g.K = static_cast<int>(n);
    g.C = dx_partial; g.ldc = s.h; g.epi = mtp::kEpiStore;
    e = gemm(s, g, str);
    if (e != hipSuccess) return MTP_ERR_HIP;
  }
  if (dw) {
    GemmDesc g{};
    g.A = dy; g.lda = n; g.a_kmajor = false;
    g.B = x; g.ldb = s.h; g.b_kmajor = false;
    g.M = static_cast<int>(n); g.N = s.h; g.K = static_cast<int>(s.T);
    g.C = dw; g.ldc = s.h; g.epi = accumulate ? mtp::kEpiF32Acc : mtp::kEpiF32;
    e = gemm(s, g, str);
    if (e != hipSuccess) return MTP_ERR_HIP;
  }
  if (db) e = mtp::column_sum(s.bf16, dy, s.T, n, db, accumulate != 0, ws, str);
  return hip_status(e);
}

int mtp_row_linear_fwd(const mtp_shard_desc* desc, int kind, const void* x_local, const void* w,
                       void* partial, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  const int64_t k = row_in(s, kind);
  if (k <= 0) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(x_local) || !ok_ptr(w) || !ok_ptr(partial)) return MTP_ERR_INVALID_ARG;
  if (!fits(s.T, k, s.esize) || !fits(s.h, k, s.esize)) return MTP_ERR_UNSUPPORTED;
  GemmDesc g{};
  g.A = x_local; g.lda = k; g.a_kmajor = true;
  g.B = w; g.ldb = k; g.b_kmajor = true;
  g.M = static_cast<int>(s.T); g.N = s.h; g.K = static_cast<int>(k);
  g.C = partial; g.ldc = s.h; g.epi = mtp::kEpiStore;
  return hip_status(gemm(s, g, static_cast<hipStream_t>(stream)));
}

int mtp_row_linear_bwd(const mtp_shard_desc* desc, int kind, const void* dy, const void* x_local,
                       const void* w, const void* gelu_preact, void* dx_local, float* dw,
                       float* db, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  const int64_t k = row_in(s, kind);
  if (k <= 0) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(dy) || !ok_ptr(x_local) || !ok_ptr(w) || !ok_opt(dx_local) || !ok_opt(dw) ||
      !ok_opt(db) || !ok_opt(gelu_preact))
    return MTP_ERR_INVALID_ARG;
  if (gelu_preact && kind != MTP_FC2 && kind != MTP_FC2_SWIGLU) return MTP_ERR_INVALID_ARG;
  const bool swiglu = kind == MTP_FC2_SWIGLU && gelu_preact != nullptr;
  if (!fits(s.T, s.h, s.esize) || !fits(s.h, k, s.esize) || !fits(s.T, k, s.esize))
    return MTP_ERR_UNSUPPORTED;
  if (db) {
    const size_t need = mtp::column_sum_ws_bytes(s.T, s.h);
    if (need > 0 && (ws == nullptr || !aligned(ws) || ws_bytes < need)) return MTP_ERR_WORKSPACE;
  }
  hipStream_t str = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (dx_local) {
    GemmDesc g{};
    g.A = dy; g.lda = s.h; g.a_kmajor = true;
    g.B = w; g.ldb = k; g.b_kmajor = false;
    g.M = static_cast<int>(s.T); g.N = static_cast<int>(k); g.K = s.h;
    g.C = dx_local; g.ldc = swiglu ? 2 * k : k;
    g.aux = const_cast<void*>(gelu_preact); g.ld_aux = swiglu ? 2 * k : k;
    g.epi = swiglu ? mtp::kEpiDSwiGLU : gelu_preact ? mtp::kEpiDGelu : mtp::kEpiStore;
   
    e = gemm(s, g, str);
    if (e != hipSuccess) return MTP_ERR_HIP;
  }
  if (dw) {
    GemmDesc g{};
    g.A = dy; g.lda = s.h; g.a_kmajor = false;
    g.B = x_local; g.ldb = k; g.b_kmajor = false;
    g.M = s.h; g.N = static_cast<int>(k); g.K = static_cast<int>(s.T);
    g.C = dw; g.ldc = k; g.epi = accumulate ? mtp::kEpiF32Acc : mtp::kEpiF32;
   
    e = gemm(s, g, str);
    if (e != hipSuccess) return MTP_ERR_HIP;
  }
  if (db) e = mtp::column_sum(s.bf16, dy, s.T, s.h, db, accumulate != 0, ws, str);
  return hip_status(e);
}

int mtp_attn_fwd(const mtp_shard_desc* desc, const void* qkv, void* ctx, float* lse,
                 const int32_t* cu_seqlens, int32_t n_seqs, float* ctx_amax_parts,
                 void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(qkv) || !ok_ptr(ctx) || !ok_ptr(lse) || !ok_opt(ctx_amax_parts))
    return MTP_ERR_INVALID_ARG;
  if (cu_seqlens && n_seqs < 1) return MTP_ERR_INVALID_ARG;
  if (ctx_amax_parts && !s.bf16) return MTP_ERR_UNSUPPORTED;
  if (!attn_fits(s)) return MTP_ERR_UNSUPPORTED;
  mtp::AttnDesc a{};
  a.qkv = qkv; a.ctx = ctx; a.lse = lse; a.amax = ctx_amax_parts;
  a.cu_seqlens = cu_seqlens; a.n_seqs = n_seqs;
  a.T = s.T; a.seq_len = desc->seq_len; a.heads = s.al; a.head_dim = s.d;
  return hip_status(mtp::attn_fwd(s.bf16, a, static_cast<hipStream_t>(stream)));
}

int mtp_attn_bwd(const mtp_shard_desc* desc, const void* qkv, const void* ctx, const float* lse,
                 const void* dctx, void* dqkv, const int32_t* cu_seqlens, int32_t n_seqs,
                 void* ws, size_t ws_bytes, float* dqkv_amax_parts, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(qkv) || !ok_ptr(ctx) || !ok_ptr(lse) || !ok_ptr(dctx) || !ok_ptr(dqkv) ||
      !ok_opt(dqkv_amax_parts))
    return MTP_ERR_INVALID_ARG;
  if (cu_seqlens && n_seqs < 1) return MTP_ERR_INVALID_ARG;
  if (dqkv_amax_parts && !s.bf16) return MTP_ERR_UNSUPPORTED;
  if (!attn_fits(s)) return MTP_ERR_UNSUPPORTED;
  const size_t need = static_cast<size_t>(s.al) * s.T * sizeof(float) * 2;
  if (need > 0 && (ws == nullptr || !aligned(ws) || ws_bytes < need)) return MTP_ERR_WORKSPACE;
  mtp::AttnDesc a{};
  a.qkv = qkv; a.ctx = const_cast<void*>(ctx); a.lse = const_cast<float*>(lse);
  a.dctx = dctx; a.dqkv = dqkv; a.delta = static_cast<float*>(ws); a.amax = dqkv_amax_parts;
  a.cu_seqlens = cu_seqlens; a.n_seqs = n_seqs;
  a.T = s.T; a.seq_len = desc->seq_len; a.heads = s.al; a.head_dim = s.d;
  return hip_status(mtp::attn_bwd(s.bf16, a, static_cast<hipStream_t>(stream)));
}

// The attention backward for callers that cannot allocate: its preprocess
// rows (D and lse * log2(e), two fp32 rows of T per local head) go to this
// fixed device buffer instead of a caller workspace.  Every GPU the library
// runs on holds its own copy until the process ends.
}  // extern "C"
namespace {
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  Host code passes this
// address, never the array's name, to kernels.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MTP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MTP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MTP_OK;
}
}  // namespace
extern "C" {

int mtp_attn_bwd_noalloc(const mtp_shard_desc* desc, const void* qkv, const void* ctx,
                         const float* lse, const void* dctx, void* dqkv,
                         const int32_t* cu_seqlens, int32_t n_seqs, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(qkv) || !ok_ptr(ctx) || !ok_ptr(lse) || !ok_ptr(dctx) || !ok_ptr(dqkv))
    return MTP_ERR_INVALID_ARG;
  if (cu_seqlens && n_seqs < 1) return MTP_ERR_INVALID_ARG;
  if (!attn_fits(s)) return MTP_ERR_UNSUPPORTED;
  const size_t need = static_cast<size_t>(s.al) * s.T * sizeof(float) * 2;
  if (need > kNoAllocScratchBytes) return MTP_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MTP_OK) return st;
  mtp::AttnDesc a{};
  a.qkv = qkv; a.ctx = const_cast<void*>(ctx); a.lse = const_cast<float*>(lse);
  a.dctx = dctx; a.dqkv = dqkv; a.delta = static_cast<float*>(ws);
  a.cu_seqlens = cu_seqlens; a.n_seqs = n_seqs;
  a.T = s.T; a.seq_len = desc->seq_len; a.heads = s.al; a.head_dim = s.d;
  return hip_status(mtp::attn_bwd(s.bf16, a, static_cast<hipStream_t>(stream)));
}

int mtp_attn_fwd_block(const mtp_shard_desc* desc, const void* qkv, int64_t q_lo, int64_t q_hi,
                       int64_t k_lo, int64_t k_hi, void* ctx, float* lse,
                       const int32_t* cu_seqlens, int32_t n_seqs, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(qkv) || !ok_ptr(ctx) || !ok_ptr(lse)) return MTP_ERR_INVALID_ARG;
  if (cu_seqlens && n_seqs < 1) return MTP_ERR_INVALID_ARG;
  if (!attn_fits(s)) return MTP_ERR_UNSUPPORTED;
  st = check_block(s, desc, q_lo, q_hi, k_lo, k_hi);
  if (st != MTP_OK) return st;
  mtp::AttnDesc a{};
  a.qkv = qkv; a.ctx = ctx; a.lse = lse;
  a.cu_seqlens = cu_seqlens; a.n_seqs = cu_seqlens ? n_seqs : 0;
  a.T = s.T; a.seq_len = desc->seq_len; a.heads = s.al; a.head_dim = s.d;
  a.q_lo = q_lo; a.q_hi = q_hi; a.k_lo = k_lo; a.k_hi = k_hi;
  return hip_status(mtp::attn_fwd(s.bf16, a, static_cast<hipStream_t>(stream)));
}
int mtp_attn_merge(const mtp_shard_desc* desc, void* ctx, float* lse, const void* ctx_part,
                   const float* lse_part, int64_t row_lo, int64_t row_hi, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!s.bf16) return MTP_ERR_UNSUPPORTED;
  if (!ok_ptr(ctx) || !ok_ptr(lse) || !ok_ptr(ctx_part) || !ok_ptr(lse_part))
    return MTP_ERR_INVALID_ARG;
  if (row_lo < 0 || row_hi > s.T || row_lo > row_hi) return MTP_ERR_INVALID_ARG;
  if (!attn_fits(s)) return MTP_ERR_UNSUPPORTED;
  mtp::AttnDesc a{};
  a.ctx = ctx; a.lse = lse;
  a.T = s.T; a.seq_len = desc->seq_len; a.heads = s.al; a.head_dim = s.d;
  return hip_status(mtp::attn_merge(a, ctx_part, lse_part, row_lo, row_hi,
                                    static_cast<hipStream_t>(stream)));
}
int mtp_attn_bwd_block(const mtp_shard_desc* desc, const void* qkv, const void* ctx,
                       const float* lse, const void* dctx, void* dqkv, int64_t q_lo,
                       int64_t q_hi, int64_t k_lo, int64_t k_hi, int accumulate,
                       const int32_t* cu_seqlens, int32_t n_seqs, void* ws, size_t ws_bytes,
                       void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!ok_ptr(qkv) || !ok_ptr(ctx) || !ok_ptr(lse) || !ok_ptr(dctx) || !ok_ptr(dqkv))
    return MTP_ERR_INVALID_ARG;
  if (cu_seqlens && n_seqs < 1) return MTP_ERR_INVALID_ARG;
  if (!attn_fits(s)) return MTP_ERR_UNSUPPORTED;
  st = check_block(s, desc, q_lo, q_hi, k_lo, k_hi);
  if (st != MTP_OK) return st;
  if (q_hi - q_lo != k_hi - k_lo) return MTP_ERR_INVALID_ARG;
  const size_t need = static_cast<size_t>(s.al) * s.T * sizeof(float) * 2;
  if (need > 0 && (ws == nullptr || !aligned(ws) || ws_bytes < need)) return MTP_ERR_WORKSPACE;
  mtp::AttnDesc a{};
  a.qkv = qkv; a.ctx = const_cast<void*>(ctx); a.lse = const_cast<float*>(lse);
  a.dctx = dctx; a.dqkv = dqkv; a.delta = static_cast<float*>(ws);
  a.cu_seqlens = cu_seqlens; a.n_seqs = cu_seqlens ? n_seqs : 0;
  a.T = s.T; a.seq_len = desc->seq_len; a.heads = s.al; a.head_dim = s.d;
  a.q_lo = q_lo; a.q_hi = q_hi; a.k_lo = k_lo; a.k_hi = k_hi;
  a.accumulate = accumulate != 0;
  return hip_status(mtp::attn_bwd(s.bf16, a, static_cast<hipStream_t>(stream)));
}

int mtp_quantize_fp8(const mtp_shard_desc* desc, const void* x, int64_t n, uint8_t* q,
                     float* scale, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!s.bf16) return MTP_ERR_UNSUPPORTED;
  if (n < 0 || (n & 7)) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(x) || !ok_ptr(q) || !ok_ptr(scale)) return MTP_ERR_INVALID_ARG;
  return hip_status(mtp::quantize_fp8(x, n, q, scale, static_cast<hipStream_t>(stream)));
}
int mtp_linear_fwd_fp8(const mtp_shard_desc* desc, int kind, const uint8_t* x8,
                       const float* x_scale, const uint8_t* w8, const float* w_scale,
                       const void* b, void* y, void* preact, float* amax_parts,
                       void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!s.bf16) return MTP_ERR_UNSUPPORTED;
  // column-parallel QKV / FC1 (GeLU or SwiGLU over the interleaved
  // gate|up product) or row-parallel PROJ / FC2 (partial)
  int64_t n = 0, k = 0;
  switch (kind) {
    case MTP_QKV: n = 3LL * s.hl; k = s.h; break;
    case MTP_FC1: n = s.fl; k = s.h; break;
    case MTP_FC1_SWIGLU: n = 2LL * s.fl; k = s.h; break;
    case MTP_PROJ: n = s.h; k = s.hl; break;
    case MTP_FC2: case MTP_FC2_SWIGLU: n = s.h; k = s.fl; break;
    default: return MTP_ERR_INVALID_ARG;
  }
  const bool fc1 = kind == MTP_FC1 || kind == MTP_FC1_SWIGLU;
  const bool swiglu = kind == MTP_FC1_SWIGLU;
  if (!ok_ptr(x8) || !ok_ptr(x_scale) || !ok_ptr(w8) || !ok_ptr(w_scale) || !ok_opt(b) ||
      !ok_ptr(y))
    return MTP_ERR_INVALID_ARG;
  if (fc1 ? !ok_ptr(preact) : preact != nullptr) return MTP_ERR_INVALID_ARG;
  if ((kind == MTP_PROJ || kind == MTP_FC2 || kind == MTP_FC2_SWIGLU || swiglu) && b != nullptr)
    return MTP_ERR_INVALID_ARG;
  if (!ok_opt(amax_parts) || (amax_parts && !fc1)) return MTP_ERR_INVALID_ARG;
  if (k % 16 != 0 || (swiglu && n % 8 != 0)) return MTP_ERR_UNSUPPORTED;
  if (!fits(s.T, k, 1) || !fits(n, k, 1)) return MTP_ERR_UNSUPPORTED;
  GemmDesc g{};
  g.A = x8; g.lda = k; g.a_kmajor = true;
  g.B = w8; g.ldb = k; g.b_kmajor = true;
  g.M = static_cast<int>(s.T); g.N = static_cast<int>(n); g.K = static_cast<int>(k);
  g.C = y; g.ldc = swiglu ? n / 2 : n; g.bias = b;
  g.aux = preact; g.ld_aux = n;
  g.epi = kind == MTP_FC1 ? mtp::kEpiGelu : swiglu ? mtp::kEpiSwiGLU : mtp::kEpiStore;
  g.fp8 = true; g.scale_a = x_scale; g.scale_b = w_scale;
  g.amax = amax_parts;
  return hip_status(mtp::gemm_bf16(g, static_cast<hipStream_t>(stream)));
}

int mtp_fp8_amax(const mtp_shard_desc* desc, const void* x, int64_t n, float* amax_parts,
                 void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!s.bf16) return MTP_ERR_UNSUPPORTED;
  if (n < 0 || (n & 7)) return MTP_ERR_INVALID_ARG;
  if ((n > 0 && !ok_ptr(x)) || !ok_ptr(amax_parts)) return MTP_ERR_INVALID_ARG;
  return hip_status(mtp::fp8_amax(x, n, amax_parts, static_cast<hipStream_t>(stream)));
}

int mtp_fp8_quantize(const mtp_shard_desc* desc, int fmt, const void* x, int64_t rows,
                     int64_t cols, const float* const* amax_parts, int32_t n_parts, uint8_t* q,
                     uint8_t* q_t, float* scale, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!s.bf16) return MTP_ERR_UNSUPPORTED;
  if (fmt != MTP_FP8_E4M3 && fmt != MTP_FP8_E5M2) return MTP_ERR_INVALID_ARG;
  if (rows < 0 || cols <= 0 || (cols & 7) || cols > (int64_t{1} << 30)) return MTP_ERR_INVALID_ARG;
  if (!amax_parts || n_parts < 1 || n_parts > mtp::kMaxPartials) return MTP_ERR_INVALID_ARG;
  for (int i = 0; i < n_parts; ++i)
    if (!ok_ptr(amax_parts[i])) return MTP_ERR_INVALID_ARG;
  // with no rows there is nothing to read or write but the scale
  if (!ok_opt(x) || !ok_opt(q) || !ok_opt(q_t) || !ok_ptr(scale)) return MTP_ERR_INVALID_ARG;
  if (rows > 0 && (!x || (!q && !q_t))) return MTP_ERR_INVALID_ARG;
  if (!fits(rows, cols, 1) || (rows + 127) / 128 > 65535) return MTP_ERR_UNSUPPORTED;
  return hip_status(mtp::fp8_quantize(fmt == MTP_FP8_E5M2 ? mtp::kFp8E5M2 : mtp::kFp8E4M3, x,
                                      rows, static_cast<int>(cols), amax_parts, n_parts, q, q_t,
                                      scale, static_cast<hipStream_t>(stream)));
}

int mtp_linear_bwd_fp8(const mtp_shard_desc* desc, int kind, const uint8_t* dy8,
                       const uint8_t* dy8_t, const float* dy_scale, const uint8_t* w8_t,
                       const float* w_scale, const uint8_t* x8_t, const float* x_scale,
                       const void* preact, void* dx, float* dw, int accumulate,
                       float* dx_amax_parts, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!s.bf16) return MTP_ERR_UNSUPPORTED;
  int64_t out = 0, in = 0;
  switch (kind) {
    case MTP_QKV: out = 3LL * s.hl; in = s.h; break;
    case MTP_FC1: out = s.fl; in = s.h; break;
    case MTP_FC1_SWIGLU: out = 2LL * s.fl; in = s.h; break;
    case MTP_PROJ: out = s.h; in = s.hl; break;
    case MTP_FC2: case MTP_FC2_SWIGLU: out = s.h; in = s.fl; break;
    default: return MTP_ERR_INVALID_ARG;
  }
  // FC2 after SwiGLU: the data gradient is the interleaved [dgate | dup]
  const bool dswiglu = kind == MTP_FC2_SWIGLU && preact != nullptr;
  if (!ok_ptr(dy_scale) || !ok_opt(dx) || !ok_opt(dw) || !ok_opt(preact)) return MTP_ERR_INVALID_ARG;
  if (preact && kind != MTP_FC2 && kind != MTP_FC2_SWIGLU) return MTP_ERR_INVALID_ARG;
  if (!ok_opt(dx_amax_parts) || (dx_amax_parts && (!dx || !preact))) return MTP_ERR_INVALID_ARG;
  if (dx && (!ok_ptr(dy8) || !ok_ptr(w8_t) || !ok_ptr(w_scale))) return MTP_ERR_INVALID_ARG;
  if (dw && (!ok_ptr(dy8_t) || !ok_ptr(x8_t) || !ok_ptr(x_scale))) return MTP_ERR_INVALID_ARG;
  // 16-byte k chunks: the reduction lengths (out for the data gradient, T
  // for the weight gradient) must be multiples of 16
  if ((dx && (out & 15)) || (dw && (s.T & 15))) return MTP_ERR_UNSUPPORTED;
  if (!fits(s.T, out, 1) || !fits(in, out, 1) || !fits(in, s.T, 1)) return MTP_ERR_UNSUPPORTED;
  hipStream_t str = static_cast<hipStream_t>(stream);
  if (dx) {
    GemmDesc g{};
    g.A = dy8; g.lda = out; g.a_kmajor = true;
    g.B = w8_t; g.ldb = out; g.b_kmajor = true;
    g.M = static_cast<int>(s.T); g.N = static_cast<int>(in); g.K = static_cast<int>(out);
    g.C = dx; g.ldc = dswiglu ? 2 * in : in;
    g.aux = const_cast<void*>(preact); g.ld_aux = dswiglu ? 2 * in : in;
    g.epi = dswiglu ? mtp::kEpiDSwiGLU : preact ? mtp::kEpiDGelu : mtp::kEpiStore;
    g.fp8 = true; g.a_e5m2 = true; g.scale_a = dy_scale; g.scale_b = w_scale;
    g.amax = dx_amax_parts;
    if (mtp::gemm_bf16(g, str) != hipSuccess) return MTP_ERR_HIP;
  }
  if (dw) {
    GemmDesc g{};
    g.A = dy8_t; g.lda = s.T; g.a_kmajor = true;
    g.B = x8_t; g.ldb = s.T; g.b_kmajor = true;
    g.M = static_cast<int>(out); g.N = static_cast<int>(in); g.K = static_cast<int>(s.T);
    g.C = dw; g.ldc = in;
    g.epi = accumulate ? mtp::kEpiF32Acc : mtp::kEpiF32;
    g.fp8 = true; g.a_e5m2 = true; g.scale_a = dy_scale; g.scale_b = x_scale;
    if (mtp::gemm_bf16(g, str) != hipSuccess) return MTP_ERR_HIP;
  }
  return MTP_OK;
}

int mtp_partial_sum(const mtp_shard_desc* desc, const void* const* partials, int32_t n_partials,
                    const void* bias, const void* residual, void* out, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!partials || n_partials < 1 || n_partials > mtp::kMaxPartials) return MTP_ERR_INVALID_ARG;
  for (int i = 0; i < n_partials; ++i)
    if (!ok_ptr(partials[i])) return MTP_ERR_INVALID_ARG;
  if (!ok_opt(bias) || !ok_opt(residual) || !ok_ptr(out)) return MTP_ERR_INVALID_ARG;
  return hip_status(mtp::partial_sum(s.bf16, partials, n_partials, bias, residual, out, s.T, s.h,
                                     static_cast<hipStream_t>(stream)));
}

int mtp_partial_sum_layernorm(const mtp_shard_desc* desc, const void* const* partials,
                              int32_t n_partials, const void* bias, const void* residual,
                              void* out, const void* gamma, const void* beta, void* ln_out,
                              float* mean, float* rstd, float* amax_parts, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!partials || n_partials < 1 || n_partials > mtp::kMaxPartials) return MTP_ERR_INVALID_ARG;
  for (int i = 0; i < n_partials; ++i)
    if (!ok_ptr(partials[i])) return MTP_ERR_INVALID_ARG;
  if (!ok_opt(bias) || !ok_opt(residual) || !ok_ptr(out) || !ok_ptr(gamma) || !ok_ptr(beta) ||
      !ok_ptr(ln_out) || !ok_ptr(mean) || !ok_ptr(rstd) || !ok_opt(amax_parts))
    return MTP_ERR_INVALID_ARG;
  if (amax_parts && !s.bf16) return MTP_ERR_UNSUPPORTED;
  return hip_status(mtp::sum_layernorm_fwd(s.bf16, partials, n_partials, bias, residual, out,
                                           gamma, beta, ln_out, mean, rstd, s.T, s.h, s.eps,
                                           amax_parts, static_cast<hipStream_t>(stream)));
}

int mtp_vocab_ce_stats(const mtp_shard_desc* desc, const float* logits, const int32_t* targets,
                       float* m, float* sm, float* z_tgt, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (s.Vl <= 0) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(logits) || !ok_ptr(targets) || !ok_ptr(m) || !ok_ptr(sm) || !ok_ptr(z_tgt))
    return MTP_ERR_INVALID_ARG;
  return hip_status(mtp::ce_stats(logits, targets, m, sm, z_tgt, s.T, s.Vl, s.r * s.Vl, s.V,
                                  static_cast<hipStream_t>(stream)));
}

int mtp_vocab_ce_combine(const mtp_shard_desc* desc, const float* const* m, const float* const* sm,
                         const float* const* z_tgt, int32_t n_ranks, float* M, float* S,
                         float* loss, float* loss_mean, void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (!m || !sm || !z_tgt || n_ranks < 1 || n_ranks > mtp::kMaxPartials) return MTP_ERR_INVALID_ARG;
  for (int i = 0; i < n_ranks; ++i)
    if (!ok_ptr(m[i]) || !ok_ptr(sm[i]) || !ok_ptr(z_tgt[i])) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(M) || !ok_ptr(S) || !ok_ptr(loss) || !ok_opt(loss_mean)) return MTP_ERR_INVALID_ARG;
  return hip_status(mtp::ce_combine(m, sm, z_tgt, n_ranks, M, S, loss, loss_mean, s.T,
                                    static_cast<hipStream_t>(stream)));
}

int mtp_vocab_ce_bwd(const mtp_shard_desc* desc, const float* logits, const int32_t* targets,
                     const float* M, const float* S, float dloss_scale, void* dlogits,
                     void* stream) {
  Shard s;
  int st = check_desc(desc, &s);
  if (st != MTP_OK) return st;
  if (s.Vl <= 0) return MTP_ERR_INVALID_ARG;
  if (!ok_ptr(logits) || !ok_ptr(targets) || !ok_ptr(M) || !ok_ptr(S) || !ok_ptr(dlogits))
    return MTP_ERR_INVALID_ARG;
  if (!isfinite(dloss_scale)) return MTP_ERR_INVALID_ARG;
  return hip_status(mtp::ce_bwd(s.bf16, logits, targets, M, S, dloss_scale, dlogits, s.T, s.Vl,
                                s.r * s.Vl, s.V, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
