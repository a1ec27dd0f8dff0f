// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Host-side only declarations; every launcher enqueues on `stream` and
// returns hipGetLastError() after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

// ------------------------------------------------------------------ GEMM
// C[M,N] = sum_k A(m,k) B(n,k), fp32 accumulate, then an epilogue.
//   A(m,k) = a_kmajor ? A[m*lda + k] : A[k*lda + m]
//   B(n,k) = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
enum Epilogue : int {
  kEpiStore = 0,    // C = acc (+ bias[n])                     C in elem type
  kEpiGelu = 1,     // aux = acc + bias (u); C = GeLU_tanh(u)   C, aux elem type
  kEpiDGelu = 2,    // C = acc * GeLU_tanh'(aux)               C, aux elem type
  kEpiF32 = 3,      // C = acc (+ bias[n])                     C fp32
  kEpiF32Acc = 4,   // C += acc                                C fp32
  // SwiGLU, columns interleaved in groups of 4 (gate 8j..8j+3, up 8j+4..8j+7):
  kEpiSwiGLU = 5,   // aux = acc; C[n/2 + i] = SiLU(gate) * up   C, aux elem type
  kEpiDSwiGLU = 6,  // acc = dg [.., N]: C/aux [.., 2N] interleaved:
                    //   C(gate) = dg * up * SiLU'(gate), C(up) = dg * SiLU(gate)
};

struct GemmDesc {
  const void* A; int64_t lda; bool a_kmajor;
  const void* B; int64_t ldb; bool b_kmajor;
  int M, N, K;
  void* C; int64_t ldc;
  const void* bias;    // [N] elem type, nullable
  void* aux; int64_t ld_aux;
  int epi;
  // FP8 operands, both k-major: A and B hold one byte per element and
  // C = (A B^T) * scale_a[0] * scale_b[0] before the epilogue; B is E4M3,
  // A is E4M3 or (a_e5m2) E5M2.
  bool fp8 = false;
  bool a_e5m2 = false;
  const float* scale_a = nullptr;
  const float* scale_b = nullptr;
  // FP8 GeLU / GeLU' epilogues (C contiguous, ldc == N): kAmaxParts partial
  // maxima of |C| as stored, in fp8_amax's form (nullable).
  float* amax = nullptr;
};

hipError_t gemm_bf16(const GemmDesc& g, hipStream_t stream);
hipError_t gemm_f32(const GemmDesc& g, hipStream_t stream);

// Per-tensor E4M3 quantization of n bf16 values (n % 8 == 0): scale[1]
// receives amax, scale[0] s = amax / 448 (1 for a zero tensor), q the codes
// of round-to-nearest-even(clamp(x / s, -448, 448)).
hipError_t quantize_fp8(const void* x, int64_t n, uint8_t* q, float* scale, hipStream_t stream);
// Per-tensor FP8 quantization in two steps, so that the shards of one tensor
// share one scale: partial maxima of |x| (kAmaxParts fp32 per shard), then
// the codes of a [rows, cols] shard, row-major and/or transposed, with the
// scale of the maximum over n_parts shards' partial maxima.
constexpr int kAmaxParts = 1024;
enum Fp8Format : int { kFp8E4M3 = 0, kFp8E5M2 = 1 };
hipError_t fp8_amax(const void* x, int64_t n, float* parts, hipStream_t stream);
hipError_t fp8_quantize(int fmt, const void* x, int64_t rows, int cols, const float* const* parts,
                        int n_parts, uint8_t* q, uint8_t* qt, float* scale, hipStream_t stream);

// Column sums of a [rows, cols] matrix into fp32 out[cols] (= or +=).
// ws must hold column_sum_ws_bytes(rows, cols) bytes.
size_t column_sum_ws_bytes(int64_t rows, int64_t cols);
hipError_t column_sum(bool bf16, const void* x, int64_t rows, int64_t cols, float* out,
                      bool accumulate, void* ws, hipStream_t stream);

// ------------------------------------------------------------- row-wise
// amax (nullable, bf16 output): kAmaxParts partial maxima of |y| in
// fp8_amax's form (their maximum is y's amax), from the LayerNorm kernel
// itself where its grid fits, else by fp8_amax on y.
hipError_t layernorm_fwd(bool bf16, const void* x, const void* gamma, const void* beta, void* y,
                         float* mean, float* rstd, int64_t T, int h, float eps, float* amax,
                         hipStream_t stream);
size_t layernorm_bwd_ws_bytes(int64_t T, int h, bool bf16);
hipError_t layernorm_bwd(bool bf16, const void* dy, const void* x, const void* gamma,
                         const float* mean, const float* rstd, const void* dres, void* dx,
                         float* dgamma, float* dbeta, bool accumulate, int64_t T, int h,
                         void* ws, hipStream_t stream);
constexpr int kMaxPartials = 16;
hipError_t partial_sum(bool bf16, const void* const* partials, int n, const void* bias,
                       const void* residual, void* out, int64_t T, int h, hipStream_t stream);
// partial_sum into out, then LayerNorm of out (one pass when h = 512*{1,2,4,8}).
hipError_t sum_layernorm_fwd(bool bf16, const void* const* partials, int n, const void* bias,
                             const void* residual, void* out, const void* gamma,
                             const void* beta, void* y, float* mean, float* rstd, int64_t T,
                             int h, float eps, float* amax, hipStream_t stream);
// LayerNorm backward of dy = sum of n partials (rounded to the storage type);
// amax as in layernorm_fwd, of dx.
hipError_t layernorm_bwd_sum(bool bf16, const void* const* dys, int n, const void* x,
                             const void* gamma, const float* mean, const float* rstd,
                             const void* dres, void* dx, float* dgamma, float* dbeta,
                             bool accumulate, int64_t T, int h, void* ws, float* amax,
                             hipStream_t stream);
hipError_t zero_f32(float* p, int64_t n, hipStream_t stream);

// ------------------------------------------------------------- attention
struct AttnDesc {
  const void* qkv; void* ctx; float* lse;
  const void* dctx; void* dqkv; float* delta;  // backward
  const int32_t* cu_seqlens; int n_seqs;        // nullable -> fixed seq_len
  int64_t T; int seq_len; int heads; int head_dim;
  // Query rows [q_lo, q_hi) attend to key rows [k_lo, k_hi) (absolute
  // positions, causal mask unchanged); a whole-sequence call uses 0..T for
  // both.  With accumulate, the backward adds into dqkv instead of storing.
  int64_t q_lo = 0, q_hi = -1, k_lo = 0, k_hi = -1;
  bool accumulate = false;
  // bf16 whole-range calls: kAmaxParts partial maxima of |ctx| (forward) or
  // |dqkv| (backward) as stored, in fp8_amax's form (nullable).
  float* amax = nullptr;
};
hipError_t attn_fwd(bool bf16, const AttnDesc& a, hipStream_t stream);
hipError_t attn_fwd_bf16_mfma(const AttnDesc& a, hipStream_t stream);
hipError_t attn_bwd_bf16_mfma(const AttnDesc& a, hipStream_t stream);
hipError_t attn_bwd(bool bf16, const AttnDesc& a, hipStream_t stream);
// Merge a partial attention result into an accumulated one over rows
// [row_lo, row_hi): lse = log(e^lse_acc + e^lse_part), ctx = weighted mean.
hipError_t attn_merge(const AttnDesc& acc, const void* ctx_part, const float* lse_part,
                      int64_t row_lo, int64_t row_hi, hipStream_t stream);

// ------------------------------------------------------------ vocab CE
hipError_t ce_stats(const float* logits, const int32_t* targets, float* m, float* s, float* zt,
                    int64_t T, int64_t V_l, int64_t v0, int64_t V, hipStream_t stream);
hipError_t ce_combine(const float* const* m, const float* const* s, const float* const* zt, int n,
                      float* M, float* S, float* loss, float* loss_mean, int64_t T,
                      hipStream_t stream);
hipError_t ce_bwd(bool bf16, const float* logits, const int32_t* targets, const float* M,
                  const float* S, float scale, void* dlogits, int64_t T, int64_t V_l, int64_t v0,
                  int64_t V, hipStream_t stream);

}  // namespace mtp
