// HBM-bound kernels of the layer shard: LayerNorm forward/backward, the
// on-device sum of tensor-parallel partials, column sums (bias gradients)
// and the vocab-parallel cross-entropy pieces.  All loads and stores are
// 16-byte vectors of 8 consecutive elements along the contiguous axis;
// every reduction accumulates in fp32 in a fixed order (deterministic).
#include "common.h"
#include "kernels.h"

namespace mtp {
namespace {

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kMaxRegChunks = 8;  // rows are cached in registers: h <= 8*8*256

template <typename T> __host__ __device__ __forceinline__ const T* cptr(const void* p) {
  return static_cast<const T*>(p);
}

// Block-wide sum over kRowThreads threads (result broadcast to all).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) s += red[i];
  return s;
}

// ----------------------------------------------------------- LayerNorm fwd
// One workgroup per token row.  Two passes over the register-cached row:
// mean, then the centred second moment (population variance).
template <typename T, int NC>
__global__ void __launch_bounds__(kRowThreads)
layernorm_fwd_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                     const T* __restrict__ beta, T* __restrict__ y, float* __restrict__ mean,
                     float* __restrict__ rstd, int h, float eps) {
  __shared__ float red[kRowWaves];
  const int64_t row = blockIdx.x;
  const int nchunk = h / 8;
  const T* xr = x + row * h;
  float v[NC][8];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    if (c < nchunk) {
      load8(xr + c * 8, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    }
  }
  const float mu = block_sum(s, red) / h;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    if (c < nchunk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float d = v[i][e] - mu; q += d * d; }
    }
  }
  const float rs = rsqrtf(block_sum(q, red) / h + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    if (c < nchunk) {
      float g[8], b[8], o[8];
      load8(gamma + c * 8, g);
      load8(beta + c * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[i][e] - mu) * rs * g[e] + b[e];
      store8(y + row * h + c * 8, o);
    }
  }
  if (threadIdx.x == 0) { mean[row] = mu; rstd[row] = rs; }
}

// ----------------------------------------------------------- LayerNorm bwd
// Workgroup b handles rows [b*rpb, (b+1)*rpb).  Per row:
//   xhat = (x-mu)*rstd, gh = dy*gamma,
//   dx = rstd*(gh - mean(gh) - xhat*mean(gh*xhat)) (+ dres).
// Column partial sums of dy*xhat and dy over the workgroup's rows go to ws;
// reduce_parts_kernel adds the partials in workgroup order.
template <typename T, int NC>
__global__ void __launch_bounds__(kRowThreads)
layernorm_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ x,
                     const T* __restrict__ gamma, const float* __restrict__ mean,
                     const float* __restrict__ rstd, const T* __restrict__ dres,
                     T* __restrict__ dx, float* __restrict__ part_g, float* __restrict__ part_b,
                     int64_t T_rows, int h, int rpb) {
  __shared__ float red[kRowWaves];
  const int nchunk = h / 8;
  float accg[NC][8], accb[NC][8];
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { accg[i][e] = 0.0f; accb[i][e] = 0.0f; }
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpb;
  const int64_t r1 = min(T_rows, r0 + rpb);
  for (int64_t row = r0; row < r1; ++row) {
    const float mu = mean[row], rs = rstd[row];
    float xh[NC][8], gh[NC][8];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + i * kRowThreads;
      if (c < nchunk) {
        float xv[8], dv[8], gv[8];
        load8(x + row * h + c * 8, xv);
        load8(dy + row * h + c * 8, dv);
        load8(gamma + c * 8, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[i][e] = (xv[e] - mu) * rs;
          gh[i][e] = dv[e] * gv[e];
          s1 += gh[i][e];
          s2 += gh[i][e] * xh[i][e];
          accg[i][e] += dv[e] * xh[i][e];
          accb[i][e] += dv[e];
        }
      }
    }
    const float m1 = block_sum(s1, red) / h;
    const float m2 = block_sum(s2, red) / h;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = threadIdx.x + i * kRowThreads;
      if (c < nchunk) {
        float o[8];
        if (dres) load8(dres + row * h + c * 8, o);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += rs * (gh[i][e] - m1 - xh[i][e] * m2);
        store8(dx + row * h + c * 8, o);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    if (c < nchunk) {
      store8(part_g + static_cast<int64_t>(blockIdx.x) * h + c * 8, accg[i]);
      store8(part_b + static_cast<int64_t>(blockIdx.x) * h + c * 8, accb[i]);
    }
  }
}

// out[c] (=|+=) sum_{b < nparts} part[b*cols + c].  A workgroup owns 16
// columns (64-byte rows of the partial matrix) and 16 part lanes: lane ty
// sums parts ty, ty+16, ... in ascending order, then lane sums are added in
// ty order, so the result does not depend on scheduling.
constexpr int kRedCols = 16;
constexpr int kRedLanes = 16;
__global__ void __launch_bounds__(kRedCols * kRedLanes)
reduce_parts_kernel(const float* __restrict__ part, int nparts, int64_t cols,
                    float* __restrict__ out, int accumulate) {
  __shared__ float red[kRedLanes][kRedCols];
  const int tx = threadIdx.x % kRedCols, ty = threadIdx.x / kRedCols;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRedCols + tx;
  float s = 0.0f;
  if (c < cols)
    for (int b = ty; b < nparts; b += kRedLanes) s += part[static_cast<int64_t>(b) * cols + c];
  red[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && c < cols) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kRedLanes; ++i) t += red[i][tx];
    out[c] = accumulate ? out[c] + t : t;
  }
}

// --------------------------------------------------------------- col sums
// Stage 1: workgroup (bx, by) sums rows [by*rpb, (by+1)*rpb) of columns
// [bx*512, bx*512+512): 64 threads x 8 columns x 4 row lanes.
template <typename T>
__global__ void __launch_bounds__(256)
colsum_part_kernel(const T* __restrict__ x, int64_t rows, int64_t cols, int rpb,
                   float* __restrict__ part) {
  __shared__ float red[4][512];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 512 + tx * 8;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rpb;
  const int64_t r1 = min(rows, r0 + rpb);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c < cols) {
    for (int64_t r = r0 + ty; r < r1; r += 4) {
      float v[8];
      load8(x + r * cols + c, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[ty][tx * 8 + e] = acc[e];
  __syncthreads();
  if (ty == 0 && c < cols) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = red[0][tx * 8 + e] + red[1][tx * 8 + e] + red[2][tx * 8 + e] + red[3][tx * 8 + e];
    store8(part + static_cast<int64_t>(blockIdx.y) * cols + c, o);
  }
}

// ------------------------------------------------------------ partial sum
struct PartialPtrs { const void* p[kMaxPartials]; };

template <typename T>
__global__ void __launch_bounds__(256)
partial_sum_kernel(PartialPtrs parts, int n, const T* __restrict__ bias,
                   const T* __restrict__ residual, T* out, int64_t total, int h) {
  const int64_t nvec = total / 8;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t off = v * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < n; ++i) {
      float t[8];
      load8(static_cast<const T*>(parts.p[i]) + off, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += t[e];
    }
    if (bias) {
      float t[8];
      load8(bias + (off % h), t);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += t[e];
    }
    if (residual) {
      float t[8];
      load8(residual + off, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += t[e];
    }
    store8(out + off, acc);
  }
}

__global__ void __launch_bounds__(256) zero_kernel(float* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

// ---------------------------------------------------------------- vocab CE
// One workgroup per token: online (max, sum-exp) over the shard's logits,
// merged across lanes and waves.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

__global__ void __launch_bounds__(256)
ce_stats_kernel(const float* __restrict__ logits, const int32_t* __restrict__ targets,
                float* __restrict__ mo, float* __restrict__ so, float* __restrict__ zo,
                int64_t V_l, int64_t v0, int64_t V) {
  __shared__ float rm[4], rs[4];
  const int64_t row = blockIdx.x;
  const float* z = logits + row * V_l;
  float m = -INFINITY, s = 0.0f;
  for (int64_t c = static_cast<int64_t>(threadIdx.x) * 8; c < V_l; c += 256 * 8) {
    float v[8];
    load8(z + c, v);
    float bm = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, v[e]);
    float bs = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) bs += __expf(v[e] - bm);
    merge_ms(m, s, bm, bs);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
    merge_ms(m, s, m2, s2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { rm[w] = m; rs[w] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = rm[0], S = rs[0];
    for (int i = 1; i < 4; ++i) merge_ms(M, S, rm[i], rs[i]);
    mo[row] = M;
    so[row] = S;
    const int64_t tg = targets[row];
    float zt = 0.0f;
    if (tg < 0 || tg >= V) zt = __int_as_float(0x7fc00000);
    else if (tg >= v0 && tg < v0 + V_l) zt = z[tg - v0];
    zo[row] = zt;
  }
}

struct ConstPtrs { const float* p[kMaxPartials]; };

__global__ void __launch_bounds__(256)
ce_combine_kernel(ConstPtrs m, ConstPtrs s, ConstPtrs zt, int n, float* __restrict__ Mo,
                  float* __restrict__ So, float* __restrict__ loss, int64_t T) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  float M = -INFINITY;
  for (int r = 0; r < n; ++r) M = fmaxf(M, m.p[r][t]);
  float S = 0.0f, z = 0.0f;
  for (int r = 0; r < n; ++r) {
    S += s.p[r][t] * __expf(m.p[r][t] - M);
    z += zt.p[r][t];
  }
  Mo[t] = M;
  So[t] = S;
  loss[t] = __logf(S) + M - z;
}

__global__ void __launch_bounds__(256)
mean_kernel(const float* __restrict__ x, int64_t n, float* __restrict__ out) {
  __shared__ float red[kRowWaves];
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += x[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) out[0] = n > 0 ? s / static_cast<float>(n) : 0.0f;
}

template <typename T>
__global__ void __launch_bounds__(256)
ce_bwd_kernel(const float* __restrict__ logits, const int32_t* __restrict__ targets,
              const float* __restrict__ M, const float* __restrict__ S, float scale,
              T* __restrict__ dlogits, int64_t V_l, int64_t v0, int blocks_per_row) {
  const int64_t row = blockIdx.x / blocks_per_row;
  const int64_t c = (static_cast<int64_t>(blockIdx.x % blocks_per_row) * 256 + threadIdx.x) * 8;
  if (c >= V_l) return;
  const float m = M[row], inv = 1.0f / S[row];
  const int64_t tg = static_cast<int64_t>(targets[row]) - v0;
  float v[8];
  load8(logits + row * V_l + c, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p = __expf(v[e] - m) * inv;
    if (c + e == tg) p -= 1.0f;
    v[e] = p * scale;
  }
  store8(dlogits + row * V_l + c, v);
}

int grid_for(int64_t nvec) {
  const int64_t b = (nvec + 255) / 256;
  return static_cast<int>(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

int ln_bwd_parts(int64_t T) {
  int64_t parts = (T + 7) / 8;
  if (parts > 512) parts = 512;
  return static_cast<int>(parts);
}

constexpr int kColRowsPerPart = 64;

int64_t colsum_parts(int64_t rows) {
  int64_t p = (rows + kColRowsPerPart - 1) / kColRowsPerPart;
  return p > 256 ? 256 : p;
}

// ---------------------------------------------------------------- launchers
// Register chunks per thread for a row of h elements (8 per chunk).
int reg_chunks(int h) {
  const int per = (h / 8 + kRowThreads - 1) / kRowThreads;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 6 ? 6 : 8;
}

template <typename T, int NC>
void launch_ln_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean,
                   float* rstd, int64_t T_rows, int h, float eps, hipStream_t s) {
  hipLaunchKernelGGL((layernorm_fwd_kernel<T, NC>), dim3(T_rows), dim3(kRowThreads), 0, s,
                     cptr<T>(x), cptr<T>(gamma), cptr<T>(beta), static_cast<T*>(y), mean, rstd,
                     h, eps);
}

template <typename T>
void ln_fwd_nc(const void* x, const void* gamma, const void* beta, void* y, float* mean,
               float* rstd, int64_t T_rows, int h, float eps, hipStream_t s) {
  switch (reg_chunks(h)) {
    case 1: launch_ln_fwd<T, 1>(x, gamma, beta, y, mean, rstd, T_rows, h, eps, s); break;
    case 2: launch_ln_fwd<T, 2>(x, gamma, beta, y, mean, rstd, T_rows, h, eps, s); break;
    case 4: launch_ln_fwd<T, 4>(x, gamma, beta, y, mean, rstd, T_rows, h, eps, s); break;
    case 6: launch_ln_fwd<T, 6>(x, gamma, beta, y, mean, rstd, T_rows, h, eps, s); break;
    default: launch_ln_fwd<T, 8>(x, gamma, beta, y, mean, rstd, T_rows, h, eps, s); break;
  }
}

template <typename T, int NC>
void launch_ln_bwd(const void* dy, const void* x, const void* gamma, const float* mean,
                   const float* rstd, const void* dres, void* dx, float* pg, float* pb,
                   int64_t T_rows, int h, int rpb, int parts, hipStream_t s) {
  hipLaunchKernelGGL((layernorm_bwd_kernel<T, NC>), dim3(parts), dim3(kRowThreads), 0, s,
                     cptr<T>(dy), cptr<T>(x), cptr<T>(gamma), mean, rstd, cptr<T>(dres),
                     static_cast<T*>(dx), pg, pb, T_rows, h, rpb);
}

template <typename T>
void ln_bwd_nc(const void* dy, const void* x, const void* gamma, const float* mean,
               const float* rstd, const void* dres, void* dx, float* pg, float* pb,
               int64_t T_rows, int h, int rpb, int parts, hipStream_t s) {
  switch (reg_chunks(h)) {
    case 1: launch_ln_bwd<T, 1>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T_rows, h, rpb, parts, s); break;
    case 2: launch_ln_bwd<T, 2>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T_rows, h, rpb, parts, s); break;
    case 4: launch_ln_bwd<T, 4>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T_rows, h, rpb, parts, s); break;
    case 6: launch_ln_bwd<T, 6>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T_rows, h, rpb, parts, s); break;
    default: launch_ln_bwd<T, 8>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T_rows, h, rpb, parts, s); break;
  }
}

}  // namespace

hipError_t layernorm_fwd(bool bf16, const void* x, const void* gamma, const void* beta, void* y,
                         float* mean, float* rstd, int64_t T, int h, float eps,
                         hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (h / 8 > kRowThreads * kMaxRegChunks) return hipErrorInvalidValue;
  if (bf16) ln_fwd_nc<bf16_t>(x, gamma, beta, y, mean, rstd, T, h, eps, s);
  else ln_fwd_nc<float>(x, gamma, beta, y, mean, rstd, T, h, eps, s);
  return hipGetLastError();
}

size_t layernorm_bwd_ws_bytes(int64_t T, int h) {
  return static_cast<size_t>(ln_bwd_parts(T)) * h * 2 * sizeof(float);
}

hipError_t layernorm_bwd(bool bf16, const void* dy, const void* x, const void* gamma,
                         const float* mean, const float* rstd, const void* dres, void* dx,
                         float* dgamma, float* dbeta, bool accumulate, int64_t T, int h,
                         void* ws, hipStream_t s) {
  if (h / 8 > kRowThreads * kMaxRegChunks) return hipErrorInvalidValue;
  const int parts = ln_bwd_parts(T);
  float* pg = static_cast<float*>(ws);
  float* pb = pg + static_cast<int64_t>(parts) * h;
  if (T > 0) {
    const int rpb = static_cast<int>((T + parts - 1) / parts);
    if (bf16) ln_bwd_nc<bf16_t>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T, h, rpb, parts, s);
    else ln_bwd_nc<float>(dy, x, gamma, mean, rstd, dres, dx, pg, pb, T, h, rpb, parts, s);
  }
  const dim3 g((h + kRedCols - 1) / kRedCols);
  hipLaunchKernelGGL(reduce_parts_kernel, g, dim3(kRedCols * kRedLanes), 0, s, pg, T > 0 ? parts : 0,
                     static_cast<int64_t>(h), dgamma, accumulate ? 1 : 0);
  hipLaunchKernelGGL(reduce_parts_kernel, g, dim3(kRedCols * kRedLanes), 0, s, pb, T > 0 ? parts : 0,
                     static_cast<int64_t>(h), dbeta, accumulate ? 1 : 0);
  return hipGetLastError();
}

size_t column_sum_ws_bytes(int64_t rows, int64_t cols) {
  return static_cast<size_t>(colsum_parts(rows)) * cols * sizeof(float);
}

hipError_t column_sum(bool bf16, const void* x, int64_t rows, int64_t cols, float* out,
                      bool accumulate, void* ws, hipStream_t s) {
  const int64_t parts = colsum_parts(rows);
  float* part = static_cast<float*>(ws);
  if (rows > 0) {
    const int rpb = static_cast<int>((rows + parts - 1) / parts);
    const dim3 g((cols + 511) / 512, parts);
    if (bf16)
      hipLaunchKernelGGL(colsum_part_kernel<bf16_t>, g, dim3(256), 0, s, cptr<bf16_t>(x), rows,
                         cols, rpb, part);
    else
      hipLaunchKernelGGL(colsum_part_kernel<float>, g, dim3(256), 0, s, cptr<float>(x), rows,
                         cols, rpb, part);
  }
  hipLaunchKernelGGL(reduce_parts_kernel, dim3((cols + kRedCols - 1) / kRedCols),
                     dim3(kRedCols * kRedLanes), 0, s, part,
                     static_cast<int>(rows > 0 ? parts : 0), cols, out, accumulate ? 1 : 0);
  return hipGetLastError();
}

hipError_t partial_sum(bool bf16, const void* const* partials, int n, const void* bias,
                       const void* residual, void* out, int64_t T, int h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  PartialPtrs pp{};
  for (int i = 0; i < n; ++i) pp.p[i] = partials[i];
  const int64_t total = T * h;
  const int grid = grid_for(total / 8);
  if (bf16)
    hipLaunchKernelGGL(partial_sum_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, pp, n,
                       cptr<bf16_t>(bias), cptr<bf16_t>(residual), static_cast<bf16_t*>(out),
                       total, h);
  else
    hipLaunchKernelGGL(partial_sum_kernel<float>, dim3(grid), dim3(256), 0, s, pp, n,
                       cptr<float>(bias), cptr<float>(residual), static_cast<float*>(out), total,
                       h);
  return hipGetLastError();
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t ce_stats(const float* logits, const int32_t* targets, float* m, float* sm, float* zt,
                    int64_t T, int64_t V_l, int64_t v0, int64_t V, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_stats_kernel, dim3(T), dim3(256), 0, s, logits, targets, m, sm, zt, V_l,
                     v0, V);
  return hipGetLastError();
}

hipError_t ce_combine(const float* const* m, const float* const* sm, const float* const* zt,
                      int n, float* M, float* S, float* loss, float* loss_mean, int64_t T,
                      hipStream_t s) {
  ConstPtrs pm{}, ps{}, pz{};
  for (int i = 0; i < n; ++i) { pm.p[i] = m[i]; ps.p[i] = sm[i]; pz.p[i] = zt[i]; }
  if (T > 0)
    hipLaunchKernelGGL(ce_combine_kernel, dim3((T + 255) / 256), dim3(256), 0, s, pm, ps, pz, n,
                       M, S, loss, T);
  if (loss_mean) hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, s, loss, T, loss_mean);
  return hipGetLastError();
}

hipError_t ce_bwd(bool bf16, const float* logits, const int32_t* targets, const float* M,
                  const float* S, float scale, void* dlogits, int64_t T, int64_t V_l, int64_t v0,
                  hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int bpr = static_cast<int>((V_l / 8 + 255) / 256);
  const dim3 g(static_cast<unsigned>(T * bpr));
  if (bf16)
    hipLaunchKernelGGL(ce_bwd_kernel<bf16_t>, g, dim3(256), 0, s, logits, targets, M, S, scale,
                       static_cast<bf16_t*>(dlogits), V_l, v0, bpr);
  else
    hipLaunchKernelGGL(ce_bwd_kernel<float>, g, dim3(256), 0, s, logits, targets, M, S, scale,
                       static_cast<float*>(dlogits), V_l, v0, bpr);
  return hipGetLastError();
}

}  // namespace mtp
