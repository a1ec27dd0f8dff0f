// HBM-bound kernels of the layer shard: LayerNorm forward/backward, the
// on-device sum of tensor-parallel partials, column sums (bias gradients)
// and the vocab-parallel cross-entropy pieces.  All loads and stores are
// 16-byte vectors of 8 consecutive elements along the contiguous axis;
// every reduction accumulates in fp32 in a fixed order (deterministic).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mtp {
namespace {

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kMaxRowChunks = 2048;  // rows of up to 16384 elements

template <typename T> __host__ __device__ __forceinline__ const T* cptr(const void* p) {
  return static_cast<const T*>(p);
}

// Load one row's NC chunks of 8 elements owned by a lane (chunks lane,
// lane+64, ...), every load issued before any use.
template <typename T, int NC>
__device__ __forceinline__ void load_row(const T* r, int lane, float v[NC][8]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) load8(r + (lane + 64 * c) * 8, v[c]);
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
// One wave per token row, four rows per workgroup; lane l owns 8-element
// chunks l, l+64, ...  Two passes over the register-cached row (NC chunks
// per lane; NC = 0 re-reads the row for rows wider than 4096): mean, then
// the centred second moment (population variance), by wave shuffles.
template <typename T, int NC>
__global__ void __launch_bounds__(256)
layernorm_fwd_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                     const T* __restrict__ beta, T* __restrict__ y, float* __restrict__ mean,
                     float* __restrict__ rstd, int64_t T_rows, int h, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T_rows) return;
  const int nchunk = h / 8;
  const T* xr = x + row * h;
  constexpr int kC = NC > 0 ? NC : 1;
  float v[kC][8];
  const int iters = NC > 0 ? NC : (nchunk + 63) / 64;
  float s = 0.0f;
  for (int i = 0; i < iters; ++i) {
    const int c = lane + i * 64;
    if (c < nchunk) {
      float t[8];
      load8(xr + c * 8, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s += t[e];
        if (NC > 0) v[i][e] = t[e];
      }
    }
  }
  const float mu = warp_sum(s) / h;
  float q = 0.0f;
  for (int i = 0; i < iters; ++i) {
    const int c = lane + i * 64;
    if (c < nchunk) {
      float t[8];
      if (NC > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = v[i][e];
      } else {
        load8(xr + c * 8, t);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float d = t[e] - mu; q += d * d; }
    }
  }
  const float rs = rsqrtf(warp_sum(q) / h + eps);
  for (int i = 0; i < iters; ++i) {
    const int c = lane + i * 64;
    if (c < nchunk) {
      float t[8], g[8], b[8], o[8];
      if (NC > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = v[i][e];
      } else {
        load8(xr + c * 8, t);
      }
      load8(gamma + c * 8, g);
      load8(beta + c * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (t[e] - mu) * rs * g[e] + b[e];
      store8(y + row * h + c * 8, o);
    }
  }
  if (lane == 0) { mean[row] = mu; rstd[row] = rs; }
}

// ----------------------------------------------------------- LayerNorm bwd
// Row pass: one wave per token row, four rows per workgroup, the two row
// means by wave shuffles only (no barrier):
//   xhat = (x-mu)*rstd, gh = dy*gamma,
//   dx = rstd*(gh - mean(gh) - xhat*mean(gh*xhat)) (+ dres).
// Lane l owns 8-element chunks l, l+64, ...  With NC > 0 the row's xhat and
// gh stay in registers (NC chunks per lane); NC = 0 re-reads x and dy for
// the second pass (rows wider than 4096).
template <typename T, int NC>
__global__ void __launch_bounds__(256)
layernorm_bwd_rows_kernel(const T* __restrict__ dy, const T* __restrict__ x,
                          const T* __restrict__ gamma, const float* __restrict__ mean,
                          const float* __restrict__ rstd, const T* __restrict__ dres,
                          T* __restrict__ dx, int64_t T_rows, int h) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T_rows) return;
  const int nchunk = h / 8;
  const float mu = mean[row], rs = rstd[row];
  const T* xr = x + row * h;
  const T* dr = dy + row * h;
  constexpr int kC = NC > 0 ? NC : 1;
  float xh[kC][8], gh[kC][8];
  float s1 = 0.0f, s2 = 0.0f;
  const int iters = NC > 0 ? NC : (nchunk + 63) / 64;
  for (int i = 0; i < iters; ++i) {
    const int c = lane + i * 64;
    if (c < nchunk) {
      float xv[8], dv[8], gv[8];
      load8(xr + c * 8, xv);
      load8(dr + c * 8, dv);
      load8(gamma + c * 8, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = (xv[e] - mu) * rs, g = dv[e] * gv[e];
        s1 += g;
        s2 += g * a;
        if (NC > 0) { xh[i][e] = a; gh[i][e] = g; }
      }
    }
  }
  const float m1 = warp_sum(s1) / h, m2 = warp_sum(s2) / h;
  for (int i = 0; i < iters; ++i) {
    const int c = lane + i * 64;
    if (c < nchunk) {
      float a[8], g[8], o[8];
      if (NC > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { a[e] = xh[i][e]; g[e] = gh[i][e]; }
      } else {
        float xv[8], dv[8], gv[8];
        load8(xr + c * 8, xv);
        load8(dr + c * 8, dv);
        load8(gamma + c * 8, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) { a[e] = (xv[e] - mu) * rs; g[e] = dv[e] * gv[e]; }
      }
      if (dres) {
        load8(dres + row * h + c * 8, o);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += rs * (g[e] - m1 - a[e] * m2);
      store8(dx + row * h + c * 8, o);
    }
  }
}

// bf16 rows whose width is a multiple of 512 (NC = h/512 chunks per lane):
// the same arithmetic with every load of the row issued before any use and
// the raw bf16 words kept in registers (4 VGPRs per 8 elements).
__device__ __forceinline__ float bfw(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? hi_bf(w) : lo_bf(w);
}

// Partial maximum of |output| of one workgroup for the FP8 scale of the
// tensor it writes (the convention of fp8_amax_parts_kernel: amax[b] for
// workgroup b, 0 in the slots no workgroup owns, so that the maximum over
// the kAmaxParts slots is the tensor's).  mx is the lane's maximum of the
// fp32 values it stored as bf16; rounding is monotonic, so the rounded
// maximum is the maximum of the stored values.  Every thread of the
// workgroup must call it (it has a barrier).
template <int NWAVES>
__device__ __forceinline__ void store_amax_part(float mx, float* amax) {
  __shared__ float wm[NWAVES];
  mx = warp_max(mx);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = wm[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) m = fmaxf(m, wm[w]);
    amax[blockIdx.x] = lo_bf(pack_bf2(m, 0.0f));
  }
  if (blockIdx.x == 0)
    for (int i = gridDim.x + threadIdx.x; i < kAmaxParts; i += NWAVES * 64) amax[i] = 0.0f;
}

template <int NC>
__global__ void __launch_bounds__(256)
layernorm_fwd_bf16_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ gamma,
                          const bf16_t* __restrict__ beta, bf16_t* __restrict__ y,
                          float* __restrict__ mean, float* __restrict__ rstd, int64_t T_rows,
                          int h, float eps, float* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  float mx = 0.0f;
  if (row < T_rows) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * h);
    uint4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = xr[lane + 64 * i];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += bfw(v[i], e);
    const float mu = warp_sum(s) / h;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float d = bfw(v[i], e) - mu; q += d * d; }
    const float rs = rsqrtf(warp_sum(q) / h + eps);
    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    const uint4* br = reinterpret_cast<const uint4*>(beta);
    uint4* yr = reinterpret_cast<uint4*>(y + row * h);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint4 g = gr[lane + 64 * i], b = br[lane + 64 * i];
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = (bfw(v[i], e) - mu) * rs * bfw(g, e) + bfw(b, e);
        mx = fmaxf(mx, fabsf(o[e]));
      }
      yr[lane + 64 * i] = make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]),
                                     pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7]));
    }
    if (lane == 0) { mean[row] = mu; rstd[row] = rs; }
  }
  if (amax) store_amax_part<4>(mx, amax);
}

template <int NC>
__global__ void __launch_bounds__(256)
layernorm_bwd_rows_bf16_kernel(const bf16_t* __restrict__ dy, const bf16_t* __restrict__ x,
                               const bf16_t* __restrict__ gamma, const float* __restrict__ mean,
                               const float* __restrict__ rstd, const bf16_t* __restrict__ dres,
                               bf16_t* __restrict__ dx, int64_t T_rows, int h) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T_rows) return;
  const float mu = mean[row], rs = rstd[row];
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * h);
  const uint4* dr = reinterpret_cast<const uint4*>(dy + row * h);
  const uint4* gr = reinterpret_cast<const uint4*>(gamma);
  uint4 xv[NC], dv[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) { xv[i] = xr[lane + 64 * i]; dv[i] = dr[lane + 64 * i]; }
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const uint4 g = gr[lane + 64 * i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = (bfw(xv[i], e) - mu) * rs, gh = bfw(dv[i], e) * bfw(g, e);
      s1 += gh;
      s2 += gh * a;
    }
  }
  const float m1 = warp_sum(s1) / h, m2 = warp_sum(s2) / h;
  const uint4* rr = reinterpret_cast<const uint4*>(dres + row * h);
  uint4* outr = reinterpret_cast<uint4*>(dx + row * h);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const uint4 g = gr[lane + 64 * i];
    const uint4 rv = dres ? rr[lane + 64 * i] : make_uint4(0, 0, 0, 0);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = (bfw(xv[i], e) - mu) * rs, gh = bfw(dv[i], e) * bfw(g, e);
      o[e] = bfw(rv, e) + rs * (gh - m1 - a * m2);
    }
    outr[lane + 64 * i] = make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]),
                                     pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7]));
  }
}

// Column pass: part_g[p][c] = sum over the rows of part p of dy*xhat,
// part_b[p][c] = sum of dy (rows ascending within a thread, the four row
// lanes added in order).  Workgroup (bx, by): columns [512 bx, 512 bx + 512),
// rows [by*rpb, (by+1)*rpb); 64 threads x 8 columns x 4 row lanes.
template <typename T>
__global__ void __launch_bounds__(256)
layernorm_bwd_cols_kernel(const T* __restrict__ dy, const T* __restrict__ x,
                          const float* __restrict__ mean, const float* __restrict__ rstd,
                          int64_t rows, int h, int rpb, float* __restrict__ part_g,
                          float* __restrict__ part_b) {
  __shared__ float red[2][4][512];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 512 + tx * 8;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rpb;
  const int64_t r1 = min(rows, r0 + rpb);
  float ag[8] = {0, 0, 0, 0, 0, 0, 0, 0}, ab[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c < h) {
#pragma unroll 8
    for (int64_t r = r0 + ty; r < r1; r += 4) {
      const float mu = mean[r], rs = rstd[r];
      float xv[8], dv[8];
      load8(x + r * h + c, xv);
      load8(dy + r * h + c, dv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ag[e] += dv[e] * ((xv[e] - mu) * rs);
        ab[e] += dv[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) { red[0][ty][tx * 8 + e] = ag[e]; red[1][ty][tx * 8 + e] = ab[e]; }
  __syncthreads();
  if (ty < 2 && c < h) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[e] = red[ty][0][tx * 8 + e] + red[ty][1][tx * 8 + e] + red[ty][2][tx * 8 + e] +
             red[ty][3][tx * 8 + e];
    store8((ty == 0 ? part_g : part_b) + static_cast<int64_t>(blockIdx.y) * h + c, o);
  }
}

// out[c] (=|+=) sum_{b < nparts} part[b*cols + c].  A workgroup owns 16
// columns (64-byte rows of the partial matrix) and 16 part lanes: lane ty
// sums parts ty, ty+16, ... in ascending order, then lane sums are added in
// ty order, so the result does not depend on scheduling.
constexpr int kRedCols = 16;
constexpr int kRedLanes = 16;
__global__ void __launch_bounds__(kRedCols * kRedLanes)
reduce_parts_kernel(const float* __restrict__ part0, float* __restrict__ out0,
                    const float* __restrict__ part1, float* __restrict__ out1, int nparts,
                    int64_t cols, int accumulate) {
  // blockIdx.y selects one of two independent (part, out) pairs.
  const float* part = blockIdx.y == 0 ? part0 : part1;
  float* out = blockIdx.y == 0 ? out0 : out1;
  __shared__ float red[kRedLanes][kRedCols];
  const int tx = threadIdx.x % kRedCols, ty = threadIdx.x / kRedCols;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRedCols + tx;
  float s = 0.0f;
  if (c < cols) {
    // eight loads in flight per thread; the additions stay in ascending b
    int b = ty;
    for (; b + 7 * kRedLanes < nparts; b += 8 * kRedLanes) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = part[static_cast<int64_t>(b + u * kRedLanes) * cols + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += t[u];
    }
    for (; b < nparts; b += kRedLanes) s += part[static_cast<int64_t>(b) * cols + c];
  }
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
#pragma unroll 8
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

// ------------------------------------------------------ FP8 quantization
// Per-tensor E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, largest finite value 448): s = amax / 448 in fp32, code =
// round-to-nearest-even(clamp(x / s, -448, 448)), with the fp32 quotient
// correctly rounded.  The rounding is done here from the format's
// definition rather than by a conversion instruction, so that the codes are
// those of that definition for every input.
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), kE4M3Max);
  const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xff) - 127;  // a > 0: floor(log2 a)
  if (e < -6) {
    // subnormal grid 2^-9 (and zero); 8 steps = 2^-6, which is code 0x08
    return sign | static_cast<uint32_t>(rintf(a * 512.0f));
  }
  // normal: a = m * 2^(e-3), m in [8, 16); rintf rounds half to even
  const uint32_t m = static_cast<uint32_t>(rintf(a * __uint_as_float(static_cast<uint32_t>(127 + 3 - e) << 23)));
  // m == 16 carries into the exponent: (e + 7) * 8 + 8 == (e + 8) * 8 + 0
  return sign | (static_cast<uint32_t>(e + 7) * 8u + (m - 8u));
}

__global__ void __launch_bounds__(64) fp8_amax_init_kernel(float* scale) { scale[1] = 0.0f; }

__global__ void __launch_bounds__(256) fp8_amax_kernel(const bf16_t* __restrict__ x, int64_t nvec,
                                                       float* scale) {
  float m = 0.0f;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    float t[8];
    load8(x + v * 8, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(t[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  // one atomic per workgroup (non-negative floats order like their bits)
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax(reinterpret_cast<unsigned int*>(scale + 1), __float_as_uint(m));
  }
}

__global__ void __launch_bounds__(256) fp8_quant_kernel(const bf16_t* __restrict__ x, int64_t nvec,
                                                        uint8_t* __restrict__ q, float* scale) {
  const float amax = scale[1];
  const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    float t[8];
    load8(x + v * 8, t);
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = e4m3_code(t[e] / s);
    const uint2 w = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                               c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
    *reinterpret_cast<uint2*>(q + v * 8) = w;
  }
}

// Code of |v| <= the format's largest value, in an 8-bit format with MANT
// mantissa bits and exponent bias BIAS (E4M3: 3, 7; E5M2: 2, 15), rounded to
// the nearest value, ties to the even mantissa, from the format's definition.
template <int MANT, int BIAS>
__device__ __forceinline__ uint32_t fp8_code(float v, float fmax) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), fmax);
  const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xff) - 127;  // a > 0: floor(log2 a)
  if (e < 1 - BIAS) {
    // subnormal grid 2^(1-BIAS-MANT), and zero; 2^MANT steps reach the
    // smallest normal value, whose code follows on
    return sign | static_cast<uint32_t>(
                      rintf(a * __uint_as_float(static_cast<uint32_t>(127 + BIAS - 1 + MANT) << 23)));
  }
  // normal: a = m * 2^(e-MANT), m in [2^MANT, 2^(MANT+1)); rintf rounds half
  // to even; m == 2^(MANT+1) carries into the exponent field
  const uint32_t m = static_cast<uint32_t>(
      rintf(a * __uint_as_float(static_cast<uint32_t>(127 + MANT - e) << 23)));
  return sign | ((static_cast<uint32_t>(e + BIAS) << MANT) + (m - (1u << MANT)));
}

// Partial maxima of |x| over n = 8 * nvec values: workgroup b of the fixed
// grid of kAmaxParts writes parts[b] (0 when it saw no element), so the
// maximum of the parts is max |x| without atomics or a reset.
__global__ void __launch_bounds__(256) fp8_amax_parts_kernel(const bf16_t* __restrict__ x,
                                                             int64_t nvec, float* parts) {
  float m = 0.0f;
  // four 16-byte loads in flight per lane
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; v + 3 * stride < nvec; v += 4 * stride) {
    uint4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = *reinterpret_cast<const uint4*>(x + (v + i * stride) * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[k] << 16)),
                           fabsf(__uint_as_float(w[k] & 0xffff0000u))));
    }
  }
  for (; v < nvec; v += stride) {
    float t[8];
    load8(x + v * 8, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(t[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) parts[blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

struct AmaxParts { const float* p[kMaxPartials]; int n; };

// x / s rounded to fp32 (the quotient the codes are defined on).  FAST: x * r
// corrected by one residual step, r = fl32(1 / s), the residual x - q0 s
// exact in an FMA, with the sign of x (the final sum would turn -0 into +0).
// Over every pair of bf16 values |x| <= amax with s = fl32(amax / fmax) in
// [2^-60, inf) this has the sign of the IEEE quotient and equals it wherever
// either magnitude reaches 2^-18; below that both round to the code of a
// signed zero in either format (checked exhaustively on the host).  Other
// scales divide.
template <bool FAST>
__device__ __forceinline__ float fp8_quotient(float x, float s, float r) {
  if constexpr (FAST) {
    const float q0 = __fmul_rn(x, r);
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0), x);
  } else {
    return x / s;
  }
}

// Codes of four fp32 values (|v| <= fmax) packed little-endian into a word:
// the conversion instruction rounds to nearest, ties to even, and keeps the
// subnormals of the format (E4M3: MANT 3; E5M2: MANT 2).
template <int MANT>
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
  if constexpr (MANT == 3) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
  } else {
    const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(c, d, lo, true));
  }
}

// Codes of x [rows, cols] (row-major bf16, cols % 8 == 0) with the scale
// s = amax / fmax, amax the maximum over the n arrays of kAmaxParts partial
// maxima (one array per shard of the tensor).  Each workgroup converts a
// tile of kQRows rows x kQCols columns and writes it row-major to q
// ([rows, cols]) and/or transposed to qt ([cols, rows]) through LDS.  A lane
// takes 4 consecutive rows x 8 columns, so it packs the 4 codes of each of
// its columns into one 4-byte LDS word; the transposed tile's rows are
// padded to 33 words, which puts the 64 lanes' words in 64 distinct banks.
constexpr int kQRows = 128, kQCols = 64, kQPitch = kQRows + 4;

// The codes of a lane's 4 rows x 8 columns: row-major words rw[i][0..1]
// (columns 0-3, 4-7 of row i) and, per column, the word of its 4 rows.
template <bool FAST, int MANT>
__device__ __forceinline__ void fp8_codes_4x8(const uint4 (&raw)[4], float s, float r, float fmax,
                                              uint32_t (&rw)[4][2], uint32_t (&col4)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = __builtin_amdgcn_fmed3f(fp8_quotient<FAST>(v[e], s, r), -fmax, fmax);
    rw[i][0] = fp8_pack4<MANT>(v[0], v[1], v[2], v[3]);
    rw[i][1] = fp8_pack4<MANT>(v[4], v[5], v[6], v[7]);
  }
  // 4x4 byte transposes: column e's word holds rows 0..3 in bytes 0..3
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a01 = __builtin_amdgcn_perm(rw[1][h], rw[0][h], 0x05010400u);  // r0c0 r1c0 r0c1 r1c1
    const uint32_t b01 = __builtin_amdgcn_perm(rw[1][h], rw[0][h], 0x07030602u);  // r0c2 r1c2 r0c3 r1c3
    const uint32_t a23 = __builtin_amdgcn_perm(rw[3][h], rw[2][h], 0x05010400u);
    const uint32_t b23 = __builtin_amdgcn_perm(rw[3][h], rw[2][h], 0x07030602u);
    col4[4 * h + 0] = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
    col4[4 * h + 1] = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
    col4[4 * h + 2] = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
    col4[4 * h + 3] = __builtin_amdgcn_perm(b23, b01, 0x07060302u);
  }
}

template <int MANT>
__global__ void __launch_bounds__(256)
fp8_convert_kernel(const bf16_t* __restrict__ x, int64_t rows, int cols, AmaxParts parts,
                   float fmax, uint8_t* __restrict__ q, uint8_t* __restrict__ qt, float* scale) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kQCols * kQPitch];
  const int tid = threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kQRows;
  const int c0 = blockIdx.x * kQCols;
  const int lc = (tid & 7) * 8, lg = tid >> 3;  // columns lc..lc+7, rows 4lg..4lg+3
  const int c = c0 + lc;
  // every load is issued before the scale is known; rows past the end read
  // as zeros (their codes are not stored)
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + 4 * lg + i;
    raw[i] = (r < rows && c < cols) ? *reinterpret_cast<const uint4*>(x + r * cols + c)
                                    : make_uint4(0, 0, 0, 0);
  }
  float m = 0.0f;
  for (int k = tid; k < parts.n * kAmaxParts; k += 256)
    m = fmaxf(m, parts.p[k / kAmaxParts][k % kAmaxParts]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / fmax : 1.0f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) scale[0] = s;
  uint32_t rw[4][2], col4[8];
  if (s >= 0x1p-60f && s < __builtin_huge_valf())
    fp8_codes_4x8<true, MANT>(raw, s, 1.0f / s, fmax, rw, col4);
  else
    fp8_codes_4x8<false, MANT>(raw, s, 1.0f, fmax, rw, col4);
  if (q && c < cols) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 4 * lg + i;
      if (r < rows) *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(rw[i][0], rw[i][1]);
    }
  }
  if (!qt) return;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint32_t*>(tile + (lc + e) * kQPitch + 4 * lg) = col4[e];
  __syncthreads();
  // transposed: output row oc (column c0 + oc) holds rows r0..r0+127; four
  // lanes per output row, 32 bytes each
  const int oc = tid >> 2, part = tid & 3;
  const int cc = c0 + oc;
  const int64_t rb = r0 + 32 * part;
  if (cc >= cols || rb >= rows) return;
  uint32_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = *reinterpret_cast<const uint32_t*>(tile + oc * kQPitch + 32 * part + 4 * j);
  uint8_t* dst = qt + static_cast<int64_t>(cc) * rows + rb;
  if (rb + 32 <= rows && (rows & 15) == 0) {
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(v[4], v[5], v[6], v[7]);
  } else {
    for (int e = 0; e < 32 && rb + e < rows; ++e) dst[e] = static_cast<uint8_t>(v[e >> 2] >> (8 * (e & 3)));
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

// The same sum for a compile-time number of partials N: every load of the
// thread's vector (the N partials, bias, residual) is issued before the first
// add, so the latency of one load is paid once per vector rather than once per
// operand.  Same fp32 order as partial_sum_kernel, so the same bits.
template <typename T, int N>
__global__ void __launch_bounds__(256)
partial_sum_n_kernel(PartialPtrs parts, const T* __restrict__ bias,
                     const T* __restrict__ residual, T* out, int64_t total, int h) {
  const int64_t nvec = total / 8;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t off = v * 8;
    float t[N][8], tb[8], tr[8];
#pragma unroll
    for (int i = 0; i < N; ++i) load8(static_cast<const T*>(parts.p[i]) + off, t[i]);
    if (bias) load8(bias + (off % h), tb);
    if (residual) load8(residual + off, tr);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += t[i][e];
    if (bias) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += tb[e];
    }
    if (residual) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += tr[e];
    }
    store8(out + off, acc);
  }
}

// Round 8 fp32 values to the storage type T in place (identity for fp32,
// round-to-nearest-even bf16 otherwise): the value a store + load would give.
template <typename T> __device__ __forceinline__ void round8(float v[8]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t w = pack_bf2(v[e], v[e + 1]);
      v[e] = lo_bf(w);
      v[e + 1] = hi_bf(w);
    }
  }
}

// ------------------------------------------- partial sum + LayerNorm fwd
// out = sum_i parts[i] (+ bias) (+ residual), rounded to T and stored, then
// the LayerNorm of that stored row: the arithmetic of partial_sum_kernel
// followed by that of the LayerNorm forward kernels, in one pass with the
// row in registers.  One wave per row, four rows per workgroup, h = 512*NC
// (lane l owns the 16-byte chunks l, l+64, ...).  A lane reads every
// element it writes before writing it, so out may alias an input.
// NP > 0 (bf16 only): NP partials known at compile time, and every load of
// the row (partials, bias, residual) is issued before the first add; the adds
// keep the order of the general path, so the bits are the same.
template <typename T, int NC, int NP = 0>
__global__ void __launch_bounds__(256)
sum_layernorm_fwd_kernel(PartialPtrs parts, int n, const T* __restrict__ bias,
                         const T* residual, T* out, const T* __restrict__ gamma,
                         const T* __restrict__ beta, T* __restrict__ y, float* __restrict__ mean,
                         float* __restrict__ rstd, int64_t T_rows, int h, float eps,
                         float* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  float mx = 0.0f;
  if (row < T_rows) {
    const int64_t base = row * h;
    float v[NC][8];
    if constexpr (NP > 0) {
      static_assert(sizeof(T) == 2, "compile-time partial count: bf16 rows");
      uint4 raw[NP][NC], rb[NC], rr[NC];
#pragma unroll
      for (int i = 0; i < NP; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          raw[i][c] = *reinterpret_cast<const uint4*>(static_cast<const T*>(parts.p[i]) + base +
                                                      (lane + 64 * c) * 8);
      if (bias) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          rb[c] = *reinterpret_cast<const uint4*>(bias + (lane + 64 * c) * 8);
      }
      if (residual) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          rr[c] = *reinterpret_cast<const uint4*>(residual + base + (lane + 64 * c) * 8);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = bfw(raw[0][c], e);
#pragma unroll
          for (int i = 1; i < NP; ++i) a += bfw(raw[i][c], e);
          if (bias) a += bfw(rb[c], e);
          if (residual) a += bfw(rr[c], e);
          v[c][e] = a;
        }
    } else {
      load_row<T, NC>(static_cast<const T*>(parts.p[0]) + base, lane, v);
      for (int i = 1; i < n; ++i) {
        float t[NC][8];
        load_row<T, NC>(static_cast<const T*>(parts.p[i]) + base, lane, t);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[c][e] += t[c][e];
      }
      if (bias) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float t[8];
          load8(bias + (lane + 64 * c) * 8, t);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[c][e] += t[e];
        }
      }
      if (residual) {
        float t[NC][8];
        load_row<T, NC>(residual + base, lane, t);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[c][e] += t[c][e];
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      round8<T>(v[c]);
      store8(out + base + (lane + 64 * c) * 8, v[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    const float mu = warp_sum(s) / h;
    float q = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float d = v[c][e] - mu; q += d * d; }
    const float rs = rsqrtf(warp_sum(q) / h + eps);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float g[8], b[8], o[8];
      load8(gamma + (lane + 64 * c) * 8, g);
      load8(beta + (lane + 64 * c) * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = (v[c][e] - mu) * rs * g[e] + b[e];
        mx = fmaxf(mx, fabsf(o[e]));
      }
      store8(y + base + (lane + 64 * c) * 8, o);
    }
    if (lane == 0) { mean[row] = mu; rstd[row] = rs; }
  }
  if (amax) store_amax_part<4>(mx, amax);
}

// ------------------------------------- LayerNorm bwd with column partials
// dy = sum_i dys[i], rounded to T when there is more than one part (the
// value partial_sum_kernel would store), then dx = dres + rstd*(gh -
// mean(gh) - xhat*mean(gh*xhat)), gh = dy*gamma, as in the row kernels
// above.  The same pass accumulates the column sums of dy*xhat and dy
// (dgamma, dbeta).  A workgroup has 8 waves; a row of h = 512*NC elements is
// held by SPLIT waves (NC/SPLIT 16-byte chunks per lane: SPLIT grows with
// the row width so that the registers allow two waves per SIMD), so
// 8/SPLIT rows are in flight per iteration and the SPLIT waves of a row add
// their two row sums through LDS (in wave order).  Row slot q of workgroup b takes rows
// q + (8/SPLIT)*b + k*(8/SPLIT)*gridDim.x.  Each lane sums dy*xhat and dy
// over its rows; the slots' sums are then added in slot order through LDS
// and workgroup b writes row b of the partial matrices, which
// reduce_parts_kernel adds in workgroup order.
template <typename T, int NC, int SPLIT>
__global__ void __launch_bounds__(512)
layernorm_bwd_fused_kernel(PartialPtrs dys, int n, const T* __restrict__ x,
                           const T* __restrict__ gamma, const float* __restrict__ mean,
                           const float* __restrict__ rstd, const T* dres, T* dx, int64_t T_rows,
                           int h, float* __restrict__ part_g, float* __restrict__ part_b,
                           float* __restrict__ amax) {
  constexpr int NCW = NC / SPLIT;     // chunks per lane
  constexpr int kSlots = 8 / SPLIT;   // rows per iteration
  __shared__ float red[2][512 * NC];
  __shared__ float xch[2][8][2];      // [iteration parity][wave][s1, s2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = wave / SPLIT, half = wave % SPLIT;
  // chunk c of this lane starts at element col(c)
  auto col = [&](int c) { return ((half * NCW + c) * 64 + lane) * 8; };
  float gm[NCW][8], ag[NCW][8], ab[NCW][8];
#pragma unroll
  for (int c = 0; c < NCW; ++c) {
    load8(gamma + col(c), gm[c]);
#pragma unroll
    for (int e = 0; e < 8; ++e) { ag[c][e] = 0.0f; ab[c][e] = 0.0f; }
  }
  float mx = 0.0f;  // max |dx| stored by this lane
  const int64_t per_iter = static_cast<int64_t>(gridDim.x) * kSlots;
  const int64_t iters = (T_rows + per_iter - 1) / per_iter;  // the same for every wave
  for (int64_t k = 0; k < iters; ++k) {
    const int64_t row = k * per_iter + static_cast<int64_t>(blockIdx.x) * kSlots + slot;
    const bool valid = row < T_rows;
    const int64_t base = row * h;
    float xv[NCW][8], dv[NCW][8];
    float s1 = 0.0f, s2 = 0.0f, rs = 0.0f;
    if (valid) {
#pragma unroll
      for (int c = 0; c < NCW; ++c) load8(x + base + col(c), xv[c]);
#pragma unroll
      for (int c = 0; c < NCW; ++c) load8(static_cast<const T*>(dys.p[0]) + base + col(c), dv[c]);
      for (int i = 1; i < n; ++i) {
        const T* src = static_cast<const T*>(dys.p[i]) + base;
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
          float t[8];
          load8(src + col(c), t);
#pragma unroll
          for (int e = 0; e < 8; ++e) dv[c][e] += t[e];
        }
      }
      if (n > 1) {
#pragma unroll
        for (int c = 0; c < NCW; ++c) round8<T>(dv[c]);
      }
      const float mu = mean[row];
      rs = rstd[row];
#pragma unroll
      for (int c = 0; c < NCW; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = (xv[c][e] - mu) * rs, g = dv[c][e] * gm[c][e];
          s1 += g;
          s2 += g * a;
          xv[c][e] = a;
          ag[c][e] += dv[c][e] * a;
          ab[c][e] += dv[c][e];
        }
    }
    s1 = warp_sum(s1);
    s2 = warp_sum(s2);
    if constexpr (SPLIT > 1) {
      const int par = static_cast<int>(k & 1);
      if (lane == 0) { xch[par][wave][0] = s1; xch[par][wave][1] = s2; }
      __syncthreads();
      s1 = 0.0f;
      s2 = 0.0f;
#pragma unroll
      for (int w = 0; w < SPLIT; ++w) {
        s1 += xch[par][slot * SPLIT + w][0];
        s2 += xch[par][slot * SPLIT + w][1];
      }
    }
    if (valid) {
      const float m1 = s1 / h, m2 = s2 / h;
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        float o[8];
        if (dres) {
          load8(dres + base + col(c), o);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] += rs * (dv[c][e] * gm[c][e] - m1 - xv[c][e] * m2);
          mx = fmaxf(mx, fabsf(o[e]));
        }
        store8(dx + base + col(c), o);
      }
    }
  }
  for (int q = 0; q < kSlots; ++q) {
    if (slot == q) {
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        float4* rg = reinterpret_cast<float4*>(&red[0][col(c)]);
        float4* rb = reinterpret_cast<float4*>(&red[1][col(c)]);
        float4 g0 = make_float4(ag[c][0], ag[c][1], ag[c][2], ag[c][3]);
        float4 g1 = make_float4(ag[c][4], ag[c][5], ag[c][6], ag[c][7]);
        float4 b0 = make_float4(ab[c][0], ab[c][1], ab[c][2], ab[c][3]);
        float4 b1 = make_float4(ab[c][4], ab[c][5], ab[c][6], ab[c][7]);
        if (q > 0) {
          const float4 pg0 = rg[0], pg1 = rg[1], pb0 = rb[0], pb1 = rb[1];
          g0 = make_float4(pg0.x + g0.x, pg0.y + g0.y, pg0.z + g0.z, pg0.w + g0.w);
          g1 = make_float4(pg1.x + g1.x, pg1.y + g1.y, pg1.z + g1.z, pg1.w + g1.w);
          b0 = make_float4(pb0.x + b0.x, pb0.y + b0.y, pb0.z + b0.z, pb0.w + b0.w);
          b1 = make_float4(pb1.x + b1.x, pb1.y + b1.y, pb1.z + b1.z, pb1.w + b1.w);
        }
        rg[0] = g0; rg[1] = g1; rb[0] = b0; rb[1] = b1;
      }
    }
    __syncthreads();
  }
  float4* og = reinterpret_cast<float4*>(part_g + static_cast<int64_t>(blockIdx.x) * h);
  float4* ob = reinterpret_cast<float4*>(part_b + static_cast<int64_t>(blockIdx.x) * h);
  const float4* rg = reinterpret_cast<const float4*>(red[0]);
  const float4* rb = reinterpret_cast<const float4*>(red[1]);
  for (int i = threadIdx.x; i < h / 4; i += 512) { og[i] = rg[i]; ob[i] = rb[i]; }
  if (amax) store_amax_part<8>(mx, amax);
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
              T* __restrict__ dlogits, int64_t V_l, int64_t v0, int64_t V, int blocks_per_row) {
  const int64_t row = blockIdx.x / blocks_per_row;
  const int64_t c = (static_cast<int64_t>(blockIdx.x % blocks_per_row) * 256 + threadIdx.x) * 8;
  if (c >= V_l) return;
  const int64_t id = targets[row];
  float v[8];
  if (id < 0 || id >= V) {
    // an id outside the vocabulary has no gradient: the row is NaN, as its
    // loss is in the stats
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_nanf("");
    store8(dlogits + row * V_l + c, v);
    return;
  }
  const float m = M[row], inv = 1.0f / S[row];
  const int64_t tg = id - v0;
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

constexpr int kColRowsPerPart = 32;

int64_t colsum_parts(int64_t rows) {
  int64_t p = (rows + kColRowsPerPart - 1) / kColRowsPerPart;
  return p > 256 ? 256 : p;
}

// ---------------------------------------------------------------- launchers

// Returns whether the kernel also wrote the partial maxima of |y| (amax given,
// the bf16 row kernel, and at most kAmaxParts workgroups).
template <typename T>
bool ln_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean,
            float* rstd, int64_t T_rows, int h, float eps, float* amax, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T_rows + 3) / 4));
  const int per_lane = (h / 8 + 63) / 64;
  if (sizeof(T) == 2 && h % 512 == 0 && per_lane <= 16) {
    float* am = (amax && grid.x <= static_cast<unsigned>(kAmaxParts)) ? amax : nullptr;
#define MTP_LN_FWD16(NC)                                                                     \
  hipLaunchKernelGGL((layernorm_fwd_bf16_kernel<NC>), grid, dim3(256), 0, s, cptr<bf16_t>(x), \
                     cptr<bf16_t>(gamma), cptr<bf16_t>(beta), static_cast<bf16_t*>(y), mean, \
                     rstd, T_rows, h, eps, am)
    switch (per_lane) {
      case 1: MTP_LN_FWD16(1); return am != nullptr;
      case 2: MTP_LN_FWD16(2); return am != nullptr;
      case 4: MTP_LN_FWD16(4); return am != nullptr;
      case 8: MTP_LN_FWD16(8); return am != nullptr;
      case 16: MTP_LN_FWD16(16); return am != nullptr;
      default: break;
    }
#undef MTP_LN_FWD16
  }
#define MTP_LN_FWD(NC)                                                                       \
  hipLaunchKernelGGL((layernorm_fwd_kernel<T, NC>), grid, dim3(256), 0, s, cptr<T>(x),          \
                     cptr<T>(gamma), cptr<T>(beta), static_cast<T*>(y), mean, rstd, T_rows, h, \
                     eps)
  if (per_lane <= 1) MTP_LN_FWD(1);
  else if (per_lane <= 2) MTP_LN_FWD(2);
  else if (per_lane <= 4) MTP_LN_FWD(4);
  else if (per_lane <= 8) MTP_LN_FWD(8);
  else MTP_LN_FWD(0);
#undef MTP_LN_FWD
  return false;
}

template <typename T>
void ln_bwd_rows(const void* dy, const void* x, const void* gamma, const float* mean,
                 const float* rstd, const void* dres, void* dx, int64_t T_rows, int h,
                 hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((T_rows + 3) / 4));
  const int per_lane = (h / 8 + 63) / 64;
  if (sizeof(T) == 2 && h % 512 == 0 && per_lane <= 16) {
#define MTP_LN_BWD16(NC)                                                                      \
  hipLaunchKernelGGL((layernorm_bwd_rows_bf16_kernel<NC>), grid, dim3(256), 0, s,               \
                     cptr<bf16_t>(dy), cptr<bf16_t>(x), cptr<bf16_t>(gamma), mean, rstd,       \
                     cptr<bf16_t>(dres), static_cast<bf16_t*>(dx), T_rows, h)
    switch (per_lane) {
      case 1: MTP_LN_BWD16(1); return;
      case 2: MTP_LN_BWD16(2); return;
      case 4: MTP_LN_BWD16(4); return;
      case 8: MTP_LN_BWD16(8); return;
      case 16: MTP_LN_BWD16(16); return;
      default: break;
    }
#undef MTP_LN_BWD16
  }
#define MTP_LN_BWD_ROWS(NC)                                                                  \
  hipLaunchKernelGGL((layernorm_bwd_rows_kernel<T, NC>), grid, dim3(256), 0, s, cptr<T>(dy),  \
                     cptr<T>(x), cptr<T>(gamma), mean, rstd, cptr<T>(dres),                 \
                     static_cast<T*>(dx), T_rows, h)
  if (per_lane <= 1) MTP_LN_BWD_ROWS(1);
  else if (per_lane <= 2) MTP_LN_BWD_ROWS(2);
  else if (per_lane <= 4) MTP_LN_BWD_ROWS(4);
  else if (per_lane <= 8) MTP_LN_BWD_ROWS(8);
  else MTP_LN_BWD_ROWS(0);
#undef MTP_LN_BWD_ROWS
}

}  // namespace

hipError_t layernorm_fwd(bool bf16, const void* x, const void* gamma, const void* beta, void* y,
                         float* mean, float* rstd, int64_t T, int h, float eps, float* amax,
                         hipStream_t s) {
  if (h / 8 > kMaxRowChunks) return hipErrorInvalidValue;
  bool fused = false;
  if (T > 0) {
    if (bf16) fused = ln_fwd<bf16_t>(x, gamma, beta, y, mean, rstd, T, h, eps, amax, s);
    else fused = ln_fwd<float>(x, gamma, beta, y, mean, rstd, T, h, eps, amax, s);
  }
  if (amax && !fused) return fp8_amax(y, T * h, amax, s);
  return hipGetLastError();
}

// Workgroups of the fused LayerNorm backward: one per 8 rows, at most 256
// (each writes one row of column partials).
static int64_t ln_bwd_blocks(int64_t T) {
  const int64_t b = (T + 7) / 8;
  return b > 256 ? 256 : b;
}

// Chunks per lane of a one-wave-per-row fused kernel (h = 512*NC), 0 if h
// does not fit (the partial sum + LayerNorm forward).
static int fused_row_nc(int h) {
  if (h % 512 != 0) return 0;
  const int nc = h / 512;
  return (nc == 1 || nc == 2 || nc == 4 || nc == 8) ? nc : 0;
}

// Chunks per row of the fused LayerNorm backward (a row split over up to 8
// waves), 0 if h does not fit.
static int fused_bwd_nc(int h) {
  if (h % 512 != 0) return 0;
  const int nc = h / 512;
  return (nc == 1 || nc == 2 || nc == 4 || nc == 8 || nc == 16 || nc == 24 || nc == 32) ? nc : 0;
}

static size_t round_up256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t layernorm_bwd_ws_bytes(int64_t T, int h, bool bf16) {
  const size_t parts = round_up256(static_cast<size_t>(ln_bwd_blocks(T)) * h * 2 * sizeof(float));
  // rows too wide for the fused kernel stage the summed gradient here
  const size_t stage = fused_bwd_nc(h) ? 0 : static_cast<size_t>(T) * h * (bf16 ? 2 : 4);
  return parts + stage;
}

hipError_t sum_layernorm_fwd(bool bf16, const void* const* partials, int n, const void* bias,
                             const void* residual, void* out, const void* gamma,
                             const void* beta, void* y, float* mean, float* rstd, int64_t T,
                             int h, float eps, float* amax, hipStream_t s) {
  if (h / 8 > kMaxRowChunks || n < 1 || n > kMaxPartials) return hipErrorInvalidValue;
  if (T == 0) return amax ? fp8_amax(y, 0, amax, s) : hipSuccess;
  const int nc = fused_row_nc(h);
  if (nc == 0) {
    const hipError_t e = partial_sum(bf16, partials, n, bias, residual, out, T, h, s);
    if (e != hipSuccess) return e;
    return layernorm_fwd(bf16, out, gamma, beta, y, mean, rstd, T, h, eps, amax, s);
  }
  PartialPtrs pp{};
  for (int i = 0; i < n; ++i) pp.p[i] = partials[i];
  const dim3 grid(static_cast<unsigned>((T + 3) / 4));
  float* am = (amax && bf16 && grid.x <= static_cast<unsigned>(kAmaxParts)) ? amax : nullptr;
#define MTP_SUM_LN(TT, NC, NP)                                                                 \
  hipLaunchKernelGGL((sum_layernorm_fwd_kernel<TT, NC, NP>), grid, dim3(256), 0, s, pp, n,       \
                     cptr<TT>(bias), cptr<TT>(residual), static_cast<TT*>(out), cptr<TT>(gamma), \
                     cptr<TT>(beta), static_cast<TT*>(y), mean, rstd, T, h, eps, am)
#define MTP_SUM_LN_T(TT, NP)                  \
  switch (nc) {                               \
    case 1: MTP_SUM_LN(TT, 1, NP); break;     \
    case 2: MTP_SUM_LN(TT, 2, NP); break;     \
    case 4: MTP_SUM_LN(TT, 4, NP); break;     \
    default: MTP_SUM_LN(TT, 8, NP); break;    \
  }
  if (bf16) {
    switch (n) {
      case 1: MTP_SUM_LN_T(bf16_t, 1) break;
      case 2: MTP_SUM_LN_T(bf16_t, 2) break;
      case 4: MTP_SUM_LN_T(bf16_t, 4) break;
      default: MTP_SUM_LN_T(bf16_t, 0) break;
    }
  } else {
    MTP_SUM_LN_T(float, 0)
  }
#undef MTP_SUM_LN_T
#undef MTP_SUM_LN
  if (amax && !am) return fp8_amax(y, T * h, amax, s);
  return hipGetLastError();
}

hipError_t layernorm_bwd_sum(bool bf16, const void* const* dys, int n, const void* x,
                             const void* gamma, const float* mean, const float* rstd,
                             const void* dres, void* dx, float* dgamma, float* dbeta,
                             bool accumulate, int64_t T, int h, void* ws, float* amax,
                             hipStream_t s) {
  if (h / 8 > kMaxRowChunks || n < 1 || n > kMaxPartials) return hipErrorInvalidValue;
  const int nc = fused_bwd_nc(h);
  float* pg = static_cast<float*>(ws);
  const dim3 rg((h + kRedCols - 1) / kRedCols, 2);
  if (nc == 0) {
    // Wide or unaligned rows: the sum (if any) goes to the staging area,
    // then the row pass and the column pass run separately.
    const int64_t parts = colsum_parts(T);
    float* pb = pg + parts * h;
    const void* dy = dys[0];
    if (n > 1 && T > 0) {
      void* stage = static_cast<char*>(ws) +
                    round_up256(static_cast<size_t>(ln_bwd_blocks(T)) * h * 2 * sizeof(float));
      const hipError_t e = partial_sum(bf16, dys, n, nullptr, nullptr, stage, T, h, s);
      if (e != hipSuccess) return e;
      dy = stage;
    }
    if (T > 0) {
      if (bf16) ln_bwd_rows<bf16_t>(dy, x, gamma, mean, rstd, dres, dx, T, h, s);
      else ln_bwd_rows<float>(dy, x, gamma, mean, rstd, dres, dx, T, h, s);
      const int rpb = static_cast<int>((T + parts - 1) / parts);
      const dim3 g((h + 511) / 512, static_cast<unsigned>(parts));
      if (bf16)
        hipLaunchKernelGGL(layernorm_bwd_cols_kernel<bf16_t>, g, dim3(256), 0, s,
                           cptr<bf16_t>(dy), cptr<bf16_t>(x), mean, rstd, T, h, rpb, pg, pb);
      else
        hipLaunchKernelGGL(layernorm_bwd_cols_kernel<float>, g, dim3(256), 0, s,
                           cptr<float>(dy), cptr<float>(x), mean, rstd, T, h, rpb, pg, pb);
    }
    hipLaunchKernelGGL(reduce_parts_kernel, rg, dim3(kRedCols * kRedLanes), 0, s, pg, dgamma, pb,
                       dbeta, static_cast<int>(T > 0 ? parts : 0), static_cast<int64_t>(h),
                       accumulate ? 1 : 0);
    if (amax) return fp8_amax(dx, T * h, amax, s);
    return hipGetLastError();
  }
  const int64_t blocks = ln_bwd_blocks(T);
  float* pb = pg + blocks * h;
  // at most 256 workgroups: the partial maxima of |dx| fit kAmaxParts
  float* am = (amax && bf16 && T > 0) ? amax : nullptr;
  if (T > 0) {
    PartialPtrs pp{};
    for (int i = 0; i < n; ++i) pp.p[i] = dys[i];
    const dim3 grid(static_cast<unsigned>(blocks));
#define MTP_LN_BWD_F(TT, NC, SPLIT)                                                             \
  hipLaunchKernelGGL((layernorm_bwd_fused_kernel<TT, NC, SPLIT>), grid, dim3(512), 0, s, pp, n,   \
                     cptr<TT>(x), cptr<TT>(gamma), mean, rstd, cptr<TT>(dres),                   \
                     static_cast<TT*>(dx), T, h, pg, pb, am)
#define MTP_LN_BWD_F_T(TT)                      \
  switch (nc) {                                 \
    case 1: MTP_LN_BWD_F(TT, 1, 1); break;      \
    case 2: MTP_LN_BWD_F(TT, 2, 1); break;      \
    case 4: MTP_LN_BWD_F(TT, 4, 1); break;      \
    case 8: MTP_LN_BWD_F(TT, 8, 2); break;      \
    case 16: MTP_LN_BWD_F(TT, 16, 4); break;    \
    case 24: MTP_LN_BWD_F(TT, 24, 8); break;    \
    default: MTP_LN_BWD_F(TT, 32, 8); break;    \
  }
    if (bf16) { MTP_LN_BWD_F_T(bf16_t) } else { MTP_LN_BWD_F_T(float) }
#undef MTP_LN_BWD_F_T
#undef MTP_LN_BWD_F
  }
  hipLaunchKernelGGL(reduce_parts_kernel, rg, dim3(kRedCols * kRedLanes), 0, s, pg, dgamma, pb,
                     dbeta, static_cast<int>(T > 0 ? blocks : 0), static_cast<int64_t>(h),
                     accumulate ? 1 : 0);
  if (amax && !am) return fp8_amax(dx, T * h, amax, s);
  return hipGetLastError();
}

hipError_t layernorm_bwd(bool bf16, const void* dy, const void* x, const void* gamma,
                         const float* mean, const float* rstd, const void* dres, void* dx,
                         float* dgamma, float* dbeta, bool accumulate, int64_t T, int h,
                         void* ws, hipStream_t s) {
  const void* dys[1] = {dy};
  return layernorm_bwd_sum(bf16, dys, 1, x, gamma, mean, rstd, dres, dx, dgamma, dbeta,
                           accumulate, T, h, ws, nullptr, s);
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
  hipLaunchKernelGGL(reduce_parts_kernel, dim3((cols + kRedCols - 1) / kRedCols, 1),
                     dim3(kRedCols * kRedLanes), 0, s, part, out, part, out,
                     static_cast<int>(rows > 0 ? parts : 0), cols, accumulate ? 1 : 0);
  return hipGetLastError();
}

hipError_t partial_sum(bool bf16, const void* const* partials, int n, const void* bias,
                       const void* residual, void* out, int64_t T, int h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  PartialPtrs pp{};
  for (int i = 0; i < n; ++i) pp.p[i] = partials[i];
  const int64_t total = T * h;
  const int grid = grid_for(total / 8);
  if (bf16 && (n == 1 || n == 2 || n == 4)) {
    auto* k = n == 1 ? partial_sum_n_kernel<bf16_t, 1>
              : n == 2 ? partial_sum_n_kernel<bf16_t, 2> : partial_sum_n_kernel<bf16_t, 4>;
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, pp, cptr<bf16_t>(bias),
                       cptr<bf16_t>(residual), static_cast<bf16_t*>(out), total, h);
    return hipGetLastError();
  }
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
                  int64_t V, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int bpr = static_cast<int>((V_l / 8 + 255) / 256);
  const dim3 g(static_cast<unsigned>(T * bpr));
  if (bf16)
    hipLaunchKernelGGL(ce_bwd_kernel<bf16_t>, g, dim3(256), 0, s, logits, targets, M, S, scale,
                       static_cast<bf16_t*>(dlogits), V_l, v0, V, bpr);
  else
    hipLaunchKernelGGL(ce_bwd_kernel<float>, g, dim3(256), 0, s, logits, targets, M, S, scale,
                       static_cast<float*>(dlogits), V_l, v0, V, bpr);
  return hipGetLastError();
}

hipError_t fp8_amax(const void* x, int64_t n, float* parts, hipStream_t s) {
  hipLaunchKernelGGL(fp8_amax_parts_kernel, dim3(kAmaxParts), dim3(256), 0, s, cptr<bf16_t>(x),
                     n / 8, parts);
  return hipGetLastError();
}

hipError_t fp8_quantize(int fmt, const void* x, int64_t rows, int cols, const float* const* parts,
                        int n_parts, uint8_t* q, uint8_t* qt, float* scale, hipStream_t s) {
  if (n_parts < 1 || n_parts > kMaxPartials || (cols & 7) || cols <= 0 || rows < 0)
    return hipErrorInvalidValue;
  AmaxParts ap{};
  for (int i = 0; i < n_parts; ++i) ap.p[i] = parts[i];
  ap.n = n_parts;
  const int64_t rt = rows > 0 ? (rows + kQRows - 1) / kQRows : 1;
  if (rt > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((cols + kQCols - 1) / kQCols), static_cast<unsigned>(rt));
  if (fmt == kFp8E5M2)
    hipLaunchKernelGGL((fp8_convert_kernel<2>), grid, dim3(256), 0, s, cptr<bf16_t>(x), rows,
                       cols, ap, 57344.0f, q, qt, scale);
  else
    hipLaunchKernelGGL((fp8_convert_kernel<3>), grid, dim3(256), 0, s, cptr<bf16_t>(x), rows,
                       cols, ap, kE4M3Max, q, qt, scale);
  return hipGetLastError();
}

hipError_t quantize_fp8(const void* x, int64_t n, uint8_t* q, float* scale, hipStream_t s) {
  hipLaunchKernelGGL(fp8_amax_init_kernel, dim3(1), dim3(64), 0, s, scale);
  if (n <= 0) {
    hipLaunchKernelGGL(fp8_quant_kernel, dim3(1), dim3(256), 0, s, cptr<bf16_t>(x), int64_t{0}, q,
                       scale);
    return hipGetLastError();
  }
  const int64_t nvec = n / 8;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((nvec + 255) / 256, 2048));
  const unsigned agrid = std::min(grid, 256u);  // at most 256 same-address atomics
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(agrid), dim3(256), 0, s, cptr<bf16_t>(x), nvec, scale);
  hipLaunchKernelGGL(fp8_quant_kernel, dim3(grid), dim3(256), 0, s, cptr<bf16_t>(x), nvec, q, scale);
  return hipGetLastError();
}

}  // namespace mtp
