// Device-side helpers shared by the libmtp kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element type traits: float storage or bf16 storage, computed in fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f2bf(v); }
};

// Load / store 4 consecutive elements (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void load4(const float* p, float v[4]) {
  float4 t = *reinterpret_cast<const float4*>(p);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float v[4]) {
  uint2 t = *reinterpret_cast<const uint2*>(p);
  v[0] = lo_bf(t.x); v[1] = hi_bf(t.x); v[2] = lo_bf(t.y); v[3] = hi_bf(t.y);
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, const float v[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}

// Load / store 8 consecutive elements.
__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  uint4 t = *reinterpret_cast<const uint4*>(p);
  v[0] = lo_bf(t.x); v[1] = hi_bf(t.x); v[2] = lo_bf(t.y); v[3] = hi_bf(t.y);
  v[4] = lo_bf(t.z); v[5] = hi_bf(t.z); v[6] = lo_bf(t.w); v[7] = hi_bf(t.w);
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                            pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Transpose an 8x8 tile of bf16 held as 8 row vectors (row i = 8 values).
// Afterwards out[j] holds column j: out[j] element i = in[i] element j.
__device__ __forceinline__ void transpose8x8_bf16(const uint4 in[8], uint4 out[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);   // w[i*4 + c/2]
  uint32_t* o = reinterpret_cast<uint32_t*>(out);                // o[j*4 + i/2]
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const uint32_t a = w[(2 * i2) * 4 + j / 2];
      const uint32_t b = w[(2 * i2 + 1) * 4 + j / 2];
      o[j * 4 + i2] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u))
                              : ((a & 0xffffu) | (b << 16));
    }
  }
}

// GeLU, tanh form, and its derivative (fp32).  With z = c (u + a u^3),
// 0.5 (1 + tanh(z)) = sigmoid(2 z), so GeLU(u) = u * s with
// s = 1 / (1 + exp(-2 z)) (one v_exp_f32 and one v_rcp_f32), and
// GeLU'(u) = s + u s (1 - s) 2 c (1 + 3 a u^2).
constexpr float kGeluC = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float kGeluA = 0.044715f;
constexpr float kGeluK = -2.0f * kGeluC * 1.4426950408889634f;  // -2 c log2(e)
__device__ __forceinline__ float gelu_sigmoid(float u) {
  const float t = kGeluK * u * fmaf(kGeluA * u, u, 1.0f);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}
__device__ __forceinline__ float gelu_tanh(float u) { return u * gelu_sigmoid(u); }
__device__ __forceinline__ float gelu_tanh_grad(float u) {
  const float s = gelu_sigmoid(u);
  return s * fmaf(u * (1.0f - s) * (2.0f * kGeluC), fmaf(3.0f * kGeluA * u, u, 1.0f), 1.0f);
}

// SiLU(z) = z s, s = 1 / (1 + e^-z) (one v_exp_f32, one v_rcp_f32), and
// SiLU'(z) = s (1 + z (1 - s)).
constexpr float kNegLog2e = -1.4426950408889634f;
__device__ __forceinline__ float silu_sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(kNegLog2e * z));
}

// v combined with the value of lane ^ 32: v_permlane32_swap exchanges the
// two 32-lane halves without an LDS round trip; the pair it returns holds,
// in every lane, the lower-half value first and the upper-half value second.
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float warp_sum(float v) {
  v = xor32_sum(v);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
  v = xor32_max(v);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace mtp
