// Softmax attention over the rank's local heads, forward and backward.
//
// The head split needs no exchange between ranks (page "Megatron-LM 3D
// parallelism guide", §2.1): each rank attends over its own a_l heads.  The
// softmax runs in fp32 (the attention_softmax_in_fp32 flag, §3.2 of the same
// page).  Key j is visible to query i iff start(i) <= j <= i, start(i) being
// the first token of i's sequence (fixed-length micro-batch or packed
// variable-length documents given by cu_seqlens).
//
// bf16 path (CDNA4 MFMA, v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//  * forward and dQ work on 128 queries per workgroup (4 waves x 32) and
//    compute S^T = K Q^T so that every lane owns one query: the row max and
//    row sum of the online softmax are in-lane except for one exchange with
//    the partner lane (lane ^ 32).  The probabilities then feed the next MFMA
//    straight from the accumulator registers as its B operand: within each
//    16-key step the lane holds keys {4g..4g+3, 8+4g..8+4g+3} (g = lane/32),
//    so the transposed LDS tiles (V^T, K^T) store their 16-byte chunks in
//    that key order.
//  * dK/dV works on 128 keys per workgroup (4 waves x 32 keys) and loops over
//    query tiles; S = Q K^T puts one key per lane, and P / dS feed the dV^T /
//    dK^T MFMAs from registers against transposed dO / Q tiles.
//  * dQ is a separate query-major pass (no atomics, deterministic).
// fp32 path: plain SIMT kernels (one query or key per workgroup).
#include "common.h"
#include "kernels.h"

namespace mtp {
namespace {

constexpr int kBQ = 128;   // queries per workgroup (forward, dQ)
constexpr int kBKV = 64;   // keys per LDS tile (forward, dQ)
constexpr int kBK2 = 128;  // keys per workgroup (dK/dV)
constexpr int kBQ2 = 64;   // queries per LDS tile (dK/dV)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
  const void* qkv; int64_t ld;      // [T, 3*hl]
  void* ctx;                        // [T, hl]
  float* lse;                       // [heads, T] natural log
  const void* dctx;                 // [T, hl]
  void* dqkv;                       // [T, 3*hl]
  float* delta;                     // [heads, T]
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

// ------------------------------------------------------------ tile staging
// A tile is 64 rows x D columns of one head, read as 8x8 blocks (8 rows x 16
// bytes).  Block b covers rows (b / (D/8))*8 .. +7 and columns (b % (D/8))*8.
template <int D>
__device__ __forceinline__ void load_block(const bf16_t* base, int64_t ld, int row0, int T,
                                           int b, uint4 r[8]) {
  constexpr int DC = D / 8;
  const int rb = b / DC, dc = b % DC;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = row0 + rb * 8 + i;
    r[i] = row < T ? *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(row) * ld + dc * 8)
                   : make_uint4(0, 0, 0, 0);
  }
}

// Natural layout [64][D]: row r, chunk c at slot r*DC + (c ^ (r & 7)).
template <int D>
__device__ __forceinline__ void store_natural(uint4* lds, int b, const uint4 r[8]) {
  constexpr int DC = D / 8;
  const int rb = b / DC, dc = b % DC;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rb * 8 + i;
    lds[row * DC + (dc ^ (row & 7))] = r[i];
  }
}

// Transposed layout [D][64]: row d has 8 chunks; logical chunk 2t+g holds
// columns 16t + {4g..4g+3} then 16t + 8 + {4g..4g+3}; it is stored at slot
// (2t+g) ^ (d & 7).
template <int D>
__device__ __forceinline__ void store_transposed(uint4* lds, int b, const uint4 r[8]) {
  constexpr int DC = D / 8;
  const int rb = b / DC, dc = b % DC;
  const int t = rb >> 1, half = rb & 1;
  uint4 tr[8];
  transpose8x8_bf16(r, tr);
  uint2* l2 = reinterpret_cast<uint2*>(lds);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = dc * 8 + j;
    const int s0 = (2 * t) ^ (row & 7), s1 = (2 * t + 1) ^ (row & 7);
    l2[(row * 8 + s0) * 2 + half] = make_uint2(tr[j].x, tr[j].y);
    l2[(row * 8 + s1) * 2 + half] = make_uint2(tr[j].z, tr[j].w);
  }
}

template <int D>
__device__ __forceinline__ bf16x8 read_natural(const uint4* lds, int row, int chunk) {
  return __builtin_bit_cast(bf16x8, lds[row * (D / 8) + (chunk ^ (row & 7))]);
}
__device__ __forceinline__ bf16x8 read_transposed(const uint4* lds, int row, int chunk) {
  return __builtin_bit_cast(bf16x8, lds[row * 8 + (chunk ^ (row & 7))]);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const f32x16& a, int off) {
  uint4 u;
  u.x = pack_bf2(a[off + 0], a[off + 1]);
  u.y = pack_bf2(a[off + 2], a[off + 3]);
  u.z = pack_bf2(a[off + 4], a[off + 5]);
  u.w = pack_bf2(a[off + 6], a[off + 7]);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 load_frag(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 zero_frag() {
  return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

// ------------------------------------------------------------- forward
template <int D>
__global__ void __launch_bounds__(256) attn_fwd_bf16(AttnParams p) {
  constexpr int DC = D / 8, KS = D / 16, MB = D / 32;
  __shared__ uint4 k_lds[2][kBKV * DC];
  __shared__ uint4 vt_lds[2][D * 8];
  const int T = p.T;
  const int nqb = (T + kBQ - 1) / kBQ;
  const int head = blockIdx.x % p.heads;
  const int q0 = (nqb - 1 - static_cast<int>(blockIdx.x) / p.heads) * kBQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;
  const int q0w = q0 + wave * 32;
  const int qi = q0w + lq;
  const bool qvalid = qi < T;
  const bool wave_active = q0w < T;
  const int qstart = seq_start(p, min(qi, T - 1));
  const int wlast = min(q0w + 31, T - 1);
  const int w_lo = seq_start(p, min(q0w, T - 1));
  const int w_smax = seq_start(p, wlast);
  const int kv_lo = seq_start(p, q0);
  const int kv_hi = min(T, q0 + kBQ);
  const int ntiles = (kv_hi - kv_lo + kBKV - 1) / kBKV;

  const bf16_t* qkv = static_cast<const bf16_t*>(p.qkv);
  const bf16_t* qb = qkv + head * D;
  const bf16_t* kb = qkv + p.hl + head * D;
  const bf16_t* vb = qkv + 2 * p.hl + head * D;

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = qvalid ? load_frag(qb + static_cast<int64_t>(qi) * p.ld + (2 * s + g) * 8) : zero_frag();

  f32x16 o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[mb][e] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // K blocks are 0..D-1, V blocks D..2D-1 (one per thread for D = 128).
  constexpr int kBlocks = 2 * D;
  uint4 r[8];
  auto load_tile = [&](int j0) {
    if (tid < kBlocks) {
      if (tid < D) load_block<D>(kb, p.ld, j0, T, tid, r);
      else load_block<D>(vb, p.ld, j0, T, tid - D, r);
    }
  };
  auto store_tile = [&](int buf) {
    if (tid < kBlocks) {
      if (tid < D) store_natural<D>(k_lds[buf], tid, r);
      else store_transposed<D>(vt_lds[buf], tid - D, r);
    }
  };
  load_tile(kv_lo);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int j0 = kv_lo + t * kBKV;
    if (t + 1 < ntiles) load_tile(j0 + kBKV);
    if (wave_active && j0 <= wlast && j0 + kBKV > w_lo) {
      f32x16 sacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[b][e] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_natural<D>(k_lds[cur], b * 32 + lq, 2 * s + g), qf[s], sacc[b], 0, 0, 0);
      }
      const bool full = (j0 + kBKV - 1 <= q0w) && (j0 >= w_smax) && (q0w + 31 < T);
      float mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = sacc[b][e] * p.scale_log2;
          if (!full) {
            const int j = j0 + b * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            if (!(qvalid && j <= qi && j >= qstart)) v = -INFINITY;
          }
          sacc[b][e] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
      const float m_new = fmaxf(m, mt);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m - m_use);
      l *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mb][e] *= alpha;
      float ls = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = fast_exp2(sacc[b][e] - m_use);
          sacc[b][e] = pe;
          ls += pe;
        }
      l += ls;
      m = m_new;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const bf16x8 pb = pack_bf16x8(sacc[t4 >> 1], 8 * (t4 & 1));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_transposed(vt_lds[cur], mb * 32 + lq, 2 * t4 + g), pb, o[mb], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32, kWave);
  if (qvalid) {
    const float inv = 1.0f / lt;
    bf16_t* out = static_cast<bf16_t*>(p.ctx) + static_cast<int64_t>(qi) * p.hl + head * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = o[mb][4 * a + c] * inv;
        store4(out + mb * 32 + 8 * a + 4 * g, v);
      }
    if (g == 0) p.lse[static_cast<int64_t>(head) * T + qi] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

// -------------------------------------------------- backward preprocess
// delta[n][i] = sum_d dctx[i, n*D + d] * ctx[i, n*D + d]  (= rowsum(P * dP)).
template <typename T>
__global__ void __launch_bounds__(256) attn_delta_kernel(AttnParams p, int D) {
  const int per_row = D / 8;                 // threads per (token, head)
  const int pairs_per_block = 256 / per_row;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * pairs_per_block + threadIdx.x / per_row;
  const int c = threadIdx.x % per_row;
  float acc = 0.0f;
  int64_t i = 0;
  int n = 0;
  if (pair < static_cast<int64_t>(p.T) * p.heads) {
    i = pair / p.heads;
    n = static_cast<int>(pair % p.heads);
    float a[8], b[8];
    load8(static_cast<const T*>(p.dctx) + i * p.hl + n * D + c * 8, a);
    load8(static_cast<const T*>(p.ctx) + i * p.hl + n * D + c * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += a[e] * b[e];
  }
  for (int o = per_row / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (c == 0 && pair < static_cast<int64_t>(p.T) * p.heads) p.delta[static_cast<int64_t>(n) * p.T + i] = acc;
}

// ------------------------------------------------------------------ dQ
template <int D>
__global__ void __launch_bounds__(256) attn_dq_bf16(AttnParams p) {
  constexpr int DC = D / 8, KS = D / 16, MB = D / 32;
  __shared__ uint4 k_lds[2][kBKV * DC];
  __shared__ uint4 v_lds[2][kBKV * DC];
  __shared__ uint4 kt_lds[2][D * 8];
  const int T = p.T;
  const int nqb = (T + kBQ - 1) / kBQ;
  const int head = blockIdx.x % p.heads;
  const int q0 = (nqb - 1 - static_cast<int>(blockIdx.x) / p.heads) * kBQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;
  const int q0w = q0 + wave * 32;
  const int qi = q0w + lq;
  const bool qvalid = qi < T;
  const bool wave_active = q0w < T;
  const int qstart = seq_start(p, min(qi, T - 1));
  const int wlast = min(q0w + 31, T - 1);
  const int w_lo = seq_start(p, min(q0w, T - 1));
  const int w_smax = seq_start(p, wlast);
  const int kv_lo = seq_start(p, q0);
  const int kv_hi = min(T, q0 + kBQ);
  const int ntiles = (kv_hi - kv_lo + kBKV - 1) / kBKV;

  const bf16_t* qkv = static_cast<const bf16_t*>(p.qkv);
  const bf16_t* qb = qkv + head * D;
  const bf16_t* kb = qkv + p.hl + head * D;
  const bf16_t* vb = qkv + 2 * p.hl + head * D;
  const bf16_t* dob = static_cast<const bf16_t*>(p.dctx) + head * D;

  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = qvalid ? load_frag(qb + static_cast<int64_t>(qi) * p.ld + (2 * s + g) * 8) : zero_frag();
    df[s] = qvalid ? load_frag(dob + static_cast<int64_t>(qi) * p.hl + (2 * s + g) * 8) : zero_frag();
  }
  const float lse2 = qvalid ? p.lse[static_cast<int64_t>(head) * T + qi] * kLog2e : 0.0f;
  const float dlt = qvalid ? p.delta[static_cast<int64_t>(head) * T + qi] : 0.0f;

  f32x16 dq[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[mb][e] = 0.0f;

  uint4 r[8];
  auto load_tile = [&](int j0) {
    if (tid < D) load_block<D>(kb, p.ld, j0, T, tid, r);
    else if (tid < 2 * D) load_block<D>(vb, p.ld, j0, T, tid - D, r);
  };
  auto store_tile = [&](int buf) {
    if (tid < D) {
      store_natural<D>(k_lds[buf], tid, r);
      store_transposed<D>(kt_lds[buf], tid, r);
    } else if (tid < 2 * D) {
      store_natural<D>(v_lds[buf], tid - D, r);
    }
  };
  load_tile(kv_lo);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int j0 = kv_lo + t * kBKV;
    if (t + 1 < ntiles) load_tile(j0 + kBKV);
    if (wave_active && j0 <= wlast && j0 + kBKV > w_lo) {
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { sacc[b][e] = 0.0f; pacc[b][e] = 0.0f; }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_natural<D>(k_lds[cur], b * 32 + lq, 2 * s + g), qf[s], sacc[b], 0, 0, 0);
          pacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_natural<D>(v_lds[cur], b * 32 + lq, 2 * s + g), df[s], pacc[b], 0, 0, 0);
        }
      }
      const bool full = (j0 + kBKV - 1 <= q0w) && (j0 >= w_smax) && (q0w + 31 < T);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float pe = fast_exp2(sacc[b][e] * p.scale_log2 - lse2);
          if (!full) {
            const int j = j0 + b * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            if (!(qvalid && j <= qi && j >= qstart)) pe = 0.0f;
          }
          sacc[b][e] = pe * (pacc[b][e] - dlt);
        }
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const bf16x8 db = pack_bf16x8(sacc[t4 >> 1], 8 * (t4 & 1));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_transposed(kt_lds[cur], mb * 32 + lq, 2 * t4 + g), db, dq[mb], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  if (qvalid) {
    bf16_t* out = static_cast<bf16_t*>(p.dqkv) + static_cast<int64_t>(qi) * p.ld + head * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = dq[mb][4 * a + c] * p.scale;
        store4(out + mb * 32 + 8 * a + 4 * g, v);
      }
  }
}

// --------------------------------------------------------------- dK / dV
template <int D>
__global__ void __launch_bounds__(256) attn_dkv_bf16(AttnParams p) {
  constexpr int DC = D / 8, KS = D / 16, MB = D / 32;
  __shared__ uint4 q_lds[2][kBQ2 * DC];
  __shared__ uint4 do_lds[2][kBQ2 * DC];
  __shared__ uint4 qt_lds[2][D * 8];
  __shared__ uint4 dot_lds[2][D * 8];
  __shared__ float lse_s[2][kBQ2], dl_s[2][kBQ2];
  __shared__ int st_s[2][kBQ2];
  const int T = p.T;
  const int head = blockIdx.x % p.heads;
  const int k0 = (static_cast<int>(blockIdx.x) / p.heads) * kBK2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lq = lane & 31;
  const int k0w = k0 + wave * 32;
  const int kj = k0w + lq;
  const bool kvalid = kj < T;
  const bool wave_active = k0w < T;
  const int w_qhi = wave_active ? seq_end(p, min(k0w + 31, T - 1)) : 0;
  const int q_lo = k0;
  const int q_hi = seq_end(p, min(k0 + kBK2 - 1, T - 1));
  const int ntiles = (q_hi - q_lo + kBQ2 - 1) / kBQ2;

  const bf16_t* qkv = static_cast<const bf16_t*>(p.qkv);
  const bf16_t* qb = qkv + head * D;
  const bf16_t* kb = qkv + p.hl + head * D;
  const bf16_t* vb = qkv + 2 * p.hl + head * D;
  const bf16_t* dob = static_cast<const bf16_t*>(p.dctx) + head * D;

  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = kvalid ? load_frag(kb + static_cast<int64_t>(kj) * p.ld + (2 * s + g) * 8) : zero_frag();
    vf[s] = kvalid ? load_frag(vb + static_cast<int64_t>(kj) * p.ld + (2 * s + g) * 8) : zero_frag();
  }
  f32x16 dk[MB], dv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dk[mb][e] = 0.0f; dv[mb][e] = 0.0f; }

  uint4 r[8];
  float st_lse = 0.0f, st_dl = 0.0f;
  int st_start = 0;
  auto load_tile = [&](int i0) {
    if (tid < D) load_block<D>(qb, p.ld, i0, T, tid, r);
    else if (tid < 2 * D) load_block<D>(dob, p.hl, i0, T, tid - D, r);
    if (tid < kBQ2) {
      const int i = i0 + tid;
      if (i < T) {
        st_lse = p.lse[static_cast<int64_t>(head) * T + i] * kLog2e;
        st_dl = p.delta[static_cast<int64_t>(head) * T + i];
        st_start = seq_start(p, i);
      } else {
        st_lse = 0.0f; st_dl = 0.0f; st_start = T;
      }
    }
  };
  auto store_tile = [&](int buf) {
    if (tid < D) {
      store_natural<D>(q_lds[buf], tid, r);
      store_transposed<D>(qt_lds[buf], tid, r);
    } else if (tid < 2 * D) {
      store_natural<D>(do_lds[buf], tid - D, r);
      store_transposed<D>(dot_lds[buf], tid - D, r);
    }
    if (tid < kBQ2) { lse_s[buf][tid] = st_lse; dl_s[buf][tid] = st_dl; st_s[buf][tid] = st_start; }
  };
  load_tile(q_lo);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int i0 = q_lo + t * kBQ2;
    if (t + 1 < ntiles) load_tile(i0 + kBQ2);
    // queries [i0, i0+64) against this wave's keys [k0w, k0w+32)
    if (wave_active && i0 + kBQ2 > k0w && i0 < w_qhi) {
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { sacc[b][e] = 0.0f; pacc[b][e] = 0.0f; }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_natural<D>(q_lds[cur], b * 32 + lq, 2 * s + g), kf[s], sacc[b], 0, 0, 0);
          pacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_natural<D>(do_lds[cur], b * 32 + lq, 2 * s + g), vf[s], pacc[b], 0, 0, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int qo = b * 32 + 8 * a + 4 * g;  // query offset of elements 4a..4a+3
          const float4 l4 = *reinterpret_cast<const float4*>(&lse_s[cur][qo]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dl_s[cur][qo]);
          const int4 s4 = *reinterpret_cast<const int4*>(&st_s[cur][qo]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
          const int sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * a + c;
            const int i = i0 + qo + c;
            float pe = fast_exp2(sacc[b][e] * p.scale_log2 - lv[c]);
            if (!(kvalid && i < T && kj <= i && kj >= sv[c])) pe = 0.0f;
            sacc[b][e] = pe;
            pacc[b][e] = pe * (pacc[b][e] - dv4[c]);
          }
        }
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const bf16x8 pb = pack_bf16x8(sacc[t4 >> 1], 8 * (t4 & 1));
        const bf16x8 db = pack_bf16x8(pacc[t4 >> 1], 8 * (t4 & 1));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          dv[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_transposed(dot_lds[cur], mb * 32 + lq, 2 * t4 + g), pb, dv[mb], 0, 0, 0);
          dk[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_transposed(qt_lds[cur], mb * 32 + lq, 2 * t4 + g), db, dk[mb], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  if (kvalid) {
    bf16_t* base = static_cast<bf16_t*>(p.dqkv) + static_cast<int64_t>(kj) * p.ld + head * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float vk[4], vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vk[c] = dk[mb][4 * a + c] * p.scale;
          vv[c] = dv[mb][4 * a + c];
        }
        store4(base + p.hl + mb * 32 + 8 * a + 4 * g, vk);
        store4(base + 2 * p.hl + mb * 32 + 8 * a + 4 * g, vv);
      }
  }
}

// ------------------------------------------------------------ fp32 path
// Forward: one workgroup (one wave) per (query, head).  Pass 1 finds the
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

AttnParams make_params(const AttnDesc& a) {
  AttnParams p{};
  p.qkv = a.qkv; p.ld = 3LL * a.heads * a.head_dim;
  p.ctx = a.ctx; p.lse = a.lse; p.dctx = a.dctx; p.dqkv = a.dqkv; p.delta = a.delta;
  p.cu = a.cu_seqlens; p.n_seqs = a.n_seqs;
  p.T = static_cast<int>(a.T); p.seq_len = a.seq_len; p.heads = a.heads;
  p.hl = a.heads * a.head_dim;
  p.scale = 1.0f / sqrtf(static_cast<float>(a.head_dim));
  p.scale_log2 = p.scale * kLog2e;
  return p;
}

}  // namespace

hipError_t attn_fwd(bool bf16, const AttnDesc& a, hipStream_t s) {
  if (a.T == 0 || a.heads == 0) return hipSuccess;
  const AttnParams p = make_params(a);
  if (bf16) {
    const int blocks = static_cast<int>((a.T + kBQ - 1) / kBQ) * a.heads;
    if (a.head_dim == 128) hipLaunchKernelGGL(attn_fwd_bf16<128>, dim3(blocks), dim3(256), 0, s, p);
    else if (a.head_dim == 64) hipLaunchKernelGGL(attn_fwd_bf16<64>, dim3(blocks), dim3(256), 0, s, p);
    else return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL(attn_fwd_f32, dim3(static_cast<unsigned>(a.T * a.heads)), dim3(64), 0, s,
                       p, a.head_dim);
  }
  return hipGetLastError();
}

hipError_t attn_bwd(bool bf16, const AttnDesc& a, hipStream_t s) {
  if (a.T == 0 || a.heads == 0) return hipSuccess;
  const AttnParams p = make_params(a);
  const int per_row = a.head_dim / 8;
  const int64_t pairs = a.T * a.heads;
  const int pairs_per_block = 256 / per_row;
  const dim3 dgrid(static_cast<unsigned>((pairs + pairs_per_block - 1) / pairs_per_block));
  if (bf16) hipLaunchKernelGGL(attn_delta_kernel<bf16_t>, dgrid, dim3(256), 0, s, p, a.head_dim);
  else hipLaunchKernelGGL(attn_delta_kernel<float>, dgrid, dim3(256), 0, s, p, a.head_dim);
  if (bf16) {
    const int qblocks = static_cast<int>((a.T + kBQ - 1) / kBQ) * a.heads;
    const int kblocks = static_cast<int>((a.T + kBK2 - 1) / kBK2) * a.heads;
    if (a.head_dim == 128) {
      hipLaunchKernelGGL(attn_dkv_bf16<128>, dim3(kblocks), dim3(256), 0, s, p);
      hipLaunchKernelGGL(attn_dq_bf16<128>, dim3(qblocks), dim3(256), 0, s, p);
    } else if (a.head_dim == 64) {
      hipLaunchKernelGGL(attn_dkv_bf16<64>, dim3(kblocks), dim3(256), 0, s, p);
      hipLaunchKernelGGL(attn_dq_bf16<64>, dim3(qblocks), dim3(256), 0, s, p);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    const dim3 grid(static_cast<unsigned>(a.T * a.heads));
    hipLaunchKernelGGL(attn_dkv_f32, grid, dim3(64), 0, s, p, a.head_dim);
    hipLaunchKernelGGL(attn_dq_f32, grid, dim3(64), 0, s, p, a.head_dim);
  }
  return hipGetLastError();
}

}  // namespace mtp
