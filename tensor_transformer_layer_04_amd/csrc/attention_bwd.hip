// Attention backward for bf16 shards on CDNA4 MFMA.
//
// Given q, k, v (the qkv shard), ctx = O, lse and dO = dctx:
//   D_i = rowsum(dO_i * O_i);  P = exp(S - lse) recomputed from q, k;
//   dV = P^T dO;  dP = dO V^T;  dS = P * (dP - D);  dQ = dS K / sqrt(d);
//   dK = dS^T Q / sqrt(d)
// (the chain rule through the softmax of the attention the pages describe:
// page "Megatron-LM 3D parallelism guide", §2.1 per-head attention, §3.3
// FlashAttention-2 recomputing P from the saved log-sum-exp).
//
// Two block kinds in one launch, no atomics (deterministic):
//  * dK/dV: a workgroup owns 64 keys of one head (2 key groups of 32, one key
//    per lane) and walks the query tiles that can see them; the query rows of
//    every 64-query tile are split between two waves per key group, whose
//    partial dK/dV are summed at the end.  S = Q K^T and dP = dO V^T come out
//    with one key per lane; P and dS then feed dV^T += dO^T P and
//    dK^T += Q^T dS from registers, with dO^T and Q^T gathered from the
//    natural [query][d] tiles by ds_read_b64_tr_b16 in the query order the
//    lane holds.
//  * dQ: a workgroup owns 64 queries (2 groups of 32, one query per lane) and
//    splits every 64-key tile between two waves, like the forward:
//    S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T.
// Tiles go HBM -> LDS with buffer_load ... lds, double-buffered.  The chunk
// swizzle of the [row][d] tiles, ((r & 3) << 2 | (r >> 2) & 3) for 16-chunk
// rows, keeps both access patterns conflict-free: 16 consecutive rows read
// at one chunk (ds_read_b128) and 4 rows read across one 64-byte segment
// (the transpose read).
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace mtp {
namespace {

constexpr int kBT = 64;  // rows (queries or keys) per tile and per workgroup
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const bf16_t* qkv;
  int ld;  // 3 * hl
  const bf16_t* dctx;
  int hl;
  const float* lse;    // [heads, T] log-sum-exp times log2(e)
  const float* delta;  // [heads, T]
  bf16_t* dqkv;
  const int32_t* cu;
  int n_seqs;
  int T, seq_len, heads, nblk;
  int q_lo, q_hi, k_lo, k_hi;  // query and key row ranges (absolute)
  int accumulate;              // add into dqkv instead of storing
  float scale, scale_log2;
  uint32_t qkv_bytes, dctx_bytes, stat_bytes;
  float* amax;  // partial maxima of |dqkv|, zeroed by the preprocess (nullable)
};

__device__ __forceinline__ int seq_index(const BwdParams& p, int i) {
  int lo = 0, hi = p.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}
__device__ __forceinline__ int seq_start(const BwdParams& p, int i) {
  if (!p.cu) return (i / p.seq_len) * p.seq_len;
  return p.cu[seq_index(p, i)];
}
__device__ __forceinline__ int seq_end(const BwdParams& p, int i) {
  if (!p.cu) return min(p.T, (i / p.seq_len + 1) * p.seq_len);
  return p.cu[seq_index(p, i) + 1];
}

// Chunk swizzle of a [row][d] tile with D/8 16-byte chunks per row.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Copy rows [r0, r0+64) of a token-major bf16 matrix (columns col0..col0+D-1)
// into a swizzled LDS tile; rows outside [0, T) read as zeros.
template <int D>
__device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int lane,
                                           int r0, int T, int col0, uint32_t ld_bytes) {
  constexpr int kCpr = D / 8;
  constexpr int kPer = kBT * kCpr / 64 / 4;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = wave * kPer + i;
    const int q = j * 64 + lane;
    const int row = q / kCpr, pc = q % kCpr;
    const int lc = pc ^ swz<D>(row);
    const int r = r0 + row;
    const uint32_t off =
        (r >= 0 && r < T) ? static_cast<uint32_t>(r) * ld_bytes + (col0 + lc * 8) * 2 : kOOB;
    copy16_to_lds(rs, tile + j * 1024, off);
  }
}

// Copy stat[head][r0..r0+63] (lse or delta, fp32) into the first 256 bytes
// of a 1 KB LDS block (one copy; lanes 16..63 fetch zeros).
__device__ __forceinline__ void issue_stat(__amdgpu_buffer_rsrc_t rs, char* dst, int lane, int head,
                                           int r0, int T, int rmax) {
  const int r = r0 + 4 * lane;
  const uint32_t off =
      (lane < 16 && r >= 0 && r < rmax) ? (static_cast<uint32_t>(head) * T + r) * 4u : kOOB;
  copy16_to_lds(rs, dst, off);
}

// Row operand (8 consecutive d of row `row`, chunk c = 2 s + g) of a tile.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* t, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(t + row * (D * 2) + ((c ^ swz<D>(row)) << 4));
}

// Transposed operand: lane l gets column dbase + l%32 of rows
// rb + 16 t + {4g..4g+3, 8+4g..8+4g+3} (g = l/32), the row order in which a
// 32x32 MFMA accumulator holds its rows.
template <int D>
__device__ __forceinline__ bf16x8 col_frag(const char* t, int rb, int tstep, int dbase, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int r1 = rb + 16 * tstep + 4 * (G >> 1) + (s >> 2), r2 = r1 + 8;
  const int col = dbase + 16 * (G & 1) + 4 * (s & 3);
  const int c = col >> 3, w = (col & 7) * 2;
  const v4i16 lo = tr_read(t + r1 * (D * 2) + ((c ^ swz<D>(r1)) << 4) + w);
  const v4i16 hi = tr_read(t + r2 * (D * 2) + ((c ^ swz<D>(r2)) << 4) + w);
  return cat_bf16x8(lo, hi);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int off) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf2(a[off], a[off + 1]),
                                               pack_bf2(a[off + 2], a[off + 3]),
                                               pack_bf2(a[off + 4], a[off + 5]),
                                               pack_bf2(a[off + 6], a[off + 7])));
}

// Schedule N LDS reads and the N MFMAs that consume them in order with a
// window of kWin reads in flight: kWin reads, then (MFMA, read) pairs, then
// the last kWin MFMAs.
constexpr int kWin = 4;
template <int N>
__device__ __forceinline__ void window_schedule() {
  constexpr int W = N > kWin ? kWin : N;
  __builtin_amdgcn_sched_group_barrier(0x100, W, 0);
#pragma unroll
  for (int t = 0; t < N - W; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, W, 0);
}

// Rank r of the causal block lengths -> the key block and the query block of
// that rank, longest first.  A key block's queries run to the end of its
// sequence and a query block's keys start at the start of its sequence, so
// for sequences of one length (a multiple of 64) rank r is local position r /
// n_seq from the start (keys) or from the end (queries) of sequence r % n_seq.
// Otherwise (packed documents, ragged lengths) the ranks follow the block
// index, which only approximates longest-first.
__device__ __forceinline__ void ranked_blocks(const BwdParams& p, int r, int& kblk, int& qblk) {
  const int nbs = p.seq_len / kBT;
  if (!p.cu && p.seq_len % kBT == 0 && nbs > 0 && p.nblk % nbs == 0) {
    const int n_seq = p.nblk / nbs;
    const int li = r / n_seq, sq = r % n_seq;
    kblk = sq * nbs + li;
    qblk = sq * nbs + nbs - 1 - li;
  } else {
    kblk = r;
    qblk = p.nblk - 1 - r;
  }
}

// ----------------------------------------------------------------- dK / dV
// Key-major pass.  Every key block is handled by two workgroups: one
// accumulates dV^T += dO^T P (needs S only), the other dK^T += Q^T dS (needs
// S and dP).  Each then holds one 32 x D accumulator per wave instead of
// two, which leaves room for two waves per SIMD; the two roles run side by
// side on the chip.  Per 64-query tile and wave (32 keys, 32 query rows of
// the tile): S = Q K^T [, dP = dO V^T] with one key per lane, P / dS on the
// vector units, then the transposed-operand MFMAs.
template <int D, bool want_dk>
__device__ __forceinline__ void dkv_block(const BwdParams& p, int kblk, int head,
                                          char* sq0, char* sq1, char* so0, char* so1, char* st0,
                                          char* st1, float& mx) {
  constexpr int KS = D / 16, DB = D / 32;
  const int T = p.T;
  const int k0 = p.k_lo + kblk * kBT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave & 1, qh = wave >> 1;
  const int lk = lane & 31, g = lane >> 5;
  const int ka = k0 + kg * 32;  // first key of this wave
  const int kj = ka + lk;       // this lane's key
  const bool kvalid = kj < p.k_hi;
  const int ka_last = min(ka + 31, p.k_hi - 1);
  // queries that see this lane's key: [kj, kend) within the query range;
  // wend <= every lane's kend
  const int kend = kvalid ? min(seq_end(p, kj), p.q_hi) : kj;
  const int wend = (ka + 31 < p.k_hi) ? min(seq_end(p, ka), p.q_hi) : 0;
  const int q_lo = max(k0, p.q_lo);
  const int q_hi = min(seq_end(p, min(k0 + kBT - 1, T - 1)), p.q_hi);
  const int nt = (((q_hi - q_lo + kBT - 1) / kBT) + 1) & ~1;
  const int rb = qh * 32;

  const uint32_t ld_bytes = static_cast<uint32_t>(p.ld) * 2;
  const uint32_t ldo_bytes = static_cast<uint32_t>(p.hl) * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qkv, p.qkv_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.dctx, p.dctx_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse, p.stat_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.delta, p.stat_bytes);

  // K^T (and for dK, V^T) fragments, B operands of S = Q K^T / dP = dO V^T:
  // lane holds d = 16 s + 8 g .. +7 of key kj.
  bf16x8 kf[KS], vf[KS];
  {
    const bf16_t* kr = p.qkv + static_cast<int64_t>(kvalid ? kj : 0) * p.ld + p.hl + head * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 a = kvalid ? *reinterpret_cast<const uint4*>(kr + 16 * s + 8 * g)
                             : make_uint4(0, 0, 0, 0);
      const uint4 b = (kvalid && want_dk)
                          ? *reinterpret_cast<const uint4*>(kr + p.hl + 16 * s + 8 * g)
                          : make_uint4(0, 0, 0, 0);
      kf[s] = __builtin_bit_cast(bf16x8, a);
      vf[s] = __builtin_bit_cast(bf16x8, b);
    }
  }
  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[d][e] = 0.0f;

  auto issue = [&](char* tq, char* to, char* ts, int r0) {
    issue_rows<D>(rq, tq, wave, lane, r0, p.q_hi, head * D, ld_bytes);
    issue_rows<D>(ro, to, wave, lane, r0, p.q_hi, head * D, ldo_bytes);
    // waves 0/2 copy lse, 1/3 copy D (the pairs write identical bytes)
    issue_stat((wave & 1) ? rd : rl, ts + (wave & 1) * 1024, lane, head, r0, T, p.q_hi);
  };

  auto compute = [&](const char* tq, const char* to, const char* ts, int r0) {
    const int qa = r0 + rb;  // first query row of this wave's half
    // wave-uniform skip: no query of the half sees a key of this wave
    if (qa >= p.q_hi || ka >= p.k_hi || min(qa + 31, p.q_hi - 1) < ka ||
        ka_last < seq_start(p, min(qa, T - 1)))
      return;
    f32x16 s_acc, p_acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s_acc[e] = 0.0f; p_acc[e] = 0.0f; }
    // The Q (and dO) row fragments are read a window of kWin reads ahead of
    // the MFMAs that use them, so LDS latency overlaps the matrix pipe.
    if (want_dk) {
      bf16x8 fr[2 * KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        fr[2 * s] = row_frag<D>(tq, rb + lk, 2 * s + g);
        fr[2 * s + 1] = row_frag<D>(to, rb + lk, 2 * s + g);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * s], kf[s], s_acc, 0, 0, 0);
        p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * s + 1], vf[s], p_acc, 0, 0, 0);
      }
      window_schedule<2 * KS>();
    } else {
      bf16x8 fr[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) fr[s] = row_frag<D>(tq, rb + lk, 2 * s + g);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s], kf[s], s_acc, 0, 0, 0);
      window_schedule<KS>();
    }
    // accumulator rows: query qa + 8 (e/4) + 4 g + e%4; column: key kj.
    // Query qi sees key kj iff kj <= qi < end of kj's sequence; a tile whose
    // first query is at or past the wave's last key and whose last query is
    // before the end of the first key's sequence needs no mask.
    const float* lse = reinterpret_cast<const float*>(ts);
    const float* dl = lse + 256;
    const bool full = (qa >= ka + 31) && (qa + 31 < wend);
    float v[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int qr = rb + 8 * a + 4 * g;
      const float4 l4 = *reinterpret_cast<const float4*>(lse + qr);
      const float4 d4 = *reinterpret_cast<const float4*>(dl + qr);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * a + c;
        v[e] = __builtin_amdgcn_exp2f(fmaf(s_acc[e], p.scale_log2, -lv[c]));
        if (want_dk) v[e] *= p_acc[e] - dv4[c];
      }
    }
    if (!full) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qi = qa + 8 * (e >> 2) + 4 * g + (e & 3);
        if (!(qi >= kj && qi < kend)) v[e] = 0.0f;
      }
    }
    const char* tt = want_dk ? tq : to;  // dK^T += Q^T dS, dV^T += dO^T P
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int o = 8 * t2;
      const bf16x8 vb = __builtin_bit_cast(
          bf16x8, make_uint4(pack_bf2(v[o], v[o + 1]), pack_bf2(v[o + 2], v[o + 3]),
                             pack_bf2(v[o + 4], v[o + 5]), pack_bf2(v[o + 6], v[o + 7])));
#pragma unroll
      for (int d = 0; d < DB; ++d)
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_frag<D>(tt, rb, t2, 32 * d, lane), vb,
                                                         acc[d], 0, 0, 0);
    }
  };

  auto stage_ready = [&]() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
  };
  issue(sq0, so0, st0, q_lo);
  issue(sq1, so1, st1, q_lo + kBT);
  {
    constexpr int kTileInstr = 2 * (kBT * (D / 8) / 64 / 4) + 1;
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kTileInstr) : "memory");
    __syncthreads();
  }
  for (int t = 0; t < nt; t += 2) {
    const int r0 = q_lo + t * kBT;
    compute(sq0, so0, st0, r0);
    stage_ready();
    issue(sq0, so0, st0, r0 + 2 * kBT);
    compute(sq1, so1, st1, r0 + kBT);
    stage_ready();
    issue(sq1, so1, st1, r0 + 3 * kBT);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  // Sum the two query halves: the half-1 wave parks its accumulator in LDS.
  float* park = reinterpret_cast<float*>(kg == 0 ? sq0 : sq1);
  if (qh == 1) {
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) park[(d * 16 + e) * 64 + lane] = acc[d][e];
  }
  __syncthreads();
  if (qh == 0 && kvalid) {
    bf16_t* out = p.dqkv + static_cast<int64_t>(kj) * p.ld + (want_dk ? p.hl : 2 * p.hl) + head * D;
    const float sc = want_dk ? p.scale : 1.0f;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float w[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = 4 * a + c;
          w[c] = (acc[d][e] + park[(d * 16 + e) * 64 + lane]) * sc;
        }
        if (p.accumulate) {
          float o[4];
          load4(out + 32 * d + 8 * a + 4 * g, o);
#pragma unroll
          for (int c = 0; c < 4; ++c) w[c] += o[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(w[c]));
        store4(out + 32 * d + 8 * a + 4 * g, w);
      }
  }
}

// ---------------------------------------------------------------------- dQ
template <int D>
__device__ __forceinline__ void dq_block(const BwdParams& p, int qblk, int head, char* sk0,
                                         char* sk1, char* sv0, char* sv1, float& mx) {
  constexpr int KS = D / 16, DB = D / 32;
  const int T = p.T;
  const int q0 = p.q_lo + qblk * kBT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = wave & 1, kh = wave >> 1;
  const int lq = lane & 31, g = lane >> 5;
  const int qa = q0 + qg * 32;
  const int qi = qa + lq;
  const bool qvalid = qi < p.q_hi;
  const int qstart = max(seq_start(p, min(qi, T - 1)), p.k_lo);
  const int wq_last = min(qa + 31, p.q_hi - 1);
  const int w_start_lo = max(seq_start(p, min(qa, T - 1)), p.k_lo);
  const int w_start_hi = max(seq_start(p, wq_last), p.k_lo);
  const int kv_lo = max(seq_start(p, min(q0, T - 1)), p.k_lo);
  const int kv_hi = min(p.k_hi, q0 + kBT);
  const int nt = (((kv_hi - kv_lo + kBT - 1) / kBT) + 1) & ~1;

  const uint32_t ld_bytes = static_cast<uint32_t>(p.ld) * 2;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.qkv, p.qkv_bytes);

  // Q^T and dO^T fragments (B operands): lane holds d = 16 s + 8 g .. +7 of
  // query qi.
  bf16x8 qf[KS], of[KS];
  {
    const bf16_t* qr = p.qkv + static_cast<int64_t>(qvalid ? qi : 0) * p.ld + head * D;
    const bf16_t* orow = p.dctx + static_cast<int64_t>(qvalid ? qi : 0) * p.hl + head * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 a = qvalid ? *reinterpret_cast<const uint4*>(qr + 16 * s + 8 * g) : make_uint4(0, 0, 0, 0);
      const uint4 b = qvalid ? *reinterpret_cast<const uint4*>(orow + 16 * s + 8 * g) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, a);
      of[s] = __builtin_bit_cast(bf16x8, b);
    }
  }
  const float lse2 = qvalid ? p.lse[static_cast<int64_t>(head) * T + qi] : 0.0f;
  const float dlt = qvalid ? p.delta[static_cast<int64_t>(head) * T + qi] : 0.0f;

  f32x16 dq[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[d][e] = 0.0f;

  auto issue = [&](char* tk, char* tv, int k0) {
    issue_rows<D>(rs, tk, wave, lane, k0, p.k_hi, p.hl + head * D, ld_bytes);
    issue_rows<D>(rs, tv, wave, lane, k0, p.k_hi, 2 * p.hl + head * D, ld_bytes);
  };

  auto compute = [&](const char* tk, const char* tv, int j0) {
    const int ja = j0 + kh * 32;
    if (qa >= p.q_hi || ja > wq_last || ja + 31 < w_start_lo) return;
    const int rb = kh * 32;
    f32x16 s_acc, p_acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s_acc[e] = 0.0f; p_acc[e] = 0.0f; }
    {
      bf16x8 fr[2 * KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        fr[2 * s] = row_frag<D>(tk, rb + lq, 2 * s + g);
        fr[2 * s + 1] = row_frag<D>(tv, rb + lq, 2 * s + g);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * s], qf[s], s_acc, 0, 0, 0);
        p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[2 * s + 1], of[s], p_acc, 0, 0, 0);
      }
      window_schedule<2 * KS>();
    }
    // Rows: key ja + 8 (e/4) + 4 g + e%4; column: query qi.
    // keys past the key range (the next chunk's, or past T) are masked too
    const bool full = (ja + 31 <= qa) && (ja >= w_start_hi) && (qa + 31 < p.q_hi) &&
                      (ja + 31 < p.k_hi);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float pe = __builtin_amdgcn_exp2f(fmaf(s_acc[e], p.scale_log2, -lse2));
      if (!full) {
        const int j = ja + 8 * (e >> 2) + 4 * g + (e & 3);
        if (!(qvalid && j <= qi && j >= qstart && j < p.k_hi)) pe = 0.0f;
      }
      p_acc[e] = pe * (p_acc[e] - dlt);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 sb = pack8(p_acc, 8 * t);
#pragma unroll
      for (int d = 0; d < DB; ++d)
        dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_frag<D>(tk, rb, t, 32 * d, lane), sb,
                                                        dq[d], 0, 0, 0);
    }
  };

  auto stage_ready = [&]() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
  };
  issue(sk0, sv0, kv_lo);
  issue(sk1, sv1, kv_lo + kBT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int t = 0; t < nt; t += 2) {
    const int j0 = kv_lo + t * kBT;
    compute(sk0, sv0, j0);
    stage_ready();
    issue(sk0, sv0, j0 + 2 * kBT);
    compute(sk1, sv1, j0 + kBT);
    stage_ready();
    issue(sk1, sv1, j0 + 3 * kBT);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  float* park = reinterpret_cast<float*>(qg == 0 ? sk0 : sk1);
  if (kh == 1) {
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) park[(d * 16 + e) * 64 + lane] = dq[d][e];
  }
  __syncthreads();
  if (kh == 0 && qvalid) {
    bf16_t* out = p.dqkv + static_cast<int64_t>(qi) * p.ld + head * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = 4 * a + c;
          v[c] = (dq[d][e] + park[(d * 16 + e) * 64 + lane]) * p.scale;
        }
        if (p.accumulate) {
          float o[4];
          load4(out + 32 * d + 8 * a + 4 * g, o);
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] += o[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(v[c]));
        store4(out + 32 * d + 8 * a + 4 * g, v);
      }
  }
}

// ------------------------------------------------------------- one launch
// Every (rank, head) has three workgroups: dK and dV of the key block of that
// rank and dQ of the query block of that rank.  The dQ pass alone cannot
// fill the chip once its short blocks are done; in one launch its blocks fill
// the slots the key-major blocks leave.  Blocks are issued rank-major
// (longest first), and the three roles of one head are 'heads' blocks apart,
// so with a head count that is a multiple of 8 they land on one XCD and share
// its L2 for the Q, dO, K and V tiles they all read.
template <int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_mfma(BwdParams p) {
  constexpr int kTile = kBT * D * 2;
  __shared__ __attribute__((aligned(1024))) char t0[kTile];
  __shared__ __attribute__((aligned(1024))) char t1[kTile];
  __shared__ __attribute__((aligned(1024))) char t2[kTile];
  __shared__ __attribute__((aligned(1024))) char t3[kTile];
  __shared__ __attribute__((aligned(1024))) char st0[2048];  // lse | delta
  __shared__ __attribute__((aligned(1024))) char st1[2048];
  const int per_rank = 3 * p.heads;
  const int r = blockIdx.x / per_rank, j = blockIdx.x % per_rank;
  const int role = j / p.heads, head = j % p.heads;
  int kblk, qblk;
  ranked_blocks(p, r, kblk, qblk);
  float mx = 0.0f;  // largest |dqkv| this lane stores
  if (role == 1)
    dq_block<D>(p, qblk, head, t0, t1, t2, t3, mx);
  else if (role == 0)
    dkv_block<D, true>(p, kblk, head, t0, t1, t2, t3, st0, st1, mx);
  else
    dkv_block<D, false>(p, kblk, head, t0, t1, t2, t3, st0, st1, mx);
  // The partial maximum of what this workgroup stored (rounded to bf16 like
  // the values) raises slot blockIdx.x mod kAmaxParts, which the preprocess
  // zeroed: the grid has more workgroups than slots, and the maximum does
  // not depend on the order of the atomic updates.
  if (p.amax) {
    mx = warp_max(mx);
    __syncthreads();
    float* wm = reinterpret_cast<float*>(st0);
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float m = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
      atomicMax(reinterpret_cast<unsigned int*>(p.amax + blockIdx.x % kAmaxParts),
                __float_as_uint(lo_bf(pack_bf2(m, 0.0f))));
    }
  }
}

}  // namespace

hipError_t attn_bwd_bf16_mfma(const AttnDesc& a, hipStream_t s) {
  BwdParams p{};
  p.qkv = static_cast<const bf16_t*>(a.qkv);
  p.ld = 3 * a.heads * a.head_dim;
  p.dctx = static_cast<const bf16_t*>(a.dctx);
  p.hl = a.heads * a.head_dim;
  p.lse = a.delta + a.heads * a.T;  // lse * log2(e), written by the preprocess
  p.delta = a.delta;
  p.dqkv = static_cast<bf16_t*>(a.dqkv);
  p.cu = a.cu_seqlens;
  p.n_seqs = a.n_seqs;
  p.T = static_cast<int>(a.T);
  p.seq_len = a.seq_len;
  p.heads = a.heads;
  p.q_lo = static_cast<int>(a.q_lo);
  p.q_hi = static_cast<int>(a.q_hi < 0 ? a.T : a.q_hi);
  p.k_lo = static_cast<int>(a.k_lo);
  p.k_hi = static_cast<int>(a.k_hi < 0 ? a.T : a.k_hi);
  p.accumulate = a.accumulate ? 1 : 0;
  p.amax = a.amax;
  // one rank (and so one dK/dV and one dQ block) per 64 rows; the two
  // ranges have equal lengths (whole sequence, or equal chunks)
  p.nblk = (p.q_hi - p.q_lo + kBT - 1) / kBT;
  if (p.nblk <= 0) return hipSuccess;
  p.scale = 1.0f / sqrtf(static_cast<float>(a.head_dim));
  p.scale_log2 = p.scale * kLog2e;
  const int64_t qb = a.T * p.ld * 2, ob = a.T * p.hl * 2, sb = a.T * a.heads * 4;
  if (qb >= static_cast<int64_t>(kOOB) || ob >= static_cast<int64_t>(kOOB) ||
      sb >= static_cast<int64_t>(kOOB))
    return hipErrorInvalidValue;
  p.qkv_bytes = static_cast<uint32_t>(qb);
  p.dctx_bytes = static_cast<uint32_t>(ob);
  p.stat_bytes = static_cast<uint32_t>(sb);
  const dim3 grid(static_cast<unsigned>(3 * p.nblk * a.heads));  // dK, dQ and dV roles
  if (a.head_dim == 128) {
    hipLaunchKernelGGL(attn_bwd_mfma<128>, grid, dim3(256), 0, s, p);
  } else if (a.head_dim == 64) {
    hipLaunchKernelGGL(attn_bwd_mfma<64>, grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mtp
