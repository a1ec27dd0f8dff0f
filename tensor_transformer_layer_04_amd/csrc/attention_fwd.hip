// Attention forward for bf16 shards on CDNA4 MFMA.
//
// Per local head n: S = q_n k_n^T / sqrt(d), key j visible to query i iff
// start(i) <= j <= i, P = softmax(S) in fp32 (online, base 2), ctx_n = P v_n,
// lse = natural-log log-sum-exp of each score row.  The head split needs no
// exchange between ranks and the softmax runs in fp32 (page "Megatron-LM 3D
// parallelism guide", §2.1 and the attention_softmax_in_fp32 flag of §3.2).
//
// Work decomposition (one workgroup = QG*KH waves, 32*QG queries of one head):
//  * waves (g, h) for query group g in [0, QG) (32 queries) and key part h
//    in [0, KH): every tile of 32*KH keys is split into KH parts of 32 keys,
//    so KH waves share each query group and keep separate online-softmax
//    states, merged exactly at the end.  QG = KH = 2 (four waves, two
//    workgroups per CU) measured best at the 7B shard shape: four query
//    groups halve the K/V copies per (query, key) pair but leave one
//    workgroup per CU with nothing to balance the long causal row blocks.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 puts one query per lane (16
//    keys each, the other 16 in lane ^ 32), so row max and row sum are
//    in-lane plus one exchange.  P^T then feeds O^T += V^T P^T straight from
//    registers; its contraction order is the key order the lane holds
//    ({4g..4g+3, 8+4g..8+4g+3} per 16 keys), and V^T is gathered from the
//    natural [key][d] tile in that order with ds_read_b64_tr_b16.
//  * K and V tiles go HBM -> LDS with buffer_load ... lds; keys outside
//    [0, T) read as zeros (buffer offset past num_records).  The loop is
//    software-pipelined: K runs two tiles ahead and V one, and the S MFMAs
//    of the next tile are issued before the softmax of the current one.
//  * Scores stay in log2 units: p = exp2(s * scale * log2(e) - m) is one FMA
//    and one v_exp_f32.  The reference max m of a row moves (and O is
//    rescaled) only when a tile's max exceeds it by more than 8, so p < 2^8;
//    the result is exact for any reference at or below the running max.
//  * Blocks are dispatched longest causal row block first, so the shorter
//    ones fill the CUs that finish early.
#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace mtp {
namespace {

constexpr int kQG = 2;  // query groups of 32 per workgroup
constexpr int kKH = 2;  // key parts of 32 per tile (waves per query group)
constexpr int kFQ = 32 * kQG;    // queries per workgroup
constexpr int kFK = 32 * kKH;    // keys per tile
constexpr int kFW = kQG * kKH;   // waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct FwdParams {
  const bf16_t* qkv;
  int ld;  // elements per token row of qkv (3 * hl)
  bf16_t* ctx;
  int hl;
  float* lse;
  const int32_t* cu;
  int n_seqs;
  int T, seq_len, heads, nqb;
  int q_lo, q_hi, k_lo, k_hi;  // query and key row ranges (absolute)
  float scale_log2;
  uint32_t qkv_bytes;
  float* amax;  // partial maxima of |ctx|, one per workgroup (nullable)
};

__device__ __forceinline__ int seq_start(const FwdParams& p, int i) {
  if (!p.cu) return (i / p.seq_len) * p.seq_len;
  int lo = 0, hi = p.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return p.cu[lo];
}

// K tile: row = key, D*2 bytes; 16-byte chunk c of row r at c ^ swz_key(r).
template <int D>
__device__ __forceinline__ int swz_key(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// V tile: row = key, D*2 bytes; 64-byte segment s of row r at s ^ swz_val(r).
template <int D>
__device__ __forceinline__ int swz_val(int r) {
  return r & (D / 32 - 1);
}

// Copy keys [k0, k0+kFK) of one head's K (V) columns into an LDS tile.
template <int D, bool VAL>
__device__ __forceinline__ void issue_kv(__amdgpu_buffer_rsrc_t rs, char* tile, int wave, int lane,
                                         int k0, int T, int col0, uint32_t ld_bytes) {
  constexpr int kCpr = D / 8;                 // chunks per key row
  constexpr int kInstr = kFK * kCpr / 64;     // 1 KB copies per tile
  constexpr int kPer = kInstr / kFW;
  static_assert(kInstr % kFW == 0, "copies split evenly over the waves");
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = wave * kPer + i;
    const int q = j * 64 + lane;
    const int row = q / kCpr, pc = q % kCpr;
    const int lc = VAL ? (((pc >> 2) ^ swz_val<D>(row)) << 2) | (pc & 3) : pc ^ swz_key<D>(row);
    const int key = k0 + row;
    const uint32_t off = (key >= 0 && key < T)
                             ? static_cast<uint32_t>(key) * ld_bytes + (col0 + lc * 8) * 2
                             : kOOB;
    copy16_to_lds(rs, tile + j * 1024, off);
  }
}

template <int D>
__global__ void __launch_bounds__(64 * kFW, (8 + kFW - 1) / kFW) attn_fwd_mfma(FwdParams p) {
  constexpr int KS = D / 16;  // k-steps of S over d
  constexpr int DB = D / 32;  // 32-wide d blocks of O
  constexpr int kTileBytes = kFK * D * 2;
  __shared__ __attribute__((aligned(1024))) char sk0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sk1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sv0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sv1[kTileBytes];

  const int T = p.T;
  const int item = blockIdx.x;
  const int head = item % p.heads;
  const int qblk = p.nqb - 1 - item / p.heads;
  const int q0 = p.q_lo + qblk * kFQ;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = wave % kQG, kh = wave / kQG;
  const int lq = lane & 31, g = lane >> 5;
  const int qa = q0 + qg * 32;            // first query of this wave
  const int qi = qa + lq;                 // this lane's query
  const bool qvalid = qi < p.q_hi;
  // keys visible to a query: from the start of its sequence (and of the
  // key range) up to itself
  const int qstart = max(seq_start(p, min(qi, T - 1)), p.k_lo);
  const int wq_last = min(qa + 31, p.q_hi - 1);
  const int w_start_lo = max(seq_start(p, min(qa, T - 1)), p.k_lo);
  const int w_start_hi = max(seq_start(p, wq_last), p.k_lo);
  const int kv_lo = max(seq_start(p, min(q0, T - 1)), p.k_lo);
  const int kv_hi = min(p.k_hi, q0 + kFQ);
  const int nt = (((kv_hi - kv_lo + kFK - 1) / kFK) + 1) & ~1;

  const uint32_t ld_bytes = static_cast<uint32_t>(p.ld) * 2;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.qkv, p.qkv_bytes);
  const int kcol = p.hl + head * D, vcol = 2 * p.hl + head * D;

  // Q^T fragments (B operand of S^T): lane holds d = 16 s + 8 g .. +7 of
  // query qi.
  bf16x8 qf[KS];
  {
    const bf16_t* qrow = p.qkv + static_cast<int64_t>(qvalid ? qi : 0) * p.ld + head * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * g)
                             : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  auto issue_k = [&](char* tk, int k0) {
    issue_kv<D, false>(rs, tk, wave, lane, k0, p.k_hi, kcol, ld_bytes);
  };
  auto issue_v = [&](char* tv, int k0) {
    issue_kv<D, true>(rs, tv, wave, lane, k0, p.k_hi, vcol, ld_bytes);
  };
  // Wave-uniform: does any (query, key) pair of this wave's part of the tile
  // at key j0 exist?
  auto visible = [&](int j0) {
    const int ja = j0 + kh * 32;
    return !(qa >= p.q_hi || ja > wq_last || ja + 31 < w_start_lo);
  };

  // S^T of this wave's part of the tile at key j0 (K rows from LDS).
  auto s_tile = [&](const char* tk) {
    const int krow = kh * 32 + lq;
    bf16x8 kfr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = 2 * s + g;
      kfr[s] = *reinterpret_cast<const bf16x8*>(tk + krow * (D * 2) +
                                                ((c ^ swz_key<D>(krow)) << 4));
    }
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[s], qf[s], sacc, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
    return sacc;
  };

  // Online softmax of the scores of the tile at key j0 and O^T += V^T P^T.
  auto softmax_pv = [&](f32x16 sacc, const char* tv, int j0) {
    const int ja = j0 + kh * 32;
    // V^T operands first: their latency hides under the softmax arithmetic.
    const int G = lane >> 4, s16 = lane & 15;
    bf16x8 vfr[2][DB];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r1 = kh * 32 + 16 * t + 4 * (G >> 1) + (s16 >> 2);
      const int r2 = r1 + 8;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const int col = 32 * d + 16 * (G & 1) + 4 * (s16 & 3);
        const int seg = col >> 5, within = (col & 31) * 2;
        const v4i16 lo = tr_read(tv + r1 * (D * 2) + ((seg ^ swz_val<D>(r1)) << 6) + within);
        const v4i16 hi = tr_read(tv + r2 * (D * 2) + ((seg ^ swz_val<D>(r2)) << 6) + within);
        vfr[t][d] = cat_bf16x8(lo, hi);
      }
    }
    // keys past the key range (the next chunk's, or past T) are masked
    // too: they may precede the query
    const bool full = (ja + 31 <= qa) && (ja >= w_start_hi) && (qa + 31 < p.q_hi) &&
                      (ja + 31 < p.k_hi);
    if (!full) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = ja + 8 * (e >> 2) + 4 * g + (e & 3);
        if (!(qvalid && j <= qi && j >= qstart && j < p.k_hi)) sacc[e] = -INFINITY;
      }
    }
    float mt = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, sacc[e]);
    mt = xor32_max(mt) * p.scale_log2;
    // The reference max m only moves when some lane's tile max exceeds it
    // by more than 8 (log2 units): p = exp2(s - m) then stays below 2^8 and
    // the rescale of O and l is skipped for most tiles.
    if (__builtin_amdgcn_ballot_w64(mt > m + 8.0f)) {
      const float m_new = fmaxf(m, mt);
      const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
      m = m_new;
    }
    const float nm = m == -INFINITY ? 0.0f : -m;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[e], p.scale_log2, nm));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[e + 1], p.scale_log2, nm));
      l += p0 + p1;
      pk[e >> 1] = pack_bf2(p0, p1);
    }
    // O^T += V^T P^T over the part's 32 keys, 16 per k-step.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, make_uint4(pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]));
#pragma unroll
      for (int d = 0; d < DB; ++d)
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[t][d], pb, o[d], 0, 0, 0);
    }
  };

  // Software pipeline over key tiles t = 0 .. nt-1 (nt even; tiles past the
  // visible range are skipped, tiles past T load zeros).  K runs two tiles
  // ahead and V one: tile t's K is in kbuf[t % 2], its V in vbuf[t % 2].
  // Iteration t, after its barrier (which both publishes the copies issued
  // one iteration earlier and retires every read of the buffers refilled
  // next): copy K(t+2) into kbuf[t % 2] and V(t+1) into vbuf[(t+1) % 2],
  // issue the S MFMAs of tile t+1, then the softmax and P V of tile t, so the
  // matrix cores work on S(t+1) while the vector units run tile t's softmax.
  issue_k(sk0, kv_lo);
  issue_k(sk1, kv_lo + kFK);
  issue_v(sv0, kv_lo);
  {
    constexpr int kPerTile = (kFK * (D / 8) / 64) / kFW;  // copies per wave per tile
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kPerTile) : "memory");
    __syncthreads();
  }
  f32x16 s_cur = visible(kv_lo) ? s_tile(sk0) : f32x16{};
  auto iteration = [&](char* k_free, const char* k_next, const char* v_cur, char* v_free, int t) {
    const int j0 = kv_lo + t * kFK;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue_k(k_free, j0 + 2 * kFK);
    issue_v(v_free, j0 + kFK);
    const bool vis_next = visible(j0 + kFK);
    f32x16 s_next{};
    if (vis_next) s_next = s_tile(k_next);
    if (visible(j0)) softmax_pv(s_cur, v_cur, j0);
    s_cur = s_next;
  };
  for (int t = 0; t < nt; t += 2) {
    iteration(sk0, sk1, sv0, sv1, t);
    iteration(sk1, sk0, sv1, sv0, t + 1);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  // Merge the KH key parts of each query group.  Waves of parts 1..KH-1
  // park m, l and O in LDS (the tile buffers are free now; O of one wave
  // takes half a tile buffer); the part-0 wave combines them in part order.
  l = xor32_sum(l);
  constexpr int kOBytes = DB * 16 * 64 * 4;
  constexpr int kSlotsPerBuf = kTileBytes / kOBytes;
  static_assert(4 * kSlotsPerBuf >= kQG * (kKH - 1), "merge slots");
  auto slot_o = [&](int part) {
    const int sl = qg * (kKH - 1) + (part - 1);
    const int bi = sl / kSlotsPerBuf;
    char* const buf = bi == 0 ? sk0 : bi == 1 ? sk1 : bi == 2 ? sv0 : sv1;
    return reinterpret_cast<float*>(buf + (sl % kSlotsPerBuf) * kOBytes);
  };
  __shared__ float park_mls[kQG * kKH * 128];
  float* park_ml = park_mls + (qg * kKH) * 128;
  if (kh > 0) {
    float* po = slot_o(kh);
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) po[(d * 16 + e) * 64 + lane] = o[d][e];
    park_ml[kh * 128 + lane] = m;
    park_ml[kh * 128 + 64 + lane] = l;
  }
  __syncthreads();
  float mx = 0.0f;  // largest |ctx| this lane stores
  if (kh == 0) {
    float mk[kKH], lk[kKH];
    mk[0] = m;
    lk[0] = l;
    float mf = m;
#pragma unroll
    for (int k = 1; k < kKH; ++k) {
      mk[k] = park_ml[k * 128 + lane];
      lk[k] = park_ml[k * 128 + 64 + lane];
      mf = fmaxf(mf, mk[k]);
    }
    float ak[kKH], lt = 0.0f;
#pragma unroll
    for (int k = 0; k < kKH; ++k) {
      ak[k] = mk[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mk[k] - mf);
      lt += lk[k] * ak[k];
    }
    if (qvalid) {
      // A query that sees no key of the range (possible in a block of keys
      // that precede the queries when documents are packed) gets ctx 0 and
      // lse -inf: the empty part of a log-sum-exp merge.
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      bf16_t* out = p.ctx + static_cast<int64_t>(qi) * p.hl + head * D;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * a + c;
            const int idx = (d * 16 + e) * 64 + lane;
            float acc = o[d][e] * ak[0];
#pragma unroll
            for (int k = 1; k < kKH; ++k) acc += slot_o(k)[idx] * ak[k];
            v[c] = acc * inv;
            mx = fmaxf(mx, fabsf(v[c]));
          }
          store4(out + 32 * d + 8 * a + 4 * g, v);
        }
      if (g == 0)
        p.lse[static_cast<int64_t>(head) * T + qi] =
            lt > 0.0f ? (mf + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
  }
  // The partial maximum of this workgroup's ctx for an FP8 scale (slot
  // blockIdx.x, rounded to bf16 like the values; workgroup 0 zeroes the
  // slots no workgroup owns).
  if (p.amax) {
    mx = warp_max(mx);
    __syncthreads();
    if (lane == 0) park_mls[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      float mw = park_mls[0];
#pragma unroll
      for (int w = 1; w < kFW; ++w) mw = fmaxf(mw, park_mls[w]);
      p.amax[blockIdx.x] = lo_bf(pack_bf2(mw, 0.0f));
    }
    if (blockIdx.x == 0)
      for (int i = static_cast<int>(gridDim.x) + threadIdx.x; i < kAmaxParts; i += 64 * kFW)
        p.amax[i] = 0.0f;
  }
}

}  // namespace

hipError_t attn_fwd_bf16_mfma(const AttnDesc& a, hipStream_t s) {
  FwdParams p{};
  p.qkv = static_cast<const bf16_t*>(a.qkv);
  p.ld = 3 * a.heads * a.head_dim;
  p.ctx = static_cast<bf16_t*>(a.ctx);
  p.hl = a.heads * a.head_dim;
  p.lse = a.lse;
  p.cu = a.cu_seqlens;
  p.n_seqs = a.n_seqs;
  p.T = static_cast<int>(a.T);
  p.seq_len = a.seq_len;
  p.heads = a.heads;
  p.q_lo = static_cast<int>(a.q_lo);
  p.q_hi = static_cast<int>(a.q_hi < 0 ? a.T : a.q_hi);
  p.k_lo = static_cast<int>(a.k_lo);
  p.k_hi = static_cast<int>(a.k_hi < 0 ? a.T : a.k_hi);
  p.nqb = (p.q_hi - p.q_lo + kFQ - 1) / kFQ;
  if (p.nqb <= 0) return a.amax ? fp8_amax(a.ctx, 0, a.amax, s) : hipSuccess;
  p.scale_log2 = kLog2e / sqrtf(static_cast<float>(a.head_dim));
  const int64_t bytes = a.T * p.ld * 2;
  if (bytes >= static_cast<int64_t>(kOOB)) return hipErrorInvalidValue;
  p.qkv_bytes = static_cast<uint32_t>(bytes);
  const dim3 grid(static_cast<unsigned>(p.nqb * a.heads));
  // the kernel writes the amax parts of ctx when its grid fits them
  p.amax = grid.x <= static_cast<unsigned>(kAmaxParts) ? a.amax : nullptr;
  if (a.head_dim == 128) hipLaunchKernelGGL(attn_fwd_mfma<128>, grid, dim3(64 * kFW), 0, s, p);
  else if (a.head_dim == 64) hipLaunchKernelGGL(attn_fwd_mfma<64>, grid, dim3(64 * kFW), 0, s, p);
  else return hipErrorInvalidValue;
  if (a.amax && !p.amax) return fp8_amax(a.ctx, a.T * p.hl, a.amax, s);
  return hipGetLastError();
}

}  // namespace mtp
