// GEMMs of the column/row-parallel linear maps (forward, data gradient and
// weight gradient), bf16 on CDNA4 MFMA with fp32 accumulation, plus a plain
// fp32 SIMT path for fp32 shards.
//
// C[M,N] = sum_k A(m,k) B(n,k).  The three layouts the layer needs:
//   forward  y  = x W^T : A = x  [M,K] k-major,  B = W [N,K] k-major
//   dgrad    dx = dy W  : A = dy [M,K] k-major,  B = W [K,N] n-major
//   wgrad    dW = dy^T x: A = dy [K,M] m-major,  B = x [K,N] n-major
//
// bf16 kernel design (gfx950):
//  * One workgroup computes a BM x BN tile of C with WGM x WGN waves; each
//    wave owns a (BM/WGM) x (BN/WGN) sub-tile of 32x32 blocks computed with
//    v_mfma_f32_32x32x16_bf16.
//  * Operand tiles of 64 k are copied from HBM straight into LDS by
//    buffer_load_dwordx4 ... lds (no VGPR round trip), double-buffered: the
//    next k-tile streams in while the current one feeds the MFMAs.  Every
//    16-byte chunk that lies outside the matrix (ragged M, N or K) gets a
//    buffer offset past the resource's num_records, which the hardware
//    returns as zeros, so no edge needs a separate code path.
//  * k-major operands are stored as rows of 64 k (128 B, 8 chunks); chunk c
//    of row r sits at slot c ^ ((r >> 1) & 7), so the 16 rows read in one
//    LDS cycle by an MFMA operand load hit distinct banks.  A lane's MFMA operand (8
//    consecutive k of one row) is one ds_read_b128.
//  * m/n-major operands are stored as 64 k-rows of the tile's m range; the
//    MFMA operand (8 consecutive k of one m) is gathered by two
//    ds_read_b64_tr_b16, which transpose 4x16 blocks across each group of 16
//    lanes: lane i of a group receives element j from the address supplied
//    by lane 4j + i/4, at sub-element i%4.  64-byte segments of a k-row are
//    XOR-swizzled by k so the 8 k-rows of one transpose read spread over
//    the banks.
//  * The MFMA is issued as D = B_frag * A_frag so that each lane ends with 4
//    consecutive n of one row m (8- or 16-byte stores in the epilogue).
//  * Tiles are ordered so that the workgroups of one XCD (dispatched
//    round-robin over the 8 XCDs) share operand panels in their L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace mtp {
namespace {

constexpr int kBK = 64;
template <int N> struct IntTag { static constexpr int v = N; };
// f(IntTag<I>{}), ..., f(IntTag<N-1>{}) in order.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntTag<I>{});
    static_for<I + 1, N>(f);
  }
}

constexpr int kGroupM = 8;

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct GemmParams {
  const float* scale_a; const float* scale_b;  // FP8 kernels: per-tensor scales
  const bf16_t* A; int64_t lda;
  const bf16_t* B; int64_t ldb;
  int M, N, K;
  void* C; int64_t ldc;
  const void* bias;
  void* aux; int64_t ld_aux;
  int tiles_m, tiles_n;
  uint32_t a_bytes, b_bytes;  // extent of A and B in bytes (< 2^31)
  float* amax;  // FP8 GeLU / GeLU' instances: partial maxima of |C| (nullable)
};

// Map the linear block id to a (tile_m, tile_n) pair.  Consecutive block ids
// are dispatched round-robin over the 8 XCDs; the first step gives every XCD
// a contiguous range of tile ids so tiles that share operands share an L2
// (with nb = 8q + r blocks, the first r XCDs take q + 1 ids, the rest q).
// The second step walks tiles in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nb = gridDim.x;
  const int xcd = blockIdx.x & 7, q = nb >> 3, r = nb & 7;
  const int pid = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + (blockIdx.x >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// Chunk swizzle of a k-major row (8 chunks of 16 B).  A ds_read_b128 is
// served 16 lanes (256 B, all 64 banks) per cycle; the 16 rows those lanes
// read are 2 per 256 B of LDS, so row pairs share a slot pattern and the 8
// pairs get distinct chunk slots.
__device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }

// 64-byte segment swizzle of an m/n-major k-row holding R elements (R/32
// segments).  A transpose read (ds_read_b64_tr_b16) is served one group of
// 16 lanes at a time, and a group reads 32 bytes at one logical segment from
// each of 4 consecutive k-rows: those 4 pieces must land in distinct banks.
//  * R = 128, 256 (rows a multiple of 256 bytes, so every row starts at the
//    same bank): the segment is XORed with f(k), which gives the 4 rows 4
//    distinct segments;
//  * R = 192 (6 segments, rows of 384 bytes, so rows k and k + 2 start at
//    the same bank and k + 1 half the bank width further): an XOR would have
//    to stay inside aligned pairs of segments, and left two rows of every
//    group on the same banks (a third of the LDS cycles of these tiles went
//    to bank conflicts); instead the segment is rotated by bit 1 of k, which
//    with the row parity puts the 4 rows 0, 2, 1, 3 segments apart.
// swz_m maps a logical chunk to its LDS slot (the fragment reads), unswz_m
// a slot back to its logical chunk (the copies); for the XOR they agree.
template <int R>
__device__ __forceinline__ int swz_m(int chunk, int k) {
  constexpr int kSegs = R / 32;
  if constexpr ((kSegs & (kSegs - 1)) == 0) {
    const int f = ((k & 3) | (((k >> 3) & 1) << 2)) & (kSegs - 1);
    return chunk ^ (f << 2);
  } else {
    const int c = chunk + (((k >> 1) & 1) << 2);
    return c >= R / 8 ? c - R / 8 : c;
  }
}
template <int R>
__device__ __forceinline__ int unswz_m(int slot, int k) {
  constexpr int kSegs = R / 32;
  if constexpr ((kSegs & (kSegs - 1)) == 0) {
    return swz_m<R>(slot, k);
  } else {
    const int c = slot - (((k >> 1) & 1) << 2);
    return c < 0 ? c + R / 8 : c;
  }
}

// Issue the copy of one operand tile (R rows of the tile's m or n range x
// 64 k) into one LDS stage.  The stage is R*128 bytes, written 1 KB per
// instruction (64 lanes x 16 B, lane-contiguous); wave w issues
// instructions w*kPer .. w*kPer+kPer-1.
template <int R, int NW, bool KMAJ>
__device__ __forceinline__ void issue_tile(const u32x4& rs, char* stage, int wave,
                                           int lane, int row0, int rmax, int k0, int K,
                                           uint32_t ld_bytes) {
  constexpr int kInstr = R / 8;
  constexpr int kPer = kInstr / NW;
  static_assert(kInstr % NW == 0, "tile rows must split over the waves");
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = wave * kPer + i;
    const int q = j * 64 + lane;
    uint32_t off;
    if (KMAJ) {
      const int row = q >> 3;
      const int lc = (q & 7) ^ swz_k(row);
      const int gr = row0 + row, gk = k0 + lc * 8;
      off = (gr < rmax && gk < K) ? static_cast<uint32_t>(gr) * ld_bytes + gk * 2 : kOOB;
    } else {
      constexpr int kCpr = R / 8;  // 16-byte chunks per k-row
      const int kr = q / kCpr;
      const int lc = unswz_m<R>(q % kCpr, kr);
      const int gk = k0 + kr, gm = row0 + lc * 8;
      off = (gk < K && gm < rmax) ? static_cast<uint32_t>(gk) * ld_bytes + gm * 2 : kOOB;
    }
    copy16_raw(rs, lds_addr(stage) + j * 1024, off);
  }
}

// Byte offsets of the copies of issue_tile at k0 = 0, with the row bound
// applied (a row outside the matrix gets kOOB, which stays past num_records
// when the k offset is added).  For a tile that lies wholly inside K the
// copy offsets are these plus k0 * 2 (k-major) or k0 * ld (m/n-major), so the
// main loop adds one scalar per copy instead of recomputing each offset and
// its bounds.
template <int R, int NW, bool KMAJ>
__device__ __forceinline__ void tile_bases(uint32_t (&base)[R / 8 / NW], int wave, int lane,
                                           int row0, int rmax, uint32_t ld_bytes) {
  constexpr int kPer = R / 8 / NW;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = (wave * kPer + i) * 64 + lane;
    if (KMAJ) {
      const int row = q >> 3;
      const int lc = (q & 7) ^ swz_k(row);
      const int gr = row0 + row;
      base[i] = gr < rmax ? static_cast<uint32_t>(gr) * ld_bytes + lc * 16 : kOOB;
    } else {
      constexpr int kCpr = R / 8;
      const int kr = q / kCpr;
      const int lc = unswz_m<R>(q % kCpr, kr);
      const int gm = row0 + lc * 8;
      base[i] = gm < rmax ? static_cast<uint32_t>(kr) * ld_bytes + gm * 2 : kOOB;
    }
  }
}

// Workgroup barrier without the fence of __syncthreads(), whose release
// semantics make the compiler wait for every outstanding LDS copy
// (vmcnt(0)) first.  The caller's s_waitcnt has already waited for the
// copies the next reads need; the empty asm statements keep the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MFMA operand (8 consecutive k of one row) from a k-major LDS tile.
__device__ __forceinline__ bf16x8 frag_k(const char* t, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(t + row * 128 + ((c ^ swz_k(row)) << 4));
}

// FP8 MFMA operand (32 bytes: 32 consecutive k of one row) of k-step s
// (64 k) of a k-major LDS tile whose rows hold 128 one-byte elements: lane
// group g takes chunks 4s + 2g and 4s + 2g + 1.  Any split of the 64 k over
// the lanes serves, as long as both operands use the same one.
__device__ __forceinline__ i32x8 frag_k8(const char* t, int row, int s, int g) {
  const bf16x8 lo = frag_k(t, row, 4 * s + 2 * g);
  const bf16x8 hi = frag_k(t, row, 4 * s + 2 * g + 1);
  const bf16x8 v[2] = {lo, hi};
  return __builtin_bit_cast(i32x8, v);
}

// MFMA operand from an m/n-major LDS tile of R columns: lane l gets
// rows rb + l%32, k = 16*kk + 8*(l/32) + 0..7.
template <int R>
__device__ __forceinline__ bf16x8 frag_m(const char* t, int rb, int kk, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int k = kk * 16 + (G >> 1) * 8 + (s >> 2);
  const int m = rb + (G & 1) * 16 + (s & 3) * 4;
  const int c = m >> 3, w = (m & 7) * 2;
  const v4i16 lo = tr_read(t + k * (R * 2) + (swz_m<R>(c, k) << 4) + w);
  const v4i16 hi = tr_read(t + (k + 4) * (R * 2) + (swz_m<R>(c, k + 4) << 4) + w);
  return cat_bf16x8(lo, hi);
}

// AMAX: mx also takes the largest |value| stored to C (GeLU, GeLU' and
// SwiGLU' epilogues).
template <int EPI, typename ElemT, bool AMAX = false>
__device__ __forceinline__ void epi_apply(const GemmParams& p, int m, int n, float v[4],
                                          float& mx) {
  if (EPI == kEpiStore || EPI == kEpiGelu || EPI == kEpiF32) {
    if (p.bias) {
      float b[4];
      load4(static_cast<const ElemT*>(p.bias) + n, b);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] += b[c];
    }
  }
  if (EPI == kEpiStore) {
    store4(static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + n, v);
  } else if (EPI == kEpiGelu) {
    store4(static_cast<ElemT*>(p.aux) + static_cast<int64_t>(m) * p.ld_aux + n, v);
    float g[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) g[c] = gelu_tanh(v[c]);
    if constexpr (AMAX) {
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(g[c]));
    }
    store4(static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + n, g);
  } else if (EPI == kEpiDGelu) {
    float u[4];
    load4(static_cast<const ElemT*>(p.aux) + static_cast<int64_t>(m) * p.ld_aux + n, u);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] *= gelu_tanh_grad(u[c]);
    if constexpr (AMAX) {
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(v[c]));
    }
    store4(static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + n, v);
  } else if (EPI == kEpiDSwiGLU) {
    // v = dg at columns n..n+3 (n % 4 == 0): gate and up of these columns
    // sit at interleaved columns 2n..2n+3 and 2n+4..2n+7.
    const int64_t a = static_cast<int64_t>(m) * p.ld_aux + 2 * n;
    float gt[4], up[4], dgate[4], dup[4];
    load4(static_cast<const ElemT*>(p.aux) + a, gt);
    load4(static_cast<const ElemT*>(p.aux) + a + 4, up);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float sg = silu_sigmoid(gt[c]);
      dup[c] = v[c] * gt[c] * sg;
      dgate[c] = v[c] * up[c] * sg * fmaf(gt[c], 1.0f - sg, 1.0f);
    }
    if constexpr (AMAX) {
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fmaxf(fabsf(dgate[c]), fabsf(dup[c])));
    }
    ElemT* o = static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + 2 * n;
    store4(o, dgate);
    store4(o + 4, dup);
  } else if (EPI == kEpiF32) {
    store4(static_cast<float*>(p.C) + static_cast<int64_t>(m) * p.ldc + n, v);
  } else {  // kEpiF32Acc
    float* c = static_cast<float*>(p.C) + static_cast<int64_t>(m) * p.ldc + n;
    float o[4];
    load4(c, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += o[i];
    store4(c, v);
  }
}

// SwiGLU forward epilogue of columns n..n+3 (n % 4 == 0) of the interleaved
// gate|up product: v holds them, pv the partner group (n ^ 4).  Both lanes
// store their group as the pre-activation; the gate lane (n % 8 == 0)
// writes SiLU(gate) * up to output columns n/2 .. n/2+3 (AMAX: and takes
// their largest |value| into mx).
template <typename ElemT, bool AMAX = false>
__device__ __forceinline__ void epi_swiglu(const GemmParams& p, int m, int n, const float v[4],
                                           const float pv[4], float& mx) {
  store4(static_cast<ElemT*>(p.aux) + static_cast<int64_t>(m) * p.ld_aux + n, v);
  if ((n & 4) == 0) {
    float o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = v[c] * silu_sigmoid(v[c]) * pv[c];
    if constexpr (AMAX) {
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(o[c]));
    }
    store4(static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + n / 2, o);
  }
}

// Epilogue of one 32x32 accumulator block whose top-left element is C(mb, nb):
// the wave writes the block (lane: row lane%32, columns 8g + 4(lane/32) ..
// +3 of accumulator elements 4g..4g+3) row-major into its private LDS
// region `stage` (36-float pitch), then reads it back as row segments, so
// every global store (and every load of C or of the GeLU pre-activation)
// covers 8 rows x 32 contiguous columns.
template <int EPI, bool AMAX = false>
__device__ __forceinline__ void epi_block(const GemmParams& p, float* stage, const f32x16& a,
                                          int mb, int nb, int lane, float& mx) {
  constexpr int kPitch = 36;
  const int lrow = lane & 31, lk = lane >> 5;
  const int sr = lane >> 3, sc = (lane & 7) * 4;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(stage + lrow * kPitch + 8 * g + 4 * lk) =
        f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  float v[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(stage + (8 * r + sr) * kPitch + sc);
    v[r][0] = t[0]; v[r][1] = t[1]; v[r][2] = t[2]; v[r][3] = t[3];
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  const int n = nb + sc;
  if constexpr (EPI == kEpiSwiGLU) {
    // lanes l and l ^ 1 hold the gate and up groups of one row
    float pv[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) pv[r][c] = __shfl_xor(v[r][c], 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb + 8 * r + sr;
      if (m < p.M && n < p.N) epi_swiglu<bf16_t, AMAX>(p, m, n, v[r], pv[r], mx);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mb + 8 * r + sr;
      if (m < p.M && n < p.N) epi_apply<EPI, bf16_t, AMAX>(p, m, n, v[r], mx);
    }
  }
}

// F8: operands are FP8 bytes staged exactly like bf16 pairs (the host
// passes K and the leading dimensions in 2-byte units), multiplied by
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) in two 64-k steps per
// 128-byte k-tile; the epilogue applies the two per-tensor scales.  B is
// E4M3; A is E4M3, or E5M2 with A5 (the gradients of the backward).
template <int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI, bool F8 = false,
          bool A5 = false>
__global__ void __launch_bounds__(WGM * WGN * 64, (WGM * WGN + 3) / 4)
gemm_bf16_kernel(GemmParams p) {
  static_assert(!F8 || (AK && BKM), "FP8 operands: k-major only");
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  // NA stages of A and NB of B, each a separate object so the compiler can
  // tell the stage being filled from the stages being read.  With one
  // workgroup per CU anyway: three of both where they fit in LDS (128x256,
  // 256x128), else three of A and two of B where those fit (256x192,
  // 192x256: A's panels are shared by fewer of the tiles an XCD runs at
  // once than B's, so more of A's copies miss L2); else two of both.
  constexpr int kA = BM * 128, kB = BN * 128, kLds = 160 * 1024;
  constexpr bool kOnePerCu = 2 * (kA + kB) > kLds / 2;
  constexpr int NB = (kOnePerCu && 3 * (kA + kB) <= kLds) ? 3 : 2;
  constexpr int NA = (NB == 3 || (kOnePerCu && 3 * kA + 2 * kB < kLds)) ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) char lds_a0[kA];
  __shared__ __attribute__((aligned(1024))) char lds_a1[kA];
  __shared__ __attribute__((aligned(1024))) char lds_a2[NA > 2 ? kA : 1024];
  __shared__ __attribute__((aligned(1024))) char lds_b0[kB];
  __shared__ __attribute__((aligned(1024))) char lds_b1[kB];
  __shared__ __attribute__((aligned(1024))) char lds_b2[NB > 2 ? kB : 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_coords(p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const u32x4 ra = rsrc_words(p.A, p.a_bytes);
  const u32x4 rb = rsrc_words(p.B, p.b_bytes);
  const uint32_t lda_b = static_cast<uint32_t>(p.lda) * 2, ldb_b = static_cast<uint32_t>(p.ldb) * 2;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int lrow = lane & 31, lk = lane >> 5;
  // Operand fragments of one k-step (16 k, or 64 with F8): FM A blocks and
  // FN B blocks.
  using FragT = std::conditional_t<F8, i32x8, bf16x8>;
  struct Frags { FragT a[FM], b[FN]; };
  auto mma = [&](const FragT& b, const FragT& a, const f32x16& c) {
    // the format fields: 0 = E4M3, 1 = E5M2, for the first (B) and second (A)
    // operand as passed
    if constexpr (F8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, A5 ? 1 : 0, 0, 127, 0,
                                                              127);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
  };
  auto load_frags = [&](const char* ta, const char* tb, int kk, Frags& f) {
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < FM; ++i) f.a[i] = frag_k8(ta, wm * WTM + i * 32 + lrow, kk, lk);
#pragma unroll
      for (int j = 0; j < FN; ++j) f.b[j] = frag_k8(tb, wn * WTN + j * 32 + lrow, kk, lk);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        f.a[i] = AK ? frag_k(ta, wm * WTM + i * 32 + lrow, kk * 2 + lk)
                    : frag_m<BM>(ta, wm * WTM + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        f.b[j] = BKM ? frag_k(tb, wn * WTN + j * 32 + lrow, kk * 2 + lk)
                     : frag_m<BN>(tb, wn * WTN + j * 32, kk, lane);
    }
  };
  // The MFMAs of a k-step walk the FM x FN blocks in snake order (odd rows
  // of A fragments take the B fragments backwards), so that consecutive
  // MFMAs at a row change share their B fragment.  The board runs these
  // GEMMs at its power limit, where fewer operand bits changing between
  // instructions buys clock: the 12 shard GEMMs 911.0 / 912.2 -> 908.3 /
  // 906.9 us, the layer step 1.1733 / 1.1653 -> 1.1695 / 1.1609 ms (two
  // interleaved rounds, bit-identical results).
  // LDS reads per k-step (transpose reads come in pairs).
  constexpr int kReads = F8 ? 2 * (FM + FN) : FM * (AK ? 1 : 2) + FN * (BKM ? 1 : 2);
  constexpr int kPerMfma = (kReads + FM * FN - 1) / (FM * FN);
  // MFMAs of one k-step with the fragment reads of the next step spread
  // between them, so LDS latency hides behind the matrix pipeline.  Each
  // k-step runs at raised wave priority, dropped between steps, so that the
  // SIMD's arbiter favours a wave with MFMAs ready over its neighbour at the
  // barrier or in its copy issue (about 1% on the shard GEMMs, measured).
  auto step = [&](const Frags& f, bool prefetch, const char* ta, const char* tb, int kk,
                  Frags& nf) {
    __builtin_amdgcn_s_setprio(1);
    if (prefetch) load_frags(ta, tb, kk, nf);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        const int j = (i & 1) ? FN - 1 - jj : jj;  // snake order
        acc[i][j] = mma(f.b[j], f.a[i], acc[i][j]);
      }
    if (prefetch) {
#pragma unroll
      for (int t = 0; t < FM * FN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, kPerMfma, 0);   // then LDS reads
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // Pipeline over k-tiles (A stage kt % NA and B stage kt % NB hold tile
  // kt):
  //   steps 1..3 of tile kt, each prefetching the next step's fragments;
  //   wait for tile kt+1's copies (copies of later tiles stay in flight)
  //   and for every wave to finish reading tile kt's stages (all of tile
  //   kt's fragments are in registers by now);
  //   then step 3 of tile kt, which prefetches step 0 of tile kt+1 from the
  //   next stages.
  // The copies that refill the stages are issued one per MFMA in two
  // k-steps, the first step of a tile (slot 1) and the step after its
  // barrier (slot 0), rather than as a burst after the barrier, where the
  // copies of all waves queued behind each other and the last waves reached
  // the next barrier late.  With NA = NB = N: B of tile kt+N-1 in slot 1
  // (into the stage tile kt-1 freed), A of tile kt+N in slot 0 (into tile
  // kt's).  With NA = 3, NB = 2: A of tile kt+2 in slot 1 and B of tile kt+2
  // in slot 0, so that at each barrier only the latest A copies are still
  // in flight and the load counter can be waited down to them.
  // The barrier thus sits before the last k-step, whose MFMAs cover the
  // first fragment reads of the next tile.  It is a bare s_barrier: the
  // fence of __syncthreads() would make the compiler wait for every
  // outstanding copy, the deeper stages' included.  Tiles past K (and
  // copies issued for them) are all-zero loads that add nothing.
  const int nk = (p.K + kBK - 1) / kBK;
  Frags f0, f1;
  // One k-step (MFMAs on f, fragment reads of step kk into nf) with nc
  // operand copies issued between its MFMAs, one per MFMA.
  constexpr int kCopiesA = BM / 8 / NW, kCopiesB = BN / 8 / NW;
  constexpr bool kSym = NA == NB;
  // copies that may still be in flight at a barrier
  constexpr int kInFlight = kSym ? (NA - 2) * (kCopiesA + kCopiesB) : kCopiesA;
  auto step_c = [&](const Frags& f, const char* ta, const char* tb, int kk, Frags& nf,
                    auto&& copies, auto nc_tag) {
    constexpr int nc = decltype(nc_tag)::v;
    __builtin_amdgcn_s_setprio(1);
    copies();
    load_frags(ta, tb, kk, nf);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        const int j = (i & 1) ? FN - 1 - jj : jj;  // snake order
        acc[i][j] = mma(f.b[j], f.a[i], acc[i][j]);
      }
#pragma unroll
    for (int t = 0; t < FM * FN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t < nc) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kPerMfma, 0);
    }
    if constexpr (nc > FM * FN) __builtin_amdgcn_sched_group_barrier(0x020, nc - FM * FN, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  uint32_t abase[kCopiesA], bbase[kCopiesB];
  tile_bases<BM, NW, AK>(abase, wave, lane, m0, p.M, lda_b);
  tile_bases<BN, NW, BKM>(bbase, wave, lane, n0, p.N, ldb_b);
  // A tile wholly inside K: the precomputed offsets plus the tile's k offset;
  // else (the ragged last tile, or tiles past K) every chunk's bounds.
  auto copy_a = [&](char* sa, int k0) {
    if (k0 + kBK <= p.K) {
      const uint32_t dk = AK ? static_cast<uint32_t>(k0) * 2 : static_cast<uint32_t>(k0) * lda_b;
#pragma unroll
      for (int i = 0; i < kCopiesA; ++i)
        copy16_raw(ra, lds_addr(sa) + (wave * kCopiesA + i) * 1024, abase[i] + dk);
    } else {
      issue_tile<BM, NW, AK>(ra, sa, wave, lane, m0, p.M, k0, p.K, lda_b);
    }
  };
  auto copy_b = [&](char* sb, int k0) {
    if (k0 + kBK <= p.K) {
      const uint32_t dk = BKM ? static_cast<uint32_t>(k0) * 2 : static_cast<uint32_t>(k0) * ldb_b;
#pragma unroll
      for (int i = 0; i < kCopiesB; ++i)
        copy16_raw(rb, lds_addr(sb) + (wave * kCopiesB + i) * 1024, bbase[i] + dk);
    } else {
      issue_tile<BN, NW, BKM>(rb, sb, wave, lane, n0, p.N, k0, p.K, ldb_b);
    }
  };
  // Stage objects by compile-time index.
  auto sa = [&](auto i) -> char* {
    constexpr int v = decltype(i)::v % NA;
    return v == 0 ? lds_a0 : v == 1 ? lds_a1 : lds_a2;
  };
  auto sb = [&](auto i) -> char* {
    constexpr int v = decltype(i)::v % NB;
    return v == 0 ? lds_b0 : v == 1 ? lds_b1 : lds_b2;
  };
  // Tile kt, with J = kt mod the stage period known at compile time.
  auto tile = [&](auto j, int kt) {
    constexpr int J = decltype(j)::v;
    char* const ca = sa(IntTag<J>{});
    char* const cb = sb(IntTag<J>{});
    char* const na = sa(IntTag<J + 1>{});
    char* const nb = sb(IntTag<J + 1>{});
    if constexpr (kSym) {
      step_c(f0, ca, cb, 1, f1, [&] { copy_b(sb(IntTag<J + NB - 1>{}), (kt + NB - 1) * kBK); },
             IntTag<kCopiesB>{});
    } else {
      step_c(f0, ca, cb, 1, f1, [&] { copy_a(sa(IntTag<J + 2>{}), (kt + 2) * kBK); },
             IntTag<kCopiesA>{});
    }
    if constexpr (!F8) {  // bf16: four 16-k steps per tile, FP8: two 64-k steps
      step(f1, true, ca, cb, 2, f0);
      step(f0, true, ca, cb, 3, f1);
    }
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(kInFlight) : "memory");
    lds_barrier();
    if constexpr (kSym) {
      step_c(f1, na, nb, 0, f0, [&] { copy_a(ca, (kt + NA) * kBK); }, IntTag<kCopiesA>{});
    } else {
      step_c(f1, na, nb, 0, f0, [&] { copy_b(cb, (kt + NB) * kBK); }, IntTag<kCopiesB>{});
    }
  };
  if (nk > 0) {
    // Tiles 0 .. N-2 whole and, with NA = NB = N, A of tile N-1 (its B
    // follows in tile 0); with NA = 3, NB = 2, tiles 0 and 1.
    copy_a(lds_a0, 0);
    copy_b(lds_b0, 0);
    copy_a(lds_a1, kBK);
    if constexpr (!kSym || NA > 2) copy_b(lds_b1, kBK);
    if constexpr (kSym && NA > 2) copy_a(lds_a2, 2 * kBK);
    // Only tile 0 is needed now: the later tiles' copies may stay in flight.
    constexpr int kFirstWait = kSym ? kInFlight + kCopiesA : kCopiesA + kCopiesB;
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kFirstWait) : "memory");
    lds_barrier();
    load_frags(lds_a0, lds_b0, 0, f0);
    // The loop is unrolled over one period of the stage rotation, each tile
    // behind a (uniform) test against the tile count.
    constexpr int kPeriod = NA * NB / (NA == NB ? NA : 1);
    for (int kt = 0; kt < nk; kt += kPeriod)
      static_for<0, kPeriod>([&](auto j) {
        if (kt + decltype(j)::v < nk) tile(j, kt + decltype(j)::v);
      });
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }

  // Epilogue, staged through LDS one 32x32 block at a time (epi_block).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with the stage buffers
  constexpr int kPitch = 36;  // floats per staged row: 32 + 4 (bank spread)
  constexpr int kRegion = 32 * kPitch * 4;
  constexpr int kPerBuf = NW / 4;
  static_assert(kPerBuf * kRegion <= (BM < BN ? BM : BN) * 128, "epilogue staging does not fit");
  char* const base = (wave / kPerBuf) == 0 ? lds_a0
                   : (wave / kPerBuf) == 1 ? lds_a1
                   : (wave / kPerBuf) == 2 ? lds_b0 : lds_b1;
  float* stage = reinterpret_cast<float*>(base + (wave % kPerBuf) * kRegion);
  // FP8 GeLU / SwiGLU outputs and their gradients feed the next
  // quantization: the partial maximum of what this workgroup stores, in
  // the form of the amax pass (slot blockIdx.x, unused slots 0; rounded to
  // bf16 like the values, which keeps the order)
  constexpr bool kAmax = F8 && (EPI == kEpiGelu || EPI == kEpiDGelu || EPI == kEpiSwiGLU ||
                                EPI == kEpiDSwiGLU);
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      if constexpr (F8) {
        const f32x16 v = acc[i][j] * (p.scale_a[0] * p.scale_b[0]);
        epi_block<EPI, kAmax>(p, stage, v, m0 + wm * WTM + i * 32, n0 + wn * WTN + j * 32, lane,
                              mx);
      } else {
        epi_block<EPI>(p, stage, acc[i][j], m0 + wm * WTM + i * 32, n0 + wn * WTN + j * 32, lane,
                       mx);
      }
  if constexpr (kAmax) {
    if (p.amax) {
      mx = warp_max(mx);
      __syncthreads();  // every wave is done with its staging region
      float* wmx = reinterpret_cast<float*>(lds_a0);
      if (lane == 0) wmx[wave] = mx;
      __syncthreads();
      if (threadIdx.x == 0) {
        float m = wmx[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) m = fmaxf(m, wmx[w]);
        p.amax[blockIdx.x] = lo_bf(pack_bf2(m, 0.0f));
      }
      if (blockIdx.x == 0)
        for (int i = static_cast<int>(gridDim.x) + threadIdx.x; i < kAmaxParts; i += NW * 64)
          p.amax[i] = 0.0f;
    }
  }
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI, bool F8 = false,
          bool A5 = false>
hipError_t launch_bf16(const GemmParams& p0, hipStream_t s) {
  GemmParams p = p0;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int blocks = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, AK, BKM, EPI, F8, A5>), dim3(blocks),
                     dim3(WGM * WGN * 64), 0, s, p);
  return hipGetLastError();
}

// Tile shapes compiled in.
enum TileShape : int {
  kTile256x256 = 0,  // 8 waves (2x4), 128 KB LDS
  kTile256x128 = 1,  // 8 waves (4x2), three stages, 144 KB LDS
  kTile128x256 = 2,  // 8 waves (2x4), three stages, 144 KB LDS
  kTile128x128 = 3,  // 4 waves (2x2), 64 KB LDS
  kTile256x192 = 4,  // 8 waves (4x2), three A and two B stages, 144 KB LDS
  kTile192x256 = 5,  // 8 waves (2x4), three A and two B stages, 136 KB LDS
  kNumTiles = 6
};

int pick_tile(int M, int N) {
  // Cost = rounds of tiles over the 256 CUs x tile area / relative
  // efficiency (measured on the 7B shard shapes).  128x128 tiles run two
  // per CU, or one per CU when they fit in one round; one such round (two
  // stages, four waves) measured slower than a round of three-stage
  // 128x256 tiles of twice the area (2048 x 2048 x 4096: 46.7 vs 44.0 us).
  constexpr int kCUs = 256;
  const int bm[kNumTiles] = {256, 256, 128, 128, 256, 192};
  const int bn[kNumTiles] = {256, 128, 256, 128, 192, 256};
  const int per_cu[kNumTiles] = {1, 1, 1, 2, 1, 1};
  const double eff[kNumTiles] = {1.0, 0.9, 0.92, 0.87, 0.96, 0.96};
  constexpr double kEffAlone128 = 0.45;
  // Equal costs go to the tile grid that pads less (M = 5504, N = 4096:
  // 192x256 covers 1.2% padding, 256x192 5.5%; measured 90.6 vs 93.3 us).
  int best = 0;
  double best_cost = 1e300, best_pad = 1e300;
  for (int t = 0; t < kNumTiles; ++t) {
    const long tiles = static_cast<long>((M + bm[t] - 1) / bm[t]) * ((N + bn[t] - 1) / bn[t]);
    const double area = static_cast<double>(bm[t]) * bn[t];
    const double pad = static_cast<double>(tiles) * area;
    double cost;
    if (per_cu[t] == 2 && tiles <= kCUs) {
      cost = area / kEffAlone128;
    } else {
      const long slots = static_cast<long>(kCUs) * per_cu[t];
      cost = static_cast<double>((tiles + slots - 1) / slots) * per_cu[t] * area / eff[t];
    }
    if (cost < best_cost - 1e-9 || (cost < best_cost + 1e-9 && pad < best_pad)) {
      best_cost = cost;
      best_pad = pad;
      best = t;
    }
  }
  return best;
}

template <bool AK, bool BKM, int EPI>
hipError_t dispatch_tile(const GemmParams& p, int tile, hipStream_t s) {
  switch (tile) {
    case kTile256x128: return launch_bf16<256, 128, 4, 2, AK, BKM, EPI>(p, s);
    case kTile128x256: return launch_bf16<128, 256, 2, 4, AK, BKM, EPI>(p, s);
    case kTile128x128: return launch_bf16<128, 128, 2, 2, AK, BKM, EPI>(p, s);
    case kTile256x192: return launch_bf16<256, 192, 4, 2, AK, BKM, EPI>(p, s);
    case kTile192x256: return launch_bf16<192, 256, 2, 4, AK, BKM, EPI>(p, s);
    default: return launch_bf16<256, 256, 2, 4, AK, BKM, EPI>(p, s);
  }
}

// FP8 tiles: 128x256, 256x128, 128x128 and 256x192 (64x96 wave tiles, the
// largest whose doubled FP8 fragments fit the 256 registers of two waves
// per SIMD: 239 of them); 256x192 fills the chip in one round where
// 128x256 needs one and a half (M = 2048 with N = 6144 or 5504), and stages
// fewer bytes per k-tile than a 128x384 tile of the same area (measured
// 52-55 vs 57-60 us).  Chosen by the cost of pick_tile: rounds x tile area
// / efficiency.
constexpr int kTileF8_256x192 = kNumTiles;
int pick_tile_fp8(int M, int N) {
  constexpr int kCUs = 256;
  const int cand[4] = {kTile128x256, kTile256x128, kTile128x128, kTileF8_256x192};
  const int bm[4] = {128, 256, 128, 256}, bn[4] = {256, 128, 128, 192}, per_cu[4] = {1, 1, 2, 1};
  const double eff[4] = {0.92, 0.9, 0.87, 0.92};
  int best = kTile128x256;
  double best_cost = 1e300;
  for (int t = 0; t < 4; ++t) {
    const long tiles = static_cast<long>((M + bm[t] - 1) / bm[t]) * ((N + bn[t] - 1) / bn[t]);
    const long slots = static_cast<long>(kCUs) * per_cu[t];
    const double cost = static_cast<double>((tiles + slots - 1) / slots) * per_cu[t] *
                        bm[t] * bn[t] / eff[t];
    if (cost < best_cost - 1e-9) { best_cost = cost; best = cand[t]; }
  }
  return best;
}

template <int EPI, bool A5>
hipError_t dispatch_fp8(const GemmParams& p, int tile, hipStream_t s) {
  switch (tile) {
    case kTile256x128: return launch_bf16<256, 128, 4, 2, true, true, EPI, true, A5>(p, s);
    case kTile128x128: return launch_bf16<128, 128, 2, 2, true, true, EPI, true, A5>(p, s);
    case kTileF8_256x192: return launch_bf16<256, 192, 4, 2, true, true, EPI, true, A5>(p, s);
    default: return launch_bf16<128, 256, 2, 4, true, true, EPI, true, A5>(p, s);
  }
}

// ------------------------------------------------------------ fp32 path
constexpr int kF32Tile = 64;
constexpr int kF32BK = 16;

template <bool AK, bool BKM, int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmParams p, const float* A,
                                                      const float* B) {
  __shared__ float as[kF32BK][kF32Tile + 4];
  __shared__ float bs[kF32BK][kF32Tile + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * kF32Tile, n0 = blockIdx.x * kF32Tile;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += kF32BK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + e * 256;
      int row, k;
      if (AK) { row = idx / kF32BK; k = idx % kF32BK; } else { k = idx / kF32Tile; row = idx % kF32Tile; }
      const int gm = m0 + row, gk = k0 + k;
      float v = 0.0f;
      if (gm < p.M && gk < p.K)
        v = AK ? A[static_cast<int64_t>(gm) * p.lda + gk] : A[static_cast<int64_t>(gk) * p.lda + gm];
      as[k][row] = v;
      if (BKM) { row = idx / kF32BK; k = idx % kF32BK; } else { k = idx / kF32Tile; row = idx % kF32Tile; }
      const int gn = n0 + row, gk2 = k0 + k;
      float w = 0.0f;
      if (gn < p.N && gk2 < p.K)
        w = BKM ? B[static_cast<int64_t>(gn) * p.ldb + gk2] : B[static_cast<int64_t>(gk2) * p.ldb + gn];
      bs[k][row] = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kF32BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[k][ty * 4 + i];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = bs[k][tx * 4 + c];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(a[i], b[c], acc[i][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i, n = n0 + tx * 4;
    if constexpr (EPI == kEpiSwiGLU) {
      // threads tx and tx ^ 1 (lanes l and l ^ 1) hold the gate and up groups
      float pv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) pv[c] = __shfl_xor(acc[i][c], 1);
      float unused = 0.0f;
      if (m < p.M && n < p.N) epi_swiglu<float>(p, m, n, acc[i], pv, unused);
    } else {
      float unused = 0.0f;
      if (m < p.M && n < p.N) epi_apply<EPI, float>(p, m, n, acc[i], unused);
    }
  }
}

template <bool AK, bool BKM, int EPI>
hipError_t launch_f32(const GemmParams& p, hipStream_t s) {
  dim3 grid((p.N + kF32Tile - 1) / kF32Tile, (p.M + kF32Tile - 1) / kF32Tile);
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BKM, EPI>), grid, dim3(256), 0, s, p,
                     static_cast<const float*>(static_cast<const void*>(p.A)),
                     static_cast<const float*>(static_cast<const void*>(p.B)));
  return hipGetLastError();
}

// Bytes spanned by an operand stored with leading dimension ld: rows x ld
// elements for the leading axis, the last row only up to its used width.
int64_t operand_bytes(bool kmajor, int rows, int K, int64_t ld) {
  const int64_t outer = kmajor ? rows : K;
  const int64_t inner = kmajor ? K : rows;
  if (outer == 0 || inner == 0) return 0;
  return ((outer - 1) * ld + inner) * 2;
}

GemmParams to_params(const GemmDesc& g) {
  GemmParams p{};
  p.scale_a = g.scale_a; p.scale_b = g.scale_b;
  p.A = static_cast<const bf16_t*>(g.A); p.lda = g.lda;
  p.B = static_cast<const bf16_t*>(g.B); p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.C = g.C; p.ldc = g.ldc;
  p.bias = g.bias; p.aux = g.aux; p.ld_aux = g.ld_aux;
  return p;
}

}  // namespace

// Layout / epilogue combinations the layer uses:
//   forward (k-major, k-major):  Store, Gelu, SwiGLU, F32
//   dgrad   (k-major, n-major):  Store, DGelu, DSwiGLU
//   wgrad   (m-major, n-major):  F32, F32Acc
hipError_t gemm_bf16(const GemmDesc& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.fp8) {
    // bytes staged as bf16 pairs: K and the leading dimensions in 2-byte units
    // forward (E4M3 A): Store, Gelu, SwiGLU; data gradient (E5M2 A): Store,
    // DGelu, DSwiGLU; weight gradient (E5M2 A): F32, F32Acc
    const bool ok_epi = g.a_e5m2 ? (g.epi == kEpiStore || g.epi == kEpiDGelu ||
                                    g.epi == kEpiDSwiGLU || g.epi == kEpiF32 ||
                                    g.epi == kEpiF32Acc)
                                 : (g.epi == kEpiStore || g.epi == kEpiGelu ||
                                    g.epi == kEpiSwiGLU);
    // SwiGLU pairs the gate and up groups of 4 columns within 8
    if (!g.a_kmajor || !g.b_kmajor || (g.K & 15) || (g.lda & 15) || (g.ldb & 15) || (g.N & 3) ||
        (g.epi == kEpiSwiGLU && (g.N & 7)) || !g.scale_a || !g.scale_b || !ok_epi)
      return hipErrorInvalidValue;
    GemmDesc h = g;
    h.K = g.K / 2; h.lda = g.lda / 2; h.ldb = g.ldb / 2;
    GemmParams p = to_params(h);
    const int64_t ab = operand_bytes(true, h.M, h.K, h.lda);
    const int64_t bb = operand_bytes(true, h.N, h.K, h.ldb);
    if (ab >= static_cast<int64_t>(kOOB) || bb >= static_cast<int64_t>(kOOB)) return hipErrorInvalidValue;
    p.a_bytes = static_cast<uint32_t>(ab);
    p.b_bytes = static_cast<uint32_t>(bb);
    const int tile = pick_tile_fp8(g.M, g.N);
    // the epilogue writes the amax parts of C when its grid fits them,
    // otherwise a pass over C does
    bool amax_pass = false;
    // columns of C: SwiGLU halves the product's, SwiGLU' doubles them
    const int64_t c_cols = g.epi == kEpiSwiGLU ? g.N / 2 : g.epi == kEpiDSwiGLU ? 2LL * g.N : g.N;
    if (g.amax) {
      if ((g.epi != kEpiGelu && g.epi != kEpiDGelu && g.epi != kEpiSwiGLU &&
           g.epi != kEpiDSwiGLU) || g.ldc != c_cols)
        return hipErrorInvalidValue;
      const int bm = tile == kTile256x128 || tile == kTileF8_256x192 ? 256 : 128;
      const int bn = tile == kTile256x128 || tile == kTile128x128 ? 128
                     : tile == kTileF8_256x192 ? 192 : 256;
      const int64_t tiles = static_cast<int64_t>((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
      if (tiles <= kAmaxParts) p.amax = g.amax;
      else amax_pass = true;
    }
    hipError_t e;
    if (!g.a_e5m2) {
      switch (g.epi) {
        case kEpiGelu: e = dispatch_fp8<kEpiGelu, false>(p, tile, s); break;
        case kEpiSwiGLU: e = dispatch_fp8<kEpiSwiGLU, false>(p, tile, s); break;
        default: e = dispatch_fp8<kEpiStore, false>(p, tile, s); break;
      }
    } else {
      switch (g.epi) {
        case kEpiStore: e = dispatch_fp8<kEpiStore, true>(p, tile, s); break;
        case kEpiDGelu: e = dispatch_fp8<kEpiDGelu, true>(p, tile, s); break;
        case kEpiDSwiGLU: e = dispatch_fp8<kEpiDSwiGLU, true>(p, tile, s); break;
        case kEpiF32: e = dispatch_fp8<kEpiF32, true>(p, tile, s); break;
        default: e = dispatch_fp8<kEpiF32Acc, true>(p, tile, s); break;
      }
    }
    if (e != hipSuccess || !amax_pass) return e;
    return fp8_amax(g.C, static_cast<int64_t>(g.M) * c_cols, g.amax, s);
  }
  GemmParams p = to_params(g);
  // Buffer offsets are 32-bit and the edge handling needs every valid byte
  // offset below kOOB; the 16-byte chunks need 8-aligned rows.
  const int64_t ab = operand_bytes(g.a_kmajor, g.M, g.K, g.lda);
  const int64_t bb = operand_bytes(g.b_kmajor, g.N, g.K, g.ldb);
  if (ab >= static_cast<int64_t>(kOOB) || bb >= static_cast<int64_t>(kOOB)) return hipErrorInvalidValue;
  if ((g.lda & 7) || (g.ldb & 7) || (g.a_kmajor ? (g.K & 7) : (g.M & 7)) ||
      (g.b_kmajor ? (g.K & 7) : (g.N & 7)) || (g.N & 3))
    return hipErrorInvalidValue;
  p.a_bytes = static_cast<uint32_t>(ab);
  p.b_bytes = static_cast<uint32_t>(bb);
  const int tile = pick_tile(g.M, g.N);
  if (g.a_kmajor && g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return dispatch_tile<true, true, kEpiStore>(p, tile, s);
      case kEpiGelu: return dispatch_tile<true, true, kEpiGelu>(p, tile, s);
      case kEpiSwiGLU: return dispatch_tile<true, true, kEpiSwiGLU>(p, tile, s);
      case kEpiF32: return dispatch_tile<true, true, kEpiF32>(p, tile, s);
      default: break;
    }
  } else if (g.a_kmajor && !g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return dispatch_tile<true, false, kEpiStore>(p, tile, s);
      case kEpiDGelu: return dispatch_tile<true, false, kEpiDGelu>(p, tile, s);
      case kEpiDSwiGLU: return dispatch_tile<true, false, kEpiDSwiGLU>(p, tile, s);
      default: break;
    }
  } else if (!g.a_kmajor && !g.b_kmajor) {
    switch (g.epi) {
      case kEpiF32: return dispatch_tile<false, false, kEpiF32>(p, tile, s);
      case kEpiF32Acc: return dispatch_tile<false, false, kEpiF32Acc>(p, tile, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t gemm_f32(const GemmDesc& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const GemmParams p = to_params(g);
  if (g.a_kmajor && g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return launch_f32<true, true, kEpiStore>(p, s);
      case kEpiGelu: return launch_f32<true, true, kEpiGelu>(p, s);
      case kEpiSwiGLU: return launch_f32<true, true, kEpiSwiGLU>(p, s);
      case kEpiF32: return launch_f32<true, true, kEpiF32>(p, s);
      default: break;
    }
  } else if (g.a_kmajor && !g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return launch_f32<true, false, kEpiStore>(p, s);
      case kEpiDGelu: return launch_f32<true, false, kEpiDGelu>(p, s);
      case kEpiDSwiGLU: return launch_f32<true, false, kEpiDSwiGLU>(p, s);
      default: break;
    }
  } else if (!g.a_kmajor && !g.b_kmajor) {
    switch (g.epi) {
      case kEpiF32: return launch_f32<false, false, kEpiF32>(p, s);
      case kEpiF32Acc: return launch_f32<false, false, kEpiF32Acc>(p, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mtp
