// GEMMs of the column/row-parallel linear maps (forward, data gradient and
// weight gradient), bf16 on CDNA4 MFMA with fp32 accumulation, plus a plain
// fp32 SIMT path for fp32 shards.
//
// C[M,N] = sum_k A(m,k) B(n,k).  The three layouts the layer needs:
//   forward  y  = x W^T : A = x  [M,K] k-major,  B = W [N,K] k-major
//   dgrad    dx = dy W  : A = dy [M,K] k-major,  B = W [K,N] n-major
//   wgrad    dW = dy^T x: A = dy [K,M] m-major,  B = x [K,N] n-major
// Every operand is staged into LDS with 8 consecutive k values per 16-byte
// chunk, which is what one lane feeds to v_mfma_f32_32x32x16_bf16.  k-major
// operands are copied chunk by chunk; m/n-major operands are read as 8x8
// element blocks (8 k-rows of 8 contiguous m), transposed in registers and
// written as 8 k-contiguous chunks.  LDS rows hold 64 k values (8 chunks);
// chunk c of row r lives at slot c ^ (r & 7), so the 32 rows read by the
// lanes of one MFMA operand fetch hit distinct banks.
#include "common.h"
#include "kernels.h"

namespace mtp {
namespace {

constexpr int kBK = 64;
constexpr int kChunks = kBK / 8;
constexpr int kGroupM = 8;

struct GemmParams {
  const bf16_t* A; int64_t lda;
  const bf16_t* B; int64_t ldb;
  int M, N, K;
  void* C; int64_t ldc;
  const void* bias;
  void* aux; int64_t ld_aux;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ (row & 7));
}

// Map the linear block id to a (tile_m, tile_n) pair.  Consecutive block ids
// are dispatched round-robin over the 8 XCDs; the first step gives every XCD
// a contiguous range of tile ids so tiles that share operands share an L2.
// The second step walks tiles in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  int pid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) pid = (pid & 7) * (nb >> 3) + (pid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// Global -> register -> LDS staging of one operand tile of R rows x 64 k.
template <int R, int NT, bool KMAJOR> struct TileLoader;

template <int R, int NT> struct TileLoader<R, NT, true> {
  static constexpr int kPer = R * kChunks / NT;
  static_assert(R * kChunks % NT == 0, "tile/threads mismatch");
  uint4 r[kPer];
  __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int row0, int rmax,
                                       int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      const int row = c >> 3, kc = c & 7;
      const int grow = row0 + row, gk = k0 + kc * 8;
      if (grow < rmax && gk < K)
        r[i] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(grow) * ld + gk);
      else
        r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      lds[swz(c >> 3, c & 7)] = r[i];
    }
  }
};

template <int R, int NT> struct TileLoader<R, NT, false> {
  // R 8x8 blocks (8 k-blocks x R/8 row-blocks); thread tid takes blocks
  // tid, tid+NT, ...
  static constexpr int kBlocks = (R + NT - 1) / NT;
  uint4 r[kBlocks * 8];
  __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int row0, int rmax,
                                       int k0, int K, int tid) {
#pragma unroll
    for (int bi = 0; bi < kBlocks; ++bi) {
      const int b = tid + bi * NT;
      const int rb = b % (R / 8), kb = b / (R / 8);
      const int gr = row0 + rb * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        if (b < R && gr < rmax && gk < K)
          r[bi * 8 + j] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(gk) * ld + gr);
        else
          r[bi * 8 + j] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int bi = 0; bi < kBlocks; ++bi) {
      const int b = tid + bi * NT;
      if (b < R) {
        const int rb = b % (R / 8), kb = b / (R / 8);
        uint4 t[8];
        transpose8x8_bf16(&r[bi * 8], t);
#pragma unroll
        for (int c = 0; c < 8; ++c) lds[swz(rb * 8 + c, kb)] = t[c];
      }
    }
  }
};

template <int EPI, typename ElemT>
__device__ __forceinline__ void epi_apply(const GemmParams& p, int m, int n, float v[4]) {
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
    store4(static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + n, g);
  } else if (EPI == kEpiDGelu) {
    float u[4];
    load4(static_cast<const ElemT*>(p.aux) + static_cast<int64_t>(m) * p.ld_aux + n, u);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] *= gelu_tanh_grad(u[c]);
    store4(static_cast<ElemT*>(p.C) + static_cast<int64_t>(m) * p.ldc + n, v);
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

// One workgroup computes a BM x BN tile with WGM x WGN waves; each wave owns a
// (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA blocks.  The MFMA is issued
// as D = B_frag * A_frag so that each lane ends with 4 consecutive n of one
// row m (8- or 16-byte stores in the epilogue).
template <int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  __shared__ uint4 lds_a[2][BM * kChunks];
  __shared__ uint4 lds_b[2][BN * kChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_coords(p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  TileLoader<BM, NT, AK> la;
  TileLoader<BN, NT, BKM> lb;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (p.K + kBK - 1) / kBK;
  la.load(p.A, p.lda, m0, p.M, 0, p.K, tid);
  lb.load(p.B, p.ldb, n0, p.N, 0, p.K, tid);
  la.store(lds_a[0], tid);
  lb.store(lds_b[0], tid);
  __syncthreads();

  const int lrow = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(p.A, p.lda, m0, p.M, (kt + 1) * kBK, p.K, tid);
      lb.load(p.B, p.ldb, n0, p.N, (kt + 1) * kBK, p.K, tid);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 t = lds_a[cur][swz(wm * WTM + i * 32 + lrow, kk * 2 + lk)];
        af[i] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 t = lds_b[cur][swz(wn * WTN + j * 32 + lrow, kk * 2 + lk)];
        bfr[j] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(lds_a[cur ^ 1], tid);
      lb.store(lds_b[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue: lane holds m = lrow, n = 8*g + 4*lk + c for acc element 4*g + c.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WTM + i * 32 + lrow;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WTN + j * 32 + 8 * g + 4 * lk;
        if (n < p.N) {
          float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]};
          epi_apply<EPI, bf16_t>(p, m, n, v);
        }
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI>
hipError_t launch_bf16(const GemmParams& p0, hipStream_t s) {
  GemmParams p = p0;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int blocks = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, AK, BKM, EPI>), dim3(blocks),
                     dim3(WGM * WGN * 64), 0, s, p);
  return hipGetLastError();
}

// Tile shapes compiled in (BM x BN, 2x2 waves).
enum TileShape : int { kTile256x128 = 0, kTile128x128 = 1, kTile128x256 = 2, kNumTiles = 3 };

int pick_tile(int M, int N) {
  // Fewest full-chip waves of tiles, weighting the smaller tile as slower
  // per flop (it re-reads operands twice as often from LDS and L2).
  constexpr int kCUs = 256;
  const int bm[kNumTiles] = {256, 128, 128};
  const int bn[kNumTiles] = {128, 128, 256};
  const double eff[kNumTiles] = {1.0, 0.8, 1.0};
  int best = 0;
  double best_cost = 1e300;
  for (int t = 0; t < kNumTiles; ++t) {
    const long tiles = static_cast<long>((M + bm[t] - 1) / bm[t]) * ((N + bn[t] - 1) / bn[t]);
    const long waves = (tiles + kCUs - 1) / kCUs;
    const double cost = static_cast<double>(waves) * bm[t] * bn[t] / eff[t];
    if (cost < best_cost - 1e-9) { best_cost = cost; best = t; }
  }
  return best;
}

template <bool AK, bool BKM, int EPI>
hipError_t dispatch_tile(const GemmParams& p, int tile, hipStream_t s) {
  switch (tile) {
    case kTile128x128: return launch_bf16<128, 128, 2, 2, AK, BKM, EPI>(p, s);
    case kTile128x256: return launch_bf16<128, 256, 2, 2, AK, BKM, EPI>(p, s);
    default: return launch_bf16<256, 128, 2, 2, AK, BKM, EPI>(p, s);
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
    if (m < p.M && n < p.N) epi_apply<EPI, float>(p, m, n, acc[i]);
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

GemmParams to_params(const GemmDesc& g) {
  GemmParams p{};
  p.A = static_cast<const bf16_t*>(g.A); p.lda = g.lda;
  p.B = static_cast<const bf16_t*>(g.B); p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.C = g.C; p.ldc = g.ldc;
  p.bias = g.bias; p.aux = g.aux; p.ld_aux = g.ld_aux;
  return p;
}

}  // namespace

// Layout / epilogue combinations the layer uses:
//   forward (k-major, k-major):  Store, Gelu, F32
//   dgrad   (k-major, n-major):  Store, DGelu
//   wgrad   (m-major, n-major):  F32, F32Acc
hipError_t gemm_bf16(const GemmDesc& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const GemmParams p = to_params(g);
  const int tile = (g.tile >= 0 && g.tile < kNumTiles) ? g.tile : pick_tile(g.M, g.N);
  if (g.a_kmajor && g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return dispatch_tile<true, true, kEpiStore>(p, tile, s);
      case kEpiGelu: return dispatch_tile<true, true, kEpiGelu>(p, tile, s);
      case kEpiF32: return dispatch_tile<true, true, kEpiF32>(p, tile, s);
      default: break;
    }
  } else if (g.a_kmajor && !g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return dispatch_tile<true, false, kEpiStore>(p, tile, s);
      case kEpiDGelu: return dispatch_tile<true, false, kEpiDGelu>(p, tile, s);
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
      case kEpiF32: return launch_f32<true, true, kEpiF32>(p, s);
      default: break;
    }
  } else if (g.a_kmajor && !g.b_kmajor) {
    switch (g.epi) {
      case kEpiStore: return launch_f32<true, false, kEpiStore>(p, s);
      case kEpiDGelu: return launch_f32<true, false, kEpiDGelu>(p, s);
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
