// kp_linear: the dense projections on either side of the sparse path, as one strided-batched bf16 GEMM
//   C[b][m][n] = alpha * sum_k A[b][m][k] * W[b][n][k]      (fp32 accumulation, one rounding on the store)
//
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: the indexer cache holds a
// key and a gate per token (one projection of the hidden state gives both); the indexer and the MLA low-rank
// paths stay unquantized.  [MAX glm5_next API page, compute_dtype]: the indexer and kv_b_proj run in the compute
// dtype.  Absorbed MLA moves the query into latent space per head (W_UK[h]^T q) and the latent output back
// (W_UV[h] o): a batch over heads of the same product.
//
// Every operand is K-contiguous (a weight is stored output-major, as a linear layer keeps it), so both MFMA
// operands are plain 16-byte row reads.  One block of 4 waves per BM x BN output tile.  The block computes the
// tile transposed, D[n][m] = W . A^T on 16x16x32 bf16 MFMA (weight rows = M operand, activation rows = N
// operand), so each lane ends with 4 consecutive output columns of one row: one 8- or 16-byte store.
//   load   k advances BK (64 or 32) at a time: one 2 BK-byte segment of every tile row per stage.  Each wave moves
//          1 KiB of rows per direct global->LDS instruction (16 bytes a lane, no register staging) into a ring of 4
//          stage buffers, three stages ahead, with one barrier per stage.  Rows are XOR-swizzled (see ln_swz) so the
//          fragment reads are conflict-free.  Rows past M or N read row M-1 / N-1 (their results are never
//          stored), so every wave issues the same loads every stage and the waits are exact counts.
//   math   wave (wn, wm) owns the BN/2 x BM/2 quarter of the tile: (BN/32) x (BM/32) MFMA tiles, BK/32 k-steps a
//          stage.
// Tiles are numbered m-fastest under one weight tile, and with a grid that is a multiple of 8 consecutive tile
// numbers go to the same XCD (blocks are dealt to the 8 XCDs round-robin), so blocks sharing a weight tile share
// that XCD's L2.
//
// Bound: the decode shapes (M = tokens of a step, tens) stream their weights once -- HBM; the prefill shapes
// (M = thousands) are MFMA-bound at 2 M N K flop.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int LN_THREADS = 256;
constexpr int LN_NBUF = 4;   // stage buffers
constexpr int LN_AHEAD = 3;  // stages in flight ahead of the one being multiplied

// A stage holds BK of k for every tile row: CPR = BK / 8 chunks of 16 bytes.  Chunk c of row r sits at position
// c ^ ln_swz(r) of the row.  A fragment read takes one chunk of 16 consecutive rows; 16 / CPR consecutive rows
// fill the 256 bytes of the 64 banks once, and (r / (16 / CPR)) mod CPR gives each such group its own chunk
// positions: 16 distinct 16-byte bank groups (128-byte rows: (r >> 1) & 7; 64-byte rows: (r >> 2) & 3).
template <int CPR>
__device__ __forceinline__ int ln_swz(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}

template <int BM, int BN, int BK, class TC>
__global__ __launch_bounds__(LN_THREADS) void linear_kernel(const bf16* __restrict__ A, int64_t lda, int64_t sa,
                                                            const bf16* __restrict__ W, int64_t ldw, int64_t sw,
                                                            TC* __restrict__ C, int64_t ldc, int64_t sc, int M,
                                                            int N, int K, float alpha, int tiles_m, int tiles_n,
                                                            int splits, int nk_per, f32x4* __restrict__ part) {
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row and stage
  constexpr int RPI = 64 / CPR;              // tile rows per direct-load instruction (1 KiB)
  constexpr int LA = BM / (4 * RPI), LW = BN / (4 * RPI);  // direct-load instructions per wave per stage
  constexpr int TN = BN / 32, TM = BM / 32;  // MFMA tiles per wave along n and m
  constexpr int KS = BK / 32;                // MFMA k-steps per stage
  static_assert(LA >= 1 && LW >= 1 && KS >= 1, "tile shape");
  __shared__ __align__(1024) bf16 sA[LN_NBUF][BM * BK];
  __shared__ __align__(1024) bf16 sW[LN_NBUF][BN * BK];

  int bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) {
    const int per = gridDim.x >> 3;
    bid = (bid & 7) * per + (bid >> 3);
  }
  const int sp = bid % splits;  // k-split of this block
  bid /= splits;
  const int per_b = tiles_m * tiles_n;
  const int b = bid / per_b;
  const int t = bid - b * per_b;
  const int tn = t / tiles_m, tm = t - tn * tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  A += b * sa;
  W += b * sw;
  C += b * sc;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;

  // per-lane source of each load instruction at k = 0: row RPI (wave * L + i) + lane / CPR of the tile, the
  // chunk whose swizzled position is lane % CPR
  const bf16* srcA[LA];
  const bf16* srcW[LW];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = RPI * (wave * LA + i) + lane / CPR;
    srcA[i] = A + int64_t(min(m0 + r, M - 1)) * lda + 8 * ((lane % CPR) ^ ln_swz<CPR>(r));
  }
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int r = RPI * (wave * LW + i) + lane / CPR;
    srcW[i] = W + int64_t(min(n0 + r, N - 1)) * ldw + 8 * ((lane % CPR) ^ ln_swz<CPR>(r));
  }
  // this block's stages: [s0, s0 + nk) of the K / BK
  const int s0 = sp * nk_per;
  const int nk = min(nk_per, K / BK - s0);
  // stage s into buffer s % 4; a stage past the end re-reads the last one (never multiplied), so every
  // iteration issues LA + LW loads and the wait below is exact
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int64_t k0 = int64_t(s0 + min(s, nk - 1)) * BK;
    const uint32_t ba = lds_off(sA[s % LN_NBUF]), bw = lds_off(sW[s % LN_NBUF]);
#pragma unroll
    for (int i = 0; i < LA; ++i) lds_dma16(srcA[i] + k0, ba + uint32_t(1024 * (wave * LA + i)));
#pragma unroll
    for (int i = 0; i < LW; ++i) lds_dma16(srcW[i] + k0, bw + uint32_t(1024 * (wave * LW + i)));
  };

  // fragment rows of this wave: weight rows wn * BN/2 + 16 a + l16, activation rows wm * BM/2 + 16 c + l16; the
  // swizzle of a row depends on l16 only (tile rows are 16-aligned), so each read is a per-lane base plus a
  // constant, XOR a per-lane chunk position
  const int wn = wave >> 1, wm = wave & 1;
  const int sw_l = ln_swz<CPR>(l16);
  f32x4 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int c = 0; c < TM; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto multiply = [&](int s) __attribute__((always_inline)) {
    const uint32_t ba = lds_off(sA[s % LN_NBUF]), bw = lds_off(sW[s % LN_NBUF]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t cpos = 16 * ((4 * ks + g) ^ sw_l);
      bf16x8 fw[TN], fa[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a) fw[a] = lds_load<bf16x8>(bw + 2 * BK * (wn * (BN / 2) + 16 * a + l16) + cpos);
#pragma unroll
      for (int c = 0; c < TM; ++c) fa[c] = lds_load<bf16x8>(ba + 2 * BK * (wm * (BM / 2) + 16 * c + l16) + cpos);
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c) acc[a][c] = mfma16(fw[a], fa[c], acc[a][c]);
    }
  };

#pragma unroll
  for (int s = 0; s < LN_AHEAD; ++s) issue(s);
  for (int s = 0; s < nk; ++s) {
    // stages s .. s+2 are in flight: wait for s, publish it; after the barrier every wave is past multiply(s-1),
    // so buffer (s+3) % 4 = (s-1) % 4 is free for stage s + 3
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((LN_AHEAD - 1) * (LA + LW)));
    __syncthreads();
    issue(s + LN_AHEAD);
    multiply(s);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land in LDS after the block ends

  if (splits > 1) {
    // split K: store the fp32 partial tile in lane order, [tile][split][wave][n tile][m tile][lane]; the reduce
    // kernel adds the splits in order and writes the output
    f32x4* pt = part + (int64_t(bid) * splits + sp) * (4 * TN * TM * 64) + (wave * TN * TM) * 64 + lane;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int c = 0; c < TM; ++c) pt[(a * TM + c) * 64] = acc[a][c];
    return;
  }

  // lane holds D[n][m] for n = tile n + 4 g .. +3, m = tile m + l16
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n0 + wn * (BN / 2) + 16 * a + 4 * g;
#pragma unroll
    for (int c = 0; c < TM; ++c) {
      const int m = m0 + wm * (BM / 2) + 16 * c + l16;
      if (m >= M || n >= N) continue;
      const f32x4 v = acc[a][c] * alpha;
      TC* dst = C + int64_t(m) * ldc + n;
      if (n + 3 < N) {
        if constexpr (sizeof(TC) == 2) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < N) dst[i] = Elem<TC>::from_f32(v[i]);
      }
    }
  }
}

// k-splits for a call shape: enough blocks to keep every CU streaming (about 2 per CU) when the tile grid is
// small, each split at least 4 stages long; a pure function of the shape
// Split-K reduction: one thread per 4 outputs (one lane's f32x4 of one MFMA tile of one wave); the partials of the
// splits are added in split order, scaled once and rounded once, and stored as the unsplit kernel stores them.
template <int BM, int BN, class TC>
__global__ __launch_bounds__(256) void linear_reduce_kernel(const f32x4* __restrict__ part, int splits,
                                                            TC* __restrict__ C, int64_t ldc, int64_t sc, int M, int N,
                                                            float alpha, int tiles_m, int tiles_n) {
  constexpr int TN = BN / 32, TM = BM / 32, TILE = 4 * TN * TM * 64;
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;  // f32x4 index over all tiles
  const int64_t tile = e / TILE;
  const int r = int(e - tile * TILE);
  const int lane = r & 63, ac = (r >> 6) % (TN * TM), wave = (r >> 6) / (TN * TM);
  const int a = ac / TM, c = ac - a * TM;
  const int per_b = tiles_m * tiles_n;
  const int b = int(tile / per_b), t = int(tile - int64_t(b) * per_b);
  const int tn = t / tiles_m, tm = t - tn * tiles_m;
  const int wn = wave >> 1, wm = wave & 1, l16 = lane & 15, g = lane >> 4;
  const int n = tn * BN + wn * (BN / 2) + 16 * a + 4 * g;
  const int m = tm * BM + wm * (BM / 2) + 16 * c + l16;
  if (m >= M || n >= N) return;
  const f32x4* p = part + tile * splits * TILE + r;
  f32x4 v = p[0];
  for (int q = 1; q < splits; ++q) v += p[int64_t(q) * TILE];
  v *= alpha;
  TC* dst = C + int64_t(b) * sc + int64_t(m) * ldc + n;
  if (n + 3 < N) {
    if constexpr (sizeof(TC) == 2) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < N) dst[i] = Elem<TC>::from_f32(v[i]);
  }
}

// Tile shape for a call: a decode step (few rows) takes 64 x 64 tiles with 64-wide k stages (64 KiB of LDS, two
// blocks per CU); more rows take 128 x 128 tiles with 32-wide k stages (again 64 KiB: two blocks per CU, so one
// block's first loads and last stores overlap the other's products).
struct LinearTile {
  int BM, BN, BK;
};
static LinearTile linear_tile(int M) { return M <= 64 ? LinearTile{64, 64, 64} : LinearTile{128, 128, 32}; }

// k-splits for a call shape: only when there are fewer output tiles than compute units, enough splits for about
// two blocks per CU, each at least 4 stages long; a pure function of the shape
static int linear_splits(const LinearTile& t, int batch, int M, int N, int K, int cus) {
  const int64_t tiles = int64_t(batch) * ((M + t.BM - 1) / t.BM) * ((N + t.BN - 1) / t.BN);
  if (tiles >= cus) return 1;
  const int nk = K / t.BK;
  int sp = int((2 * int64_t(cus) + tiles - 1) / tiles);
  sp = max(1, min(sp, nk / 4));
  const int per = (nk + sp - 1) / sp;
  return (nk + per - 1) / per;  // every split non-empty
}

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

size_t linear_workspace(int batch, int M, int N, int K) {
  if (batch <= 0 || M <= 0 || N <= 0 || K < 64) return 0;
  const LinearTile t = linear_tile(M);
  const int sp = linear_splits(t, batch, M, N, K, 256);
  if (sp <= 1) return 0;
  const int64_t tiles = int64_t(batch) * ((M + t.BM - 1) / t.BM) * ((N + t.BN - 1) / t.BN);
  return size_t(tiles) * sp * t.BM * t.BN * sizeof(float);
}

template <int BM, int BN, int BK>
static kp_status launch_tile(const LinearLaunch& a, hipStream_t s) {
  const LinearTile tl{BM, BN, BK};
  const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  const int64_t tiles = int64_t(a.batch) * tiles_m * tiles_n;
  int sp = 1;
  f32x4* part = nullptr;
  if (a.ws) {
    // the split count is sized for 256 CUs (the workspace query cannot see the device); fewer fit the workspace
    sp = linear_splits(tl, a.batch, a.M, a.N, a.K, min(device_cus(), 256));
    const size_t need = size_t(tiles) * sp * BM * BN * sizeof(float);
    if (sp > 1 && a.ws_bytes >= need) {
      part = static_cast<f32x4*>(a.ws);
    } else {
      sp = 1;
    }
  }
  const int nk = a.K / BK, nk_per = (nk + sp - 1) / sp;
  const int64_t blocks = tiles * sp;
  if (blocks > 0x7fffffff) {
    set_error("kp_linear: %lld blocks exceed the grid", (long long)blocks);
    return KP_ERR_INVALID_ARG;
  }
  const int64_t rblocks = tiles * (BM * BN / 4) / 256;  // reduce: one thread per f32x4 of the partial tiles
  if (a.c_dtype == KP_DTYPE_BF16) {
    linear_kernel<BM, BN, BK, bf16><<<dim3(unsigned(blocks)), dim3(LN_THREADS), 0, s>>>(
        (const bf16*)a.A, a.lda, a.sa, (const bf16*)a.W, a.ldw, a.sw, (bf16*)a.C, a.ldc, a.sc, a.M, a.N, a.K,
        a.alpha, tiles_m, tiles_n, sp, nk_per, part);
    if (sp > 1)
      linear_reduce_kernel<BM, BN, bf16><<<dim3(unsigned(rblocks)), dim3(256), 0, s>>>(
          part, sp, (bf16*)a.C, a.ldc, a.sc, a.M, a.N, a.alpha, tiles_m, tiles_n);
  } else {
    linear_kernel<BM, BN, BK, float><<<dim3(unsigned(blocks)), dim3(LN_THREADS), 0, s>>>(
        (const bf16*)a.A, a.lda, a.sa, (const bf16*)a.W, a.ldw, a.sw, (float*)a.C, a.ldc, a.sc, a.M, a.N, a.K,
        a.alpha, tiles_m, tiles_n, sp, nk_per, part);
    if (sp > 1)
      linear_reduce_kernel<BM, BN, float><<<dim3(unsigned(rblocks)), dim3(256), 0, s>>>(
          part, sp, (float*)a.C, a.ldc, a.sc, a.M, a.N, a.alpha, tiles_m, tiles_n);
  }
  return check_launch("kp_linear");
}

kp_status launch_linear(const LinearLaunch& a, hipStream_t s) {
  if (a.batch == 0 || a.M == 0 || a.N == 0) return KP_OK;
  if (linear_tile(a.M).BM == 64) return launch_tile<64, 64, 64>(a, s);
  return launch_tile<128, 128, 32>(a, s);
}

}  // namespace kp
