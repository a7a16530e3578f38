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
// operand), so each lane ends with 4 consecutive output columns of one row.  A bf16 output tile then goes through
// LDS (the stage ring is free by then) and out as whole 16-byte row chunks: the 4096-token absorb and un-absorb,
// which write 268 / 134 MB, ran 239 -> 195 and 207 -> 159 us with it; other outputs are stored from the lanes.
//   load   k advances BK at a time (64 for both tile shapes; the kernel also takes 32): one 2 BK-byte segment of
//          every tile row per stage.  Each wave moves 1 KiB of rows per direct global->LDS instruction (16 bytes a
//          lane, no register staging) into a ring of NBUF stage buffers, NBUF - 1 stages ahead, with one barrier
//          per stage.  Rows are XOR-swizzled (see ln_swz) so the fragment reads are conflict-free.  Rows past M
//          or N read row M-1 / N-1 (their results are never stored), so every wave issues the same loads every
//          stage and the waits are exact counts.
//   math   wave (wn, wm) owns the BN/2 x BM/2 quarter of the tile: (BN/32) x (BM/32) MFMA tiles, BK/32 k-steps a
//          stage.
// Tiles are numbered m-fastest under one weight tile, and each XCD takes a contiguous run of a product's tiles
// (see linear_kernel), so blocks sharing a weight tile share that XCD's L2.  A grouped launch runs up to 8
// independent products in one grid, each spread over all XCDs.
//
// Bound: the decode shapes (M = tokens of a step, tens) stream their weights once -- HBM.  The prefill shapes
// (M = thousands) are MFMA-bound at 2 M N K flop, except the absorb and un-absorb, whose outputs and inputs
// (268 + 134 MB at 4096 tokens) put their HBM time above their MFMA time.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int LN_THREADS = 256;
constexpr int LN_MAXGROUP = 8;  // products per grouped launch

// A stage holds BK of k for every tile row: CPR = BK / 8 chunks of 16 bytes.  Chunk c of row r sits at position
// c ^ ln_swz(r) of the row.  A fragment read takes one chunk of 16 consecutive rows; 16 / CPR consecutive rows
// fill the 256 bytes of the 64 banks once, and (r / (16 / CPR)) mod CPR gives each such group its own chunk
// positions: 16 distinct 16-byte bank groups (128-byte rows: (r >> 1) & 7; 64-byte rows: (r >> 2) & 3).
template <int CPR>
__device__ __forceinline__ int ln_swz(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}

// One product of a group as the kernels see it (host-filled; passed by value in the kernel arguments).
struct LinearProb {
  const bf16* A;
  const bf16* W;
  void* C;
  f32x4* part;  // split-K partial tiles (splits > 1)
  int64_t lda, sa, ldw, sw, ldc, sc;
  int M, N, K, c_bf16, tiles_m, tiles_n, splits, nk_per;
  float alpha;
  int block0;   // first block of this product in the product grid (a multiple of 8)
  int nblocks;  // its blocks (tiles x splits); the grid gives it nblocks rounded up to a multiple of 8
  int rblock0;  // first block of its split-K reduction in the reduce grid
};
struct LinearGroup {
  int n;
  LinearProb p[LN_MAXGROUP];
};

// product of a block: the last one whose first block is at or below it (n <= 8, a uniform scalar walk)
__device__ __forceinline__ int linear_find(const LinearGroup& g, int bid, bool reduce) {
  int i = 0;
  while (i + 1 < g.n && bid >= (reduce ? g.p[i + 1].rblock0 : g.p[i + 1].block0)) ++i;
  return i;
}

// store 4 consecutive outputs n .. n+3 of row m (those below N)
__device__ __forceinline__ void linear_store4(const LinearProb& P, int64_t off, int n, f32x4 v) {
  if (P.c_bf16) {
    bf16* dst = static_cast<bf16*>(P.C) + off;
    if (n + 3 < P.N) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < P.N) dst[i] = Elem<bf16>::from_f32(v[i]);
    }
  } else {
    float* dst = static_cast<float*>(P.C) + off;
    if (n + 3 < P.N) {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < P.N) dst[i] = v[i];
    }
  }
}

// NBUF stage buffers, AHEAD = NBUF - 1 stages in flight ahead of the one being multiplied
template <int BM, int BN, int BK, int NBUF>
__global__ __launch_bounds__(LN_THREADS) void linear_kernel(const LinearGroup grp) {
  constexpr int LN_NBUF = NBUF, LN_AHEAD = NBUF - 1;
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row and stage
  constexpr int RPI = 64 / CPR;              // tile rows per direct-load instruction (1 KiB)
  constexpr int LA = BM / (4 * RPI), LW = BN / (4 * RPI);  // direct-load instructions per wave per stage
  constexpr int TN = BN / 32, TM = BM / 32;  // MFMA tiles per wave along n and m
  constexpr int KS = BK / 32;                // MFMA k-steps per stage
  static_assert(LA >= 1 && LW >= 1 && KS >= 1, "tile shape");
  // one LDS array: the stage ring while the tile is multiplied, then the staging of its bf16 output
  __shared__ __align__(1024) bf16 smem[LN_NBUF * (BM + BN) * BK];
  bf16 (*sA)[BM * BK] = reinterpret_cast<bf16 (*)[BM * BK]>(smem);
  bf16 (*sW)[BN * BK] = reinterpret_cast<bf16 (*)[BN * BK]>(smem + LN_NBUF * BM * BK);
  static_assert(BM * BN <= LN_NBUF * (BM + BN) * BK, "the output tile fits the stage ring");

  // Each product owns an 8-aligned range of 8 k blocks (blocks are dealt to the 8 XCDs round-robin, so every
  // product spreads over all XCDs); inside it, slot j runs block (j mod 8) k + j / 8, so each XCD takes a
  // contiguous run of the product's tiles (m-fastest under one weight tile: shared in that XCD's L2).  Slots
  // past the product's blocks exit at once.
  const LinearProb& P = grp.p[linear_find(grp, blockIdx.x, false)];
  const int j = blockIdx.x - P.block0, per = (P.nblocks + 7) >> 3;
  int bid = (j & 7) * per + (j >> 3);
  if (bid >= P.nblocks) return;
  const int M = P.M, N = P.N, K = P.K, splits = P.splits, nk_per = P.nk_per, tiles_m = P.tiles_m;
  const int sp = bid % splits;  // k-split of this block
  bid /= splits;
  const int per_b = tiles_m * P.tiles_n;
  const int b = bid / per_b;
  const int t = bid - b * per_b;
  const int tn = t / tiles_m, tm = t - tn * tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const bf16* A = P.A + b * P.sa;
  const bf16* W = P.W + b * P.sw;
  const int64_t lda = P.lda, ldw = P.ldw;

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
    // stages s .. s+AHEAD-1 are in flight: wait for s, publish it; after the barrier every wave is past
    // multiply(s-1), so buffer (s+AHEAD) % NBUF = (s-1) % NBUF is free for stage s + AHEAD
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((LN_AHEAD - 1) * (LA + LW)));
    __syncthreads();
    issue(s + LN_AHEAD);
    multiply(s);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land in LDS after the block ends

  if (splits > 1) {
    // split K: store the fp32 partial tile in lane order, [tile][split][wave][n tile][m tile][lane]; the reduce
    // kernel adds the splits in order and writes the output
    f32x4* pt = P.part + (int64_t(bid) * splits + sp) * (4 * TN * TM * 64) + (wave * TN * TM) * 64 + lane;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int c = 0; c < TM; ++c) pt[(a * TM + c) * 64] = acc[a][c];
    return;
  }

  if (P.c_bf16 && P.ldc % 8 == 0 && P.sc % 8 == 0) {
    // bf16 output through LDS: chunk ch (16 bytes) of tile row r sits at position ch ^ (r mod CH), which spreads the
    // 16 rows of one fragment store over distinct bank groups (BN = 128; two rows per group at BN = 64); then the
    // rows are copied out as whole 16-byte chunks
    constexpr int CH = BN / 8;
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int cc = wn * (BN / 2) + 16 * a + 4 * g;
#pragma unroll
      for (int c = 0; c < TM; ++c) {
        const int r = wm * (BM / 2) + 16 * c + l16;
        const f32x4 v = acc[a][c] * P.alpha;
        *reinterpret_cast<uint2*>(smem + r * BN + 8 * ((cc >> 3) ^ (r & (CH - 1))) + (cc & 7)) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    __syncthreads();
    bf16* Cb = static_cast<bf16*>(P.C) + int64_t(b) * P.sc;
    for (int i = threadIdx.x; i < BM * CH; i += LN_THREADS) {
      const int r = i / CH, ch = i - r * CH;
      const int m = m0 + r, n = n0 + 8 * ch;
      if (m >= M || n >= N) continue;
      const bf16* src = smem + r * BN + 8 * (ch ^ (r & (CH - 1)));
      bf16* dst = Cb + int64_t(m) * P.ldc + n;
      if (n + 8 <= N) {
        *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
      } else {
        for (int e = 0; e < N - n; ++e) dst[e] = src[e];
      }
    }
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
      linear_store4(P, int64_t(b) * P.sc + int64_t(m) * P.ldc + n, n, acc[a][c] * P.alpha);
    }
  }
}

// Split-K reduction: one thread per 4 outputs (one lane's f32x4 of one MFMA tile of one wave); the partials of the
// splits are added in split order, scaled once and rounded once, and stored as the unsplit kernel stores them.
template <int BM, int BN>
__global__ __launch_bounds__(256) void linear_reduce_kernel(const LinearGroup grp) {
  constexpr int TN = BN / 32, TM = BM / 32, TILE = 4 * TN * TM * 64;
  const LinearProb& P = grp.p[linear_find(grp, blockIdx.x, true)];
  const int64_t e = int64_t(blockIdx.x - P.rblock0) * 256 + threadIdx.x;  // f32x4 index over the product's tiles
  const int64_t tile = e / TILE;
  const int r = int(e - tile * TILE);
  const int lane = r & 63, ac = (r >> 6) % (TN * TM), wave = (r >> 6) / (TN * TM);
  const int a = ac / TM, c = ac - a * TM;
  const int tiles_m = P.tiles_m, per_b = tiles_m * P.tiles_n, splits = P.splits;
  const int b = int(tile / per_b), t = int(tile - int64_t(b) * per_b);
  const int tn = t / tiles_m, tm = t - tn * tiles_m;
  const int wn = wave >> 1, wm = wave & 1, l16 = lane & 15, g = lane >> 4;
  const int n = tn * BN + wn * (BN / 2) + 16 * a + 4 * g;
  const int m = tm * BM + wm * (BM / 2) + 16 * c + l16;
  if (m >= P.M || n >= P.N) return;
  const f32x4* p = P.part + tile * splits * TILE + r;
  // eight loads in flight at a time, added in split order
  f32x4 v = p[0];
  for (int q = 1; q < splits; q += 8) {
    f32x4 t8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q + j < splits) t8[j] = p[int64_t(q + j) * TILE];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q + j < splits) v += t8[j];
  }
  linear_store4(P, int64_t(b) * P.sc + int64_t(m) * P.ldc + n, n, v * P.alpha);
}

// Tile shape for a call: a decode step (few rows) takes 64 x 64 tiles with 64-wide k stages in 3 buffers (48 KiB
// of LDS, three blocks per CU); more rows take 128 x 128 tiles with 64-wide k stages in 2 buffers (64 KiB, two
// blocks per CU).  Several blocks per CU hide each other's load latency, first loads and last stores.  Measured on
// the 4096-token projections: 4 buffers of 32-wide stages 598 us, 2 buffers of 32-wide stages 539 us, 2 buffers of
// 64-wide stages 415 us (with the LDS-staged output); the 64-token ones went 22.7 -> 21.4 us with 3 buffers.
struct LinearTile {
  int BM, BN, BK;
};
static LinearTile linear_tile(int M) { return M <= 64 ? LinearTile{64, 64, 64} : LinearTile{128, 128, 64}; }

// k-splits of a group's products, a pure function of the shapes.  The group's work is sum(tiles x stages); spread
// over two blocks per CU it gives the stages each block slot runs on average (at least 4).  A product whose blocks
// would run more than twice that is split down to about that many stages per block (the split-K reduction costs a
// launch, so a product is split only where it would otherwise be the long pole).
static void linear_splits(const LinearTile& t, const LinearLaunch* probs, int n, int cus, int* sp) {
  int64_t work = 0;
  for (int i = 0; i < n; ++i) {
    const LinearLaunch& a = probs[i];
    if (a.batch > 0 && a.M > 0 && a.N > 0)
      work += int64_t(a.batch) * ((a.M + t.BM - 1) / t.BM) * ((a.N + t.BN - 1) / t.BN) * (a.K / t.BK);
  }
  const int64_t slots = 2 * int64_t(cus);
  const int64_t avg = (work + slots - 1) / slots, load = avg > 4 ? avg : 4;
  for (int i = 0; i < n; ++i) {
    const int nk = probs[i].K / t.BK;
    sp[i] = 1;
    if (probs[i].batch <= 0 || probs[i].M <= 0 || probs[i].N <= 0 || nk <= 2 * load) continue;
    const int want = int((nk + load - 1) / load);
    const int s1 = max(1, min(want, nk / 4));  // at least 4 stages per split
    const int per = (nk + s1 - 1) / s1;
    sp[i] = (nk + per - 1) / per;  // every split non-empty
  }
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

template <int BM, int BN, int BK, int NBUF>
static kp_status launch_group(const LinearLaunch* probs, int n, void* ws, size_t ws_bytes, hipStream_t s) {
  const LinearTile tl{BM, BN, BK};
  int spl[LN_MAXGROUP];
  linear_splits(tl, probs, n, min(device_cus(), 256), spl);  // the workspace query assumes 256 CUs
  LinearGroup g{};
  int64_t blocks = 0, rblocks = 0;
  size_t ws_off = 0;
  bool ws_ok = true;
  for (int i = 0; i < n; ++i) {
    const LinearLaunch& a = probs[i];
    LinearProb& P = g.p[g.n];
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const int64_t tiles = int64_t(a.batch) * tiles_m * tiles_n;
    if (tiles == 0) continue;
    int sp = spl[i];
    if (sp > 1) {
      const size_t need = size_t(tiles) * sp * BM * BN * sizeof(float);
      if (ws && ws_ok && ws_off + need <= ws_bytes) {
        P.part = reinterpret_cast<f32x4*>(static_cast<char*>(ws) + ws_off);
        ws_off += need;
      } else {
        ws_ok = false;  // a workspace too small for this and later products: no split from here on
        sp = 1;
      }
    }
    P.A = static_cast<const bf16*>(a.A);
    P.W = static_cast<const bf16*>(a.W);
    P.C = a.C;
    P.lda = a.lda;
    P.sa = a.sa;
    P.ldw = a.ldw;
    P.sw = a.sw;
    P.ldc = a.ldc;
    P.sc = a.sc;
    P.M = a.M;
    P.N = a.N;
    P.K = a.K;
    P.c_bf16 = a.c_dtype == KP_DTYPE_BF16;
    P.tiles_m = tiles_m;
    P.tiles_n = tiles_n;
    P.splits = sp;
    P.nk_per = (a.K / BK + sp - 1) / sp;
    P.alpha = a.alpha;
    P.block0 = int(blocks);
    P.nblocks = int(tiles * sp);  // below 2^31: the grid check after the loop covers it
    P.rblock0 = int(rblocks);
    blocks += (tiles * sp + 7) / 8 * 8;
    if (sp > 1) rblocks += tiles * (BM * BN / 4) / 256;  // one thread per f32x4 of the partial tiles
    if (blocks > 0x7fffffff || rblocks > 0x7fffffff) {
      set_error("kp_linear: %lld blocks exceed the grid", (long long)blocks);
      return KP_ERR_INVALID_ARG;
    }
    ++g.n;
  }
  if (g.n == 0) return KP_OK;
  linear_kernel<BM, BN, BK, NBUF><<<dim3(unsigned(blocks)), dim3(LN_THREADS), 0, s>>>(g);
  if (rblocks > 0) {
    // a product without splits has no reduce blocks: its rblock0 equals the next one's, and linear_find (the last
    // product whose first block is at or below) passes over it
    linear_reduce_kernel<BM, BN><<<dim3(unsigned(rblocks)), dim3(256), 0, s>>>(g);
  }
  return check_launch("kp_linear");
}

size_t linear_group_workspace(const LinearLaunch* probs, int n) {
  int maxM = 0;
  for (int i = 0; i < n; ++i) maxM = max(maxM, probs[i].M);
  if (maxM == 0) return 0;
  const LinearTile t = linear_tile(maxM);
  int spl[LN_MAXGROUP];
  linear_splits(t, probs, n, 256, spl);
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    const LinearLaunch& a = probs[i];
    const int sp = spl[i];
    if (sp <= 1) continue;
    const int64_t tiles = int64_t(a.batch) * ((a.M + t.BM - 1) / t.BM) * ((a.N + t.BN - 1) / t.BN);
    total += size_t(tiles) * sp * t.BM * t.BN * sizeof(float);
  }
  return total;
}

kp_status launch_linear_group(const LinearLaunch* probs, int n, void* ws, size_t ws_bytes, hipStream_t s) {
  int maxM = 0;
  for (int i = 0; i < n; ++i) maxM = max(maxM, probs[i].M);
  if (maxM == 0) return KP_OK;
  // one tile shape for the whole group, chosen by its largest row count
  if (linear_tile(maxM).BM == 64) return launch_group<64, 64, 64, 3>(probs, n, ws, ws_bytes, s);
  return launch_group<128, 128, 64, 2>(probs, n, ws, ws_bytes, s);
}

}  // namespace kp
