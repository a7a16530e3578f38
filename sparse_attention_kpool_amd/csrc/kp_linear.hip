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
//          stage and the waits are exact counts.  No stage past the end of k is loaded (the last stages wait for
//          every load instead): at 4096 tokens the absorb, 4 stages a tile, ran 162 -> 153 us with it.
//   units  a block of an unsplit product with at least LN_REP_MIN tiles takes LN_REP tiles in turn, as one stream
//          of stages: the next tile's first stage loads while this tile's last one is multiplied and its output
//          leaves (4096-token un-absorb 133 -> 128 us; 4 tiles a block measured no better).
//   math   wave (wn, wm) owns the BN/2 x BM/2 quarter of the tile: (BN/32) x (BM/32) MFMA tiles, BK/32 k-steps a
//          stage.
// Tiles are numbered in panels of 8 m-tiles (m-fastest inside a panel, then n), and each XCD takes a contiguous
// run of a product's tiles (see linear_kernel): the blocks of one panel run together on one XCD, so an activation
// tile is fetched from HBM once for all the n-tiles that use it, and a weight tile once for the panel.  At 4096
// tokens this cut the absorb's HBM reads from 554 to about 150 MiB (m-fastest order re-read each activation tile
// once per n-tile) and the five prefill projections from 404 to 369 us.  A grouped launch runs up to 8
// independent products in one grid, each spread over all XCDs.
//
// Bound: the decode shapes (M = tokens of a step, tens) stream their weights once -- HBM.  The prefill shapes
// (M = thousands) are MFMA-bound at 2 M N K flop, except the absorb and un-absorb, whose outputs and inputs
// (268 + 134 MB at 4096 tokens) put their HBM time above their MFMA time: at prefill sizes those two run in the
// weight-stationary kernel further down instead of these tiles.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int LN_THREADS = 256;
constexpr int LN_REP = 2;              // units per block of an unsplit product of many short tiles ...
constexpr int64_t LN_REP_MIN = 2048;   // ... of at least this many tiles
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
  int nblocks;  // its units (tiles x splits), in 8 runs of (nblocks + 7) / 8, one run per XCD
  int rep;      // units per block at most: the grid gives it 8 * ceil(run / rep) blocks
  int rblock0;  // first block of its split-K reduction in the reduce grid
};
struct LinearGroup {
  int n;
  LinearProb p[LN_MAXGROUP];
};

// Output tile t of one batch entry: panels of LN_GM m-tiles (the last one may be narrower), m-fastest inside a
// panel, then n, panels in m order.
constexpr int LN_GM = 8;
__device__ __forceinline__ void linear_tile_at(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int base = t / (LN_GM * tiles_n) * LN_GM;
  const int gm = min(LN_GM, tiles_m - base);
  const int r = t - base * tiles_n;
  tn = r / gm;
  tm = base + (r - tn * gm);
}

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
  constexpr bool LN_STAGE_ONE = BM * BN <= (BM + BN) * BK;  // the output tile fits one stage buffer

  // Each product owns an 8-aligned range of 8 k blocks (blocks are dealt to the 8 XCDs round-robin, so every
  // product spreads over all XCDs); inside it, slot j runs units (tile, k-split) of run (j mod 8), the
  // contiguous run of the product's units (in panel order) that this XCD takes: units j / 8, j / 8 + k,
  // j / 8 + 2k, ... (rep of them at most), so the blocks of one XCD always work on neighbouring units and shared
  // operand tiles stay in its L2.  Slots past the run's units exit at once.
  const LinearProb& P = grp.p[linear_find(grp, blockIdx.x, false)];
  const int j = blockIdx.x - P.block0, per = (P.nblocks + 7) >> 3;
  const int rep = P.rep, nq = (per + rep - 1) / rep;  // units per block at most; blocks per XCD run
  const int x = j & 7, q = j >> 3;
  const int run_len = min(per, P.nblocks - x * per);
  if (q >= run_len) return;
  const int n_units = min(rep, (run_len - q + nq - 1) / nq);
  const int M = P.M, N = P.N, K = P.K, splits = P.splits, nk_per = P.nk_per, tiles_m = P.tiles_m;
  const int64_t lda = P.lda, ldw = P.ldw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;

  // One unit: its batch entry, k-split, tile origin, stages [s0, s0 + nk) of the K / BK, and each load
  // instruction's per-lane source at k = 0: row RPI (wave * L + i) + lane / CPR of the tile, the chunk whose
  // swizzled position is lane % CPR
  struct Unit {
    int b, sp, m0, n0, s0, nk;
    const bf16* srcA[LA];
    const bf16* srcW[LW];
  };
  auto setup = [&](int i, Unit& U) __attribute__((always_inline)) {
    int bid = x * per + q + i * nq;
    U.sp = bid % splits;
    bid /= splits;
    const int per_b = tiles_m * P.tiles_n;
    U.b = bid / per_b;
    int tm, tn;
    linear_tile_at(bid - U.b * per_b, tiles_m, P.tiles_n, tm, tn);
    U.m0 = tm * BM;
    U.n0 = tn * BN;
    const bf16* A = P.A + U.b * P.sa;
    const bf16* W = P.W + U.b * P.sw;
#pragma unroll
    for (int l = 0; l < LA; ++l) {
      const int r = RPI * (wave * LA + l) + lane / CPR;
      U.srcA[l] = A + int64_t(min(U.m0 + r, M - 1)) * lda + 8 * ((lane % CPR) ^ ln_swz<CPR>(r));
    }
#pragma unroll
    for (int l = 0; l < LW; ++l) {
      const int r = RPI * (wave * LW + l) + lane / CPR;
      U.srcW[l] = W + int64_t(min(U.n0 + r, N - 1)) * ldw + 8 * ((lane % CPR) ^ ln_swz<CPR>(r));
    }
    U.s0 = U.sp * nk_per;
    U.nk = min(nk_per, K / BK - U.s0);
  };
  // stage s (below U.nk) of unit U into buffer buf: LA + LW loads per wave
  auto issue = [&](const Unit& U, int s, int buf) __attribute__((always_inline)) {
    const int64_t k0 = int64_t(U.s0 + s) * BK;
    const uint32_t ba = lds_off(sA[buf]), bw = lds_off(sW[buf]);
#pragma unroll
    for (int l = 0; l < LA; ++l) lds_dma16(U.srcA[l] + k0, ba + uint32_t(1024 * (wave * LA + l)));
#pragma unroll
    for (int l = 0; l < LW; ++l) lds_dma16(U.srcW[l] + k0, bw + uint32_t(1024 * (wave * LW + l)));
  };

  // fragment rows of this wave: weight rows wn * BN/2 + 16 a + l16, activation rows wm * BM/2 + 16 c + l16; the
  // swizzle of a row depends on l16 only (tile rows are 16-aligned), so each read is a per-lane base plus a
  // constant, XOR a per-lane chunk position
  const int wn = wave >> 1, wm = wave & 1;
  const int sw_l = ln_swz<CPR>(l16);
  f32x4 acc[TN][TM];
  auto multiply = [&](int buf) __attribute__((always_inline)) {
    const uint32_t ba = lds_off(sA[buf]), bw = lds_off(sW[buf]);
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

  // The stages of the block's units form one stream: stage s of unit u is stream stage G = u nk + s, in buffer
  // G % NBUF (a block takes several units only of an unsplit product whose nk >= NBUF, so every unit has the same
  // nk and the next unit's first stages are loaded while this unit's last ones are multiplied and its output
  // leaves).  The bf16 output is staged in the buffer of the unit's last stage, which no load in flight targets.
  Unit cur, nxt;
  setup(0, cur);
  const int nk = cur.nk, total = n_units * nk;
#pragma unroll
  for (int s = 0; s < LN_AHEAD; ++s)
    if (s < nk) issue(cur, s, s);
  for (int u = 0; u < n_units; ++u) {
    const bool has_next = u + 1 < n_units;
    if (has_next) setup(u + 1, nxt);
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int c = 0; c < TM; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nk; ++s) {
      // stream stages G .. min(G + AHEAD, total) - 1 are in flight (and, after a unit's first stages, its
      // predecessor's output stores, which are younger and only make the wait longer): wait for G -- the last
      // AHEAD - 1 stages of the stream wait for every load; with AHEAD <= 2 that is exact -- and publish it.
      // After the barrier every wave is past multiply(G-1) and past the previous unit's output staging, so
      // buffer (G + AHEAD) % NBUF = (G - 1) % NBUF is free for stream stage G + AHEAD.
      const int G = u * nk + s;
      if (G + LN_AHEAD - 1 < total)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((LN_AHEAD - 1) * (LA + LW)));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      if (s + LN_AHEAD < nk) issue(cur, s + LN_AHEAD, (G + LN_AHEAD) % LN_NBUF);
      else if (has_next) issue(nxt, s + LN_AHEAD - nk, (G + LN_AHEAD) % LN_NBUF);
      multiply(G % LN_NBUF);
    }
    const int last = (u * nk + nk - 1) % LN_NBUF;  // buffer of the unit's last stage

    if (splits > 1) {
      // split K: store the fp32 partial tile in lane order, [tile][split][wave][n tile][m tile][lane]; the reduce
      // kernel adds the splits in order and writes the output
      const int64_t tile = (int64_t(x * per + q + u * nq)) / splits;
      f32x4* pt = P.part + (tile * splits + cur.sp) * (4 * TN * TM * 64) + (wave * TN * TM) * 64 + lane;
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int c = 0; c < TM; ++c) pt[(a * TM + c) * 64] = acc[a][c];
    } else if (P.c_bf16 && P.ldc % 8 == 0 && P.sc % 8 == 0) {
      // bf16 output through LDS, in the last stage's buffer (rows 0 .. BM*BK/BN - 1 in its activation part, the
      // rest in its weight part): chunk ch (16 bytes) of tile row r sits at position ch ^ (r mod CH), which
      // spreads the 16 rows of one fragment store over distinct bank groups (BN = 128; two rows per group at
      // BN = 64); then the rows are copied out as whole 16-byte chunks
      constexpr int CH = BN / 8;
      constexpr int RA = BM * BK / BN;  // output rows held in the activation part
      static_assert((BM * BK) % BN == 0, "output rows do not straddle a stage buffer's parts");
      auto srow = [&](int r) __attribute__((always_inline)) -> bf16* {
        // a tile too large for one stage buffer takes the whole ring (one unit per block: no load in flight)
        if constexpr (!LN_STAGE_ONE) return smem + r * BN;
        return r < RA ? sA[last] + r * BN : sW[last] + (r - RA) * BN;
      };
      __syncthreads();  // every wave is done with the last stage's buffer
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int cc = wn * (BN / 2) + 16 * a + 4 * g;
#pragma unroll
        for (int c = 0; c < TM; ++c) {
          const int r = wm * (BM / 2) + 16 * c + l16;
          const f32x4 v = acc[a][c] * P.alpha;
          *reinterpret_cast<uint2*>(srow(r) + 8 * ((cc >> 3) ^ (r & (CH - 1))) + (cc & 7)) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
      __syncthreads();
      bf16* Cb = static_cast<bf16*>(P.C) + int64_t(cur.b) * P.sc;
      for (int i = threadIdx.x; i < BM * CH; i += LN_THREADS) {
        const int r = i / CH, ch = i - r * CH;
        const int m = cur.m0 + r, n = cur.n0 + 8 * ch;
        if (m >= M || n >= N) continue;
        const bf16* src = srow(r) + 8 * (ch ^ (r & (CH - 1)));
        bf16* dst = Cb + int64_t(m) * P.ldc + n;
        if (n + 8 <= N) {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        } else {
          for (int e = 0; e < N - n; ++e) dst[e] = src[e];
        }
      }
    } else {
      // lane holds D[n][m] for n = tile n + 4 g .. +3, m = tile m + l16
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int n = cur.n0 + wn * (BN / 2) + 16 * a + 4 * g;
#pragma unroll
        for (int c = 0; c < TM; ++c) {
          const int m = cur.m0 + wm * (BM / 2) + 16 * c + l16;
          if (m >= M || n >= N) continue;
          linear_store4(P, int64_t(cur.b) * P.sc + int64_t(m) * P.ldc + n, n, acc[a][c] * P.alpha);
        }
      }
    }
    if (has_next) cur = nxt;
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land in LDS after the block ends
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
  int tm, tn;
  linear_tile_at(t, tiles_m, P.tiles_n, tm, tn);
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
// would run more than twice that (decode tiles) or more than that (prefill tiles) is split down to about that many
// stages per block (the split-K reduction costs a launch, so a product is split only where it would otherwise be
// the long pole).  At 4096 tokens the head-weight, key and gate products (64 stages a block beside the index
// query's 24) then split in two: the grouped indexer products 210 -> 192 us; the same rule at 64 tokens made the
// decode group slower (20.7 -> 24.8 us), so decode tiles keep twice the average.
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
    if (probs[i].batch <= 0 || probs[i].M <= 0 || probs[i].N <= 0 || nk <= (t.BM >= 128 ? load : 2 * load)) continue;
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
  int64_t nb[LN_MAXGROUP], nrb[LN_MAXGROUP];  // each product's blocks and reduce blocks
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
    P.nblocks = int(tiles * sp);  // below 2^31: the grid check after the loop covers it
    // several units per block for an unsplit product of many short tiles (the next unit's first stages load
    // while this one's output leaves); every unit then has the same K / BK >= NBUF stages
    P.rep = (sp == 1 && a.K / BK >= NBUF && tiles >= LN_REP_MIN && BM * BN <= (BM + BN) * BK) ? LN_REP : 1;
    const int64_t run = (tiles * sp + 7) / 8;
    nb[g.n] = 8 * ((run + P.rep - 1) / P.rep);
    nrb[g.n] = sp > 1 ? tiles * (BM * BN / 4) / 256 : 0;  // one thread per f32x4 of the partial tiles
    blocks += nb[g.n];
    rblocks += nrb[g.n];
    if (blocks > 0x7fffffff || rblocks > 0x7fffffff) {
      set_error("kp_linear: %lld blocks exceed the grid", (long long)blocks);
      return KP_ERR_INVALID_ARG;
    }
    ++g.n;
  }
  if (g.n == 0) return KP_OK;
  // Grid layout, longest blocks first: blocks are dispatched in index order, so the block ranges go in descending
  // order of the stages one block runs (a stable order; workspace was given out above in the caller's order).  A
  // product of few long-K blocks placed after one of many short ones would start only once those were all
  // dispatched and end last (at 4096 tokens the head-weight, key and gate blocks, 32 stages each, now go before
  // the index query's 24-stage ones: the grouped indexer products about 94 -> 89 us).
  {
    int order[LN_MAXGROUP];
    for (int i = 0; i < g.n; ++i) order[i] = i;
    auto len = [&](int i) { return int64_t(g.p[i].nk_per) * g.p[i].rep; };
    for (int i = 1; i < g.n; ++i)
      for (int j = i; j > 0 && len(order[j]) > len(order[j - 1]); --j) {
        const int x = order[j];
        order[j] = order[j - 1];
        order[j - 1] = x;
      }
    LinearGroup h = g;
    int64_t b0 = 0, r0 = 0;
    for (int i = 0; i < g.n; ++i) {
      h.p[i] = g.p[order[i]];
      h.p[i].block0 = int(b0);
      h.p[i].rblock0 = int(r0);
      b0 += nb[order[i]];
      r0 += nrb[order[i]];
    }
    g = h;
  }
  linear_kernel<BM, BN, BK, NBUF><<<dim3(unsigned(blocks)), dim3(LN_THREADS), 0, s>>>(g);
  if (rblocks > 0) {
    // a product without splits has no reduce blocks: its rblock0 equals the next one's, and linear_find (the last
    // product whose first block is at or below) passes over it
    linear_reduce_kernel<BM, BN><<<dim3(unsigned(rblocks)), dim3(256), 0, s>>>(g);
  }
  return check_launch("kp_linear");
}

static bool linear_ws_shape(const LinearLaunch& a, int& nt, int& ks, int& mt);

size_t linear_group_workspace(const LinearLaunch* probs_in, int n_in) {
  // the weight-stationary products never split; the rest are sized as the tiled launch will run them
  LinearLaunch rest[LN_MAXGROUP];
  int n = 0;
  for (int i = 0; i < n_in && i < LN_MAXGROUP; ++i) {
    int nt, ks, mt;
    if (!linear_ws_shape(probs_in[i], nt, ks, mt)) rest[n++] = probs_in[i];
  }
  const LinearLaunch* probs = rest;
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

// ---------------------------------------------------------------------------------------------------------------
// Weight-stationary head products.  The absorb (N = 512, K = 256) and the un-absorb (N = 256, K = 512) of a
// prefill chunk are batches over heads whose one entry's weight is only 256 KiB, while M is thousands of tokens.
// Output-stationary tiles re-fetch a weight tile and an activation tile for every 128 x 128 outputs (128 KiB of
// operands through L2 and LDS for 32 KiB of output at K = 256), which paced these two products well above their
// HBM time.  Here one block of 8 waves owns one batch entry over a range of tokens: each wave holds its N / 8
// output columns' weight rows in registers for the whole block (N K / 1024 VGPRs: 128 for both shapes), the
// tokens stream through LDS in slabs of 16 MT rows (direct global->LDS loads, a ring of three, two slabs ahead,
// rows XOR-swizzled as in the tiled kernel), and each slab's output leaves straight from the MFMA lanes (4
// consecutive columns of one row a lane).  Per slab a block reads 16 MT K bf16 and writes 16 MT N outputs, which
// is all the HBM traffic there is besides one read of the weight per block.
//   math   D^T[n][m] = W . A^T on 16x16x32 bf16 MFMA: weight rows are the M operand (in registers), activation
//          rows the N operand (one 16-byte LDS read per lane per m-tile and k-step, shared by the wave's NT
//          n-tiles).
//   stores raw buffer stores through a resource bounded at M rows, so rows past M (the last slab of a block) are
//          dropped by the hardware and every lane issues the same stores: the waits below are exact counts.
// Slots past the end: a block whose token range is empty exits; a slab index past the block's last one re-reads
// the last slab (never multiplied), so each iteration issues the same loads.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // an 8-byte store's payload
constexpr int LWS_WAVES = 8;
constexpr int LWS_THREADS = 64 * LWS_WAVES;
constexpr int LWS_NBUF = 3;

template <int NT, int KS, int MT, bool OB>
__global__ __launch_bounds__(LWS_THREADS) void linear_ws_kernel(const LinearProb P, int batch, int mblocks,
                                                                int slabs_per_block) {
  constexpr int K = 32 * KS, CPR = K / 8;  // 16-byte chunks per activation row
  constexpr int MS = 16 * MT;              // tokens per slab
  constexpr int SLAB = MS * K;             // bf16 per slab
  constexpr int L = SLAB * 2 / (1024 * LWS_WAVES);  // direct-load instructions per wave per slab
  constexpr int ESZ = OB ? 2 : 4;                   // output element bytes
  constexpr int ROWB = 128 * NT * ESZ;              // bytes of one output row (N = 8 waves x 16 NT columns)
  constexpr int CR = ROWB / 16;                     // 16-byte chunks per output row
  constexpr int OUTB = MS * ROWB;                   // bytes of a slab's output
  constexpr int S = OUTB / (1024 * LWS_WAVES);      // 1 KiB output stores per wave per slab
  static_assert(L >= 1 && (SLAB * 2) % (1024 * LWS_WAVES) == 0, "a slab is a whole number of block-wide loads");
  static_assert(S >= 1 && OUTB % (1024 * LWS_WAVES) == 0, "a slab's output is a whole number of block-wide stores");
  static_assert(CPR >= 16 && CPR % 16 == 0 && CR >= 16 && CR % 16 == 0, "the row swizzles need 16 chunk positions");
  __shared__ __align__(1024) bf16 ring[LWS_NBUF][SLAB];
  __shared__ __align__(1024) char stage[OUTB];  // a slab's output rows, chunk c of row r at position c ^ (r mod 16)

  // blocks are dealt to the 8 XCDs round-robin; XCD x takes the contiguous run [x per, (x + 1) per) of block
  // slots, so the token ranges of one batch entry (which share its weight) run on one XCD
  const int per = int(gridDim.x >> 3);
  const int t = int(blockIdx.x & 7) * per + int(blockIdx.x >> 3);
  const int b = t / mblocks, mb = t - b * mblocks;
  const int M = P.M;
  const int m_begin = mb * slabs_per_block * MS;
  if (b >= batch || m_begin >= M) return;  // uniform over the block
  const int nslab = min(slabs_per_block, (M - m_begin + MS - 1) / MS);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int l16 = lane & 15, g = lane >> 4;

  // slab loads: wave instruction i fills LDS chunk positions 64 (wave L + i) + lane, i.e. row r, position p; the
  // chunk stored there is c = p ^ (r mod 16) of that row
  const bf16* A = P.A + int64_t(b) * P.sa;
  int lrow[L], lcol[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int q = 64 * (wave * L + i) + lane;
    lrow[i] = q / CPR;
    lcol[i] = 8 * ((q % CPR) ^ (lrow[i] & 15));
  }
  auto issue = [&](int s, int buf) __attribute__((always_inline)) {
    const int m0 = m_begin + min(s, nslab - 1) * MS;
    const uint32_t base = lds_off(ring[buf]);
#pragma unroll
    for (int i = 0; i < L; ++i)
      lds_dma16(A + int64_t(min(m0 + lrow[i], M - 1)) * P.lda + lcol[i], base + uint32_t(1024 * (wave * L + i)));
  };
  issue(0, 0);
  issue(1, 1);

  // this wave's weight rows n_w + 16 a + l16, k chunk 4 ks + g, for the whole block
  const int n_w = wave * 16 * NT;
  const bf16* W = P.W + int64_t(b) * P.sw;
  bf16x8 wf[NT][KS];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      wf[a][ks] = *reinterpret_cast<const bf16x8*>(W + int64_t(n_w + 16 * a + l16) * P.ldw + 8 * (4 * ks + g));
  // the weight is waited for here, once, and not inside the slab loop (this wait also covers slabs 0 and 1)
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(wf[a][ks]));

  // output rows of one batch entry through a buffer resource bounded at M rows
  const uint64_t cb = reinterpret_cast<uint64_t>(static_cast<char*>(P.C) + int64_t(b) * P.sc * ESZ);
  const uint64_t cb_u = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(cb >> 32)))) << 32) |
                        uint32_t(__builtin_amdgcn_readfirstlane(int(cb)));
  const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(cb_u), 0, __builtin_amdgcn_readfirstlane(int(int64_t(M) * P.ldc * ESZ)), 0x00020000);
  const float alpha = P.alpha;
  const uint32_t st = lds_off(stage);

  for (int s = 0; s < nslab; ++s) {
    // issue order: slab loads (L a wave) then the slab's stores (S a wave) each iteration, after slabs 0 and 1
    // up front; vector-memory operations complete in issue order, so slab s has landed once at most the ops
    // issued after it are outstanding: slab 1 (s = 0); slab 2 and stores 0 (s = 1); stores s-2, slab s+1 and
    // stores s-1 (s >= 2)
    if (s == 0)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
    else if (s == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(L + S));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(L + 2 * S));
    // slab s is visible to every wave; every wave is done with slab s - 1's buffer and its staged output
    __syncthreads();
    issue(s + 2, (s + 2) % LWS_NBUF);
    const uint32_t base = lds_off(ring[s % LWS_NBUF]);
    f32x4 acc[NT][MT];
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int c = 0; c < MT; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // activation fragments one k-step ahead of the MFMAs that use them
    bf16x8 fa[2][MT];
    auto read_fa = [&](int ks, bf16x8(&f)[MT]) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < MT; ++c) f[c] = lds_load<bf16x8>(base + (16 * c + l16) * (2 * K) + 16 * ((4 * ks + g) ^ l16));
    };
    read_fa(0, fa[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) read_fa(ks + 1, fa[(ks + 1) & 1]);
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int c = 0; c < MT; ++c) acc[a][c] = mfma16(wf[a][ks], fa[ks & 1][c], acc[a][c]);
    }
    // lane holds D^T[n][m] for n = n_w + 16 a + 4 g .. +3 and m = slab row 16 c + l16: staged, then the slab's
    // rows leave as whole 1 KiB wave stores
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int c = 0; c < MT; ++c) {
        const f32x4 v = acc[a][c] * alpha;
        const int r = 16 * c + l16, nb = (n_w + 16 * a + 4 * g) * ESZ;
        const uint32_t at = st + uint32_t(r * ROWB + 16 * ((nb >> 4) ^ (r & 15)) + (nb & 15));
        if constexpr (OB)
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(uintptr_t(at)) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        else
          *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(uintptr_t(at)) = v;
      }
    __syncthreads();
    const int m0 = m_begin + s * MS;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int q = 64 * (wave * S + i) + lane, r = q / CR, cl = q % CR;
      const u32x4 v = lds_load<u32x4>(st + uint32_t(r * ROWB + 16 * (cl ^ (r & 15))));
      __builtin_amdgcn_raw_buffer_store_b128(v, dst, int(int64_t(m0 + r) * P.ldc * ESZ + 16 * cl), 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land in LDS after the block ends
}

// The shapes the weight-stationary kernel takes: the two head-product shapes with a prefill's token count, 16-byte
// aligned operands, and row offsets that fit its 32-bit store offsets.
static bool linear_ws_shape(const LinearLaunch& a, int& nt, int& ks, int& mt) {
  if (a.N == 512 && a.K == 256) {
    nt = 4, ks = 8, mt = 2;
  } else if (a.N == 256 && a.K == 512) {
    nt = 2, ks = 16, mt = 2;
  } else {
    return false;
  }
  const int esz = a.c_dtype == KP_DTYPE_BF16 ? 2 : 4;
  const auto al = [](const void* p, int n) { return (reinterpret_cast<uintptr_t>(p) & uintptr_t(n - 1)) == 0; };
  return a.batch >= 8 && a.M >= 512 && al(a.A, 16) && al(a.W, 16) && al(a.C, 16) && a.lda % 8 == 0 &&
         a.sa % 8 == 0 && a.ldw % 8 == 0 && a.sw % 8 == 0 && (a.ldc * esz) % 16 == 0 && (a.sc * esz) % 16 == 0 &&
         (int64_t(a.M) + 64) * a.ldc * esz < (int64_t(1) << 31);
}

static kp_status launch_linear_ws(const LinearLaunch& a, hipStream_t s) {
  int nt = 0, ks = 0, mt = 0;
  linear_ws_shape(a, nt, ks, mt);
  const int ms = 16 * mt;
  const int cus = device_cus();
  // about one block per CU: the token ranges of a batch entry split its rows into whole slabs
  const int mblocks = max(1, min((a.M + ms - 1) / ms, (cus + a.batch - 1) / a.batch));
  const int slabs = ((a.M + ms - 1) / ms + mblocks - 1) / mblocks;
  const int64_t blocks = (int64_t(a.batch) * mblocks + 7) / 8 * 8;
  if (blocks > 0x7fffffff) {
    set_error("kp_linear: %lld blocks exceed the grid", (long long)blocks);
    return KP_ERR_INVALID_ARG;
  }
  LinearProb P{};
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
  P.alpha = a.alpha;
  const dim3 grid{unsigned(blocks)}, blk{unsigned(LWS_THREADS)};
  if (nt == 4 && P.c_bf16)
    linear_ws_kernel<4, 8, 2, true><<<grid, blk, 0, s>>>(P, a.batch, mblocks, slabs);
  else if (nt == 4)
    linear_ws_kernel<4, 8, 2, false><<<grid, blk, 0, s>>>(P, a.batch, mblocks, slabs);
  else if (P.c_bf16)
    linear_ws_kernel<2, 16, 2, true><<<grid, blk, 0, s>>>(P, a.batch, mblocks, slabs);
  else
    linear_ws_kernel<2, 16, 2, false><<<grid, blk, 0, s>>>(P, a.batch, mblocks, slabs);
  return check_launch("kp_linear");
}

kp_status launch_linear_group(const LinearLaunch* probs_in, int n_in, void* ws, size_t ws_bytes, hipStream_t s) {
  // products of the weight-stationary shapes take a launch of their own; the rest share the tiled launch, which
  // goes first: its grid check is the last check that can fail, so an error leaves nothing enqueued (a
  // weight-stationary grid, at most batch + one block per CU rounded to 8, always fits)
  LinearLaunch rest[LN_MAXGROUP];
  int n = 0, ws_idx[LN_MAXGROUP], n_ws = 0;
  for (int i = 0; i < n_in; ++i) {
    int nt, ks, mt;
    if (linear_ws_shape(probs_in[i], nt, ks, mt)) ws_idx[n_ws++] = i;
    else rest[n++] = probs_in[i];
  }
  int maxM = 0;
  for (int i = 0; i < n; ++i) maxM = max(maxM, rest[i].M);
  if (maxM > 0) {
    // one tile shape for the whole group, chosen by its largest row count
    const kp_status st = linear_tile(maxM).BM == 64 ? launch_group<64, 64, 64, 3>(rest, n, ws, ws_bytes, s)
                                                    : launch_group<128, 128, 64, 2>(rest, n, ws, ws_bytes, s);
    if (st != KP_OK) return st;
  }
  for (int i = 0; i < n_ws; ++i) {
    const kp_status st = launch_linear_ws(probs_in[ws_idx[i]], s);
    if (st != KP_OK) return st;
  }
  return KP_OK;
}

}  // namespace kp
