// dsa_indexer_score: scores[q, p] = sum_h w[q, h] * ReLU(q_idx[q, h, :] . pooled[seq(q), p, :]), p < n_c(q).
//
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: the indexer scores pools
// of 4 tokens.  [GLM-5.3-Flash model card, "Raw config fields"]: 32 index heads of dim 128.  The weighted ReLU
// sum is the layer specification's definition.
//
// Mapping onto the matrix cores: for one query, [32 heads x D] . [D x 32 pools] is one 32x32 MFMA tile
// (32x32x16 bf16, or 32x32x2 f32), the index heads forming M.  Lane group g of the 32x32 layout carries the
// channels [g*D/2, (g+1)*D/2).  The epilogue stays in registers: each lane holds 16 heads of one pool, weights
// them with ReLU, sums in-lane, then adds its partner lane (l ^ 32).
//
// Data path: pooled keys stream in tiles loaded with fully coalesced 16-byte loads (a wave instruction covers
// 1 KiB of consecutive pooled rows; the pools of one page are contiguous) and read back from LDS in the MFMA
// operand layout.  Page ids are looked up once per block (never in the tile loop), so no key load waits on
// another global load.
//
// Two kernels:
//   decode   a persistent grid (two 4-wave blocks per compute unit): the 32-pool tiles of all queries are split
//            into one contiguous range per wave of about equal length; a wave streams its range query by query
//            through a private LDS tile (tiles kept two ahead in registers), with no block-wide barrier.
//   prefill  16 consecutive queries per block that the caller says share a sequence (a prefill chunk); each
//            64-pool tile goes straight from global memory into LDS (no register staging), four tiles in
//            flight, and is computed by all 8 waves for 2 queries each.  If the queries turn out to belong to
//            different sequences, the block handles one sequence at a time, so results never depend on that
//            promise.
//
// Bound: decode is HBM-bound (the pooled-key stream, 256 B per pool at D = 128 bf16 for 32 x 128 MACs, i.e.
// 32 flop/B: above the VALU ridge, so the contraction runs on MFMA); prefill is MFMA-bound.
#include <type_traits>

#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

template <class T, int D>
struct ScoreShape {
  static constexpr int KPL = Elem<T>::kpl;
  static constexpr int STEPS = D / (2 * KPL);          // 32x32 k-steps over D
  static constexpr int EPC = 16 / int(sizeof(T));      // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                  // chunks per pooled row
  static constexpr int RS = D + EPC;                   // LDS row stride (elements): +16 B against conflicts
  static constexpr int TCH = 32 * CPR;                 // 16-byte chunks per 32-pool tile
};

// Index-query fragments (A operand) and head weights of one query, in the 32x32 layout.
template <class T, int D>
__device__ __forceinline__ void score_query_frags(const T* __restrict__ q_idx, const float* __restrict__ w, int row,
                                                  bool rv, int Hi, int n, int g,
                                                  typename Elem<T>::frag (&qa)[ScoreShape<T, D>::STEPS],
                                                  float (&wv)[16]) {
  using S = ScoreShape<T, D>;
  using E = Elem<T>;
  const bool hv = (n < Hi) && rv;
  const T* qp = q_idx + (int64_t(rv ? row : 0) * Hi + (hv ? n : 0)) * D + g * (D / 2);
#pragma unroll
  for (int s = 0; s < S::STEPS; ++s) qa[s] = hv ? E::frag_load(qp + s * S::KPL) : E::frag_zero();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = 8 * (i / 4) + 4 * g + (i % 4);
    wv[i] = (h < Hi && rv) ? w[int64_t(row) * Hi + h] : 0.f;
  }
}

// ReLU-weighted head sums of one 32-pool tile for QW queries; lanes 0..31 get the scores of pools 0..31.  The
// queries' MFMA chains are interleaved k-step by k-step, so QW independent accumulations are in flight.
template <class T, int D, int QW>
__device__ __forceinline__ void score_mma(const typename Elem<T>::frag (&qa)[QW][ScoreShape<T, D>::STEPS],
                                          const typename Elem<T>::frag (&kb)[ScoreShape<T, D>::STEPS],
                                          f32x16 (&acc)[QW]) {
#pragma unroll
  for (int r = 0; r < QW; ++r) acc[r] = f32x16{};
#pragma unroll
  for (int s = 0; s < ScoreShape<T, D>::STEPS; ++s)
#pragma unroll
    for (int r = 0; r < QW; ++r) acc[r] = mfma32(qa[r][s], kb[s], acc[r]);
}

template <int QW>
__device__ __forceinline__ void score_reduce(const f32x16 (&acc)[QW], const float (&wv)[QW][16], float (&sc)[QW]) {
  // ReLU as an integer max on the bits: a negative float (and -0) has the sign bit set, i.e. is a negative
  // int32, so max(bits, 0) gives +0 for it and leaves a positive float unchanged -- one instruction, where
  // fmaxf needs a NaN-quieting step first.  (The element is copied to a scalar before the bit cast: a bit cast
  // applied to a vector element expression directly reads element 0.)
#pragma unroll
  for (int r = 0; r < QW; ++r) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float s = acc[r][i];
      part += wv[r][i] * __builtin_bit_cast(float, max(__builtin_bit_cast(int, s), 0));
    }
    // partner lane l ^ 32 holds the other 16 heads of the same pool.  v_permlane32_swap(x, y) swaps the upper
    // half of x with the lower half of y, returning [x lanes 0..31, y lanes 0..31] and [x lanes 32..63,
    // y lanes 32..63]; with x = part their sum in lanes 0..31 (the lanes that keep the score) is
    // part[l] + part[l + 32] -- one VALU op instead of an LDS permute.  y is a separate zero: the instruction
    // rewrites both of its registers, so x and y must not be the same register.
    // (The results are copied to scalars before the bit casts, which read element 0 of a vector element
    // expression.)
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, part), 0u, false, false);
    const uint32_t lo = sw[0], hi = sw[1];
    sc[r] = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
  }
}

template <class T, int D, int QW>
__device__ __forceinline__ void score_tiles(const typename Elem<T>::frag (&qa)[QW][ScoreShape<T, D>::STEPS],
                                            const typename Elem<T>::frag (&kb)[ScoreShape<T, D>::STEPS],
                                            const float (&wv)[QW][16], float (&sc)[QW]) {
  f32x16 acc[QW];
  score_mma<T, D, QW>(qa, kb, acc);
  score_reduce<QW>(acc, wv, sc);
}

constexpr int SC_MAXCHUNK = 4096;    // decode: scores buffered in LDS per block (SC_MAXCHUNK / 4 per wave)
constexpr int SC_DBLOCKS_PER_CU = 2;  // decode: persistent blocks of 4 waves per compute unit
constexpr int SC_MAXPEND = 64;        // decode: pools pooled in the scoring launch (one per lane)

// The persistent decode grids split the TILE-pool tiles of all queries, taken query by query, into one contiguous
// range per wave of about equal length, so rows of any length mix keep every wave streaming.  Wave gw of n_waves
// gets `left` tiles starting at tile tc of query qc; false when its range is empty.  seq0 is q_seq of query `lane`
// (lanes below n_q; queries past 64 read q_seq themselves).  With at most 64 queries, one wave scan (one query per
// lane) gives both the total and the cursor; more queries take a second pass.
template <int TILE>
__device__ __forceinline__ bool decode_wave_range(const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
                                                  int n_q, int P, int64_t ld, int64_t gw, int64_t n_waves, int lane,
                                                  int64_t& left, int& qc, int& tc, int& seq0) {
  auto tiles_of = [&](int q) __attribute__((always_inline)) {
    return uint32_t((min(int64_t((q_pos[q] + 1) / P), ld) + TILE - 1) / TILE);  // ld bounds a row
  };
  int64_t total = 0;
  uint32_t nt0 = 0, inc0 = 0;
  seq0 = 0;
  for (int q0 = 0; q0 < n_q; q0 += 64) {
    const int q = q0 + lane;
    const uint32_t nt = q < n_q ? tiles_of(q) : 0u;
    if (q0 == 0) seq0 = q < n_q ? q_seq[q] : 0;
    uint32_t sum;
    const uint32_t inc = wave_scan_u32(nt, sum);
    if (q0 == 0) {
      nt0 = nt;
      inc0 = inc;
    }
    total += sum;
  }
  const int64_t t_begin = gw * total / n_waves, t_end = (gw + 1) * total / n_waves;
  left = t_end - t_begin;
  qc = tc = 0;
  if (t_begin >= t_end) return false;
  if (n_q <= 64) {
    const uint64_t m = __ballot(int64_t(inc0) > t_begin);
    const int l = __builtin_ctzll(m);
    qc = l;
    tc = int(t_begin - int64_t(__builtin_amdgcn_readlane(int(inc0 - nt0), l)));
  } else {
    int64_t before = 0;
    for (int q0 = 0; q0 < n_q; q0 += 64) {
      const int q = q0 + lane;
      const uint32_t nt = q < n_q ? tiles_of(q) : 0u;
      uint32_t sum;
      const uint32_t inc = wave_scan_u32(nt, sum);
      if (before + sum > t_begin) {
        const uint64_t m = __ballot(before + inc > t_begin);
        const int l = __builtin_ctzll(m);
        qc = q0 + l;
        tc = int(t_begin - before - int64_t(__builtin_amdgcn_readlane(int(inc - nt), l)));
        break;
      }
      before += sum;
    }
  }
  return true;
}

// Pools pooled in the same launch as the decode scoring (dsa_compress_score): entry e < n is pool pool_id[e] of
// sequence pool_seq[e], pooled from key / gate rows src[e] (src NULL: row e), exactly as kpool_compress does.
template <class T>
struct PendPools {
  const T* keys;
  const T* gates;  // may be NULL
  const T* ape;    // may be NULL
  const int32_t* src;
  const int32_t* pool_seq;
  const int32_t* pool_id;
  T* pooled;  // the pooled cache the entries are written to
  int n;      // 0 .. SC_MAXPEND
};

// channel c of entry e's pooled key, rounded to the storage type: the value kpool_compress stores
template <class T>
__device__ __forceinline__ T pend_value(const PendPools<T>& pp, int64_t src_row, int c, int P, int D) {
  return Elem<T>::from_f32(pool_channel<T>(pp.keys + src_row * P * D + c,
                                           pp.gates ? pp.gates + src_row * P * D + c : nullptr,
                                           pp.ape ? pp.ape + c : nullptr, P, D));
}

// ---------------------------------------------------------------------------------------------------------------
// decode: a persistent grid; the 32-pool tiles of all queries, taken query by query, are split into one contiguous
// range per wave of about equal length, so rows of any length mix keep every wave streaming.  A wave covers its
// range as segments, one per query it touches (and at most 31 tiles and 63 pages each): per segment it loads the
// query's fragments and page ids once, streams the tiles through its private LDS tile two ahead in registers, and
// writes the segment's scores out.  No block-wide barrier: waves run independently.
//
// FUSE: the launch also pools the entries of `pend` (at most 64, one per lane).  Global wave w writes entries
// w, w + waves, ... to the pooled cache.  A wave whose segment contains an entry's pool does not wait for that
// write: it pools the entry itself (the same function of the same inputs, so the same bits) and puts the row into
// its LDS tile over whatever the tile load read from the cache, before the tile is multiplied.  The first entry of
// a segment is pooled in the segment's prologue, beside its other loads; further ones (several pools of one
// sequence completing in one call) are pooled when their tile comes.
// ---------------------------------------------------------------------------------------------------------------
template <class T, int D, bool FUSE>
__global__ __launch_bounds__(256) void score_decode_kernel(
    const T* pooled, const int32_t* __restrict__ bt, int bt_stride, int log2_ppp,
    const T* __restrict__ q_idx, const float* __restrict__ w, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int n_q, int Hi, int P, float* __restrict__ scores, int64_t ld,
    const PendPools<T> pend) {
  using S = ScoreShape<T, D>;
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int CHT = S::TCH / 64;  // chunks per lane per tile
  __shared__ __align__(16) T tiles[4][32 * S::RS];
  __shared__ float sbuf[4][SC_MAXCHUNK / 4];  // each wave's scores of one segment, written out after its loop

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  auto pools_of = [&](int q) __attribute__((always_inline)) {
    return int(min(int64_t((q_pos[q] + 1) / P), ld));  // ld bounds a row
  };
  // FUSE: lane e holds entry e (lanes past the list: sequence -1, which no query has)
  constexpr int NPV = (D + 63) / 64;  // channels per lane of one pooled row
  int pend_seq = -1, pend_id = 0, pend_src = 0;
  const int gw = int(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(wave), nw = int(gridDim.x) * 4;
  // pooled row of entry e (lane's channels lane + 64 i), and its cache row
  auto pool_entry = [&](int e, T(&v)[NPV]) __attribute__((always_inline)) {
    const int64_t sr = __builtin_amdgcn_readlane(pend_src, e);
#pragma unroll
    for (int i = 0; i < NPV; ++i)
      if (lane + 64 * i < D) v[i] = pend_value(pend, sr, lane + 64 * i, P, D);
    return paged_row(bt, bt_stride, __builtin_amdgcn_readlane(pend_seq, e), __builtin_amdgcn_readlane(pend_id, e),
                     log2_ppp);
  };
  auto store_entry = [&](int64_t row, const T(&v)[NPV]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPV; ++i)
      if (lane + 64 * i < D) pend.pooled[row * D + lane + 64 * i] = v[i];
  };
  // Wave gw writes entries gw, gw + nw, ...: the first one pooled in its first segment's prologue (its loads join
  // that prologue's) and stored after its last segment, so the write costs the scoring no latency; any further
  // ones (a grid of fewer waves than entries) at once.
  T wv_e[NPV];
  int64_t w_row = 0;
  bool w_pooled = false;
  const bool w_own = FUSE && gw < pend.n;
  if constexpr (FUSE) {
    if (lane < pend.n) {
      pend_seq = pend.pool_seq[lane];
      pend_id = pend.pool_id[lane];
      pend_src = pend.src ? pend.src[lane] : lane;
    }
    for (int e = gw + nw; e < pend.n; e += nw) {
      T v[NPV];
      store_entry(pool_entry(e, v), v);
    }
  }
  int64_t left;
  int qc, tc, seq0;  // query and tile of the cursor; q_seq of query `lane` (first 64 queries)
  if (!decode_wave_range<32>(q_seq, q_pos, n_q, P, ld, int64_t(blockIdx.x) * 4 + wave, int64_t(gridDim.x) * 4,
                             lane, left, qc, tc, seq0)) {
    if (w_own) {
      w_row = pool_entry(gw, wv_e);
      store_entry(w_row, wv_e);
    }
    return;
  }

  T* tile = tiles[wave];
  float* sb = sbuf[wave];
  const int ppp_mask = (1 << log2_ppp) - 1;
  while (left > 0 && qc < n_q) {
    const int n_c = pools_of(qc);
    const int nt = (n_c + 31) / 32;
    // tiles of this segment: the scores fit the wave's buffer (32 tiles), and the pools span at most 64 pages
    // (one page id per lane)
    int seg = int(min(int64_t(min(nt - tc, SC_MAXCHUNK / 4 / 32)), left));
    while (seg > 1 && (((min((tc + seg) * 32, n_c) - 1) >> log2_ppp) - ((tc * 32) >> log2_ppp)) >= 64) --seg;
    if (seg > 0) {
      // (the segment's bounds are wave-uniform: pinned to scalar registers so the load addresses stay scalar)
      const int qi = __builtin_amdgcn_readfirstlane(qc);
      const int seq = qi < 64 ? __builtin_amdgcn_readlane(seq0, qi) : q_seq[qi];
      const int w_begin = __builtin_amdgcn_readfirstlane(tc * 32);
      const int w_end = __builtin_amdgcn_readfirstlane(min(w_begin + seg * 32, n_c));
      F qa[1][S::STEPS];
      float wv[1][16];
      score_query_frags<T, D>(q_idx, w, qi, true, Hi, n, g, qa[0], wv[0]);
      // page id of each page the segment touches: lane l holds page (w_begin >> log2_ppp) + l
      const int pg0 = w_begin >> log2_ppp;
      const int npg = ((w_end - 1) >> log2_ppp) - pg0 + 1;
      const int page_reg = lane < npg ? bt[int64_t(seq) * bt_stride + pg0 + lane] : 0;
      // FUSE: the segment's first pending pool (pr: its offset from w_begin, -1 if none), pooled now; `more` holds
      // any further entries that fall in the segment.  The wave's own entry to write is pooled in its first
      // prologue.
      T pv[NPV];
      int pr = -1;
      uint64_t more = 0;
      if constexpr (FUSE) {
        if (w_own && !w_pooled) {
          w_row = pool_entry(gw, wv_e);
          w_pooled = true;
        }
        const uint64_t mm = __ballot(pend_seq == seq && pend_id >= w_begin && pend_id < w_end);
        if (mm) {
          const int e = __builtin_ctzll(mm);
          pr = __builtin_amdgcn_readlane(pend_id, e) - w_begin;
          pool_entry(e, pv);
          more = mm & (mm - 1);
        }
      }
      // The first tile needs the page ids anyway: wait for every prologue load here, so that only tile loads are
      // in flight in the loop and the compiler's wait counts there stay exact.
      __builtin_amdgcn_s_waitcnt(0);
      // Loads and steps are unconditional (a tile past the range re-reads a valid pool) and no global store sits in
      // the loop (stores share the load counter and would force full drains): a wave waits only for the tile it
      // stores to LDS, never for the one loaded after it.
      auto run = [&](auto scalar_pages) __attribute__((always_inline)) {
        // scalar_pages: 256-byte pooled rows and pages of >= 4 rows, so the 4 rows of one wave load lie in one
        // page: its id is uniform (a readlane) and the address a scalar base plus lane * 16.
        auto load_tile = [&](int t, u32x4(&R)[CHT]) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < CHT; ++i) {
            if constexpr (decltype(scalar_pages)::value) {
              int p4 = w_begin + t * 32 + 4 * i;
              p4 = p4 < w_end ? p4 : w_begin;  // past the range: re-read valid pools, never scored
              const int page = __builtin_amdgcn_readlane(page_reg, (p4 >> log2_ppp) - pg0);
              const char* rp = reinterpret_cast<const char*>(pooled) +
                               ((int64_t(page) << log2_ppp) + (p4 & ppp_mask)) * int64_t(D * sizeof(T));
              R[i] = *reinterpret_cast<const u32x4*>(rp + lane * 16);
            } else {
              const int c = i * 64 + lane;
              int pool = w_begin + t * 32 + c / S::CPR;
              pool = pool < w_end ? pool : w_begin;  // past the range: re-read a valid pool, never scored
              const int page = __shfl(page_reg, (pool >> log2_ppp) - pg0);
              const int64_t row = (int64_t(page) << log2_ppp) + (pool & ppp_mask);
              R[i] = *reinterpret_cast<const u32x4*>(pooled + row * D + (c % S::CPR) * S::EPC);
            }
          }
        };
        auto step = [&](int t, u32x4(&R)[CHT]) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < CHT; ++i) {
            const int c = i * 64 + lane;
            *reinterpret_cast<u32x4*>(tile + (c / S::CPR) * S::RS + (c % S::CPR) * S::EPC) = R[i];
          }
          if constexpr (FUSE) {
            // pending pools of this tile replace the rows just stored (LDS operations of a wave run in order)
            const int r = pr - t * 32;
            if (r >= 0 && r < 32) {
#pragma unroll
              for (int i = 0; i < NPV; ++i)
                if (lane + 64 * i < D) tile[r * S::RS + lane + 64 * i] = pv[i];
            }
            for (uint64_t m = more; m; m &= m - 1) {
              const int e = __builtin_ctzll(m);
              const int rr = __builtin_amdgcn_readlane(pend_id, e) - w_begin - t * 32;
              if (rr < 0 || rr >= 32) continue;
              T v[NPV];
              pool_entry(e, v);
#pragma unroll
              for (int i = 0; i < NPV; ++i)
                if (lane + 64 * i < D) tile[rr * S::RS + lane + 64 * i] = v[i];
            }
          }
          load_tile(t + 2, R);
          F kb[S::STEPS];
          const T* kp = tile + n * S::RS + g * (D / 2);
#pragma unroll
          for (int s = 0; s < S::STEPS; ++s) kb[s] = E::frag_load(kp + s * S::KPL);
          float sc[1];
          score_tiles<T, D, 1>(qa, kb, wv, sc);
          if (g == 0) sb[t * 32 + n] = sc[0];  // slots past the range are never written out
        };
        u32x4 R0[CHT], R1[CHT];
        load_tile(0, R0);
        __builtin_amdgcn_sched_barrier(0);  // keep tile 0's loads older than tile 1's, as in the loop
        load_tile(1, R1);
        for (int t = 0; t < seg; t += 2) {
          step(t, R0);
          step(t + 1, R1);
        }
      };
      if (S::CPR == 16 && log2_ppp >= 2) run(std::true_type{});
      else run(std::false_type{});
      float* srow = scores + int64_t(qi) * ld + w_begin;
      for (int i = lane; i < w_end - w_begin; i += 64) srow[i] = sb[i];
      left -= seg;
      tc += seg;
    }
    if (tc >= nt) {
      ++qc;
      tc = 0;
    }
  }
  if constexpr (FUSE) {
    if (w_own) {
      if (!w_pooled) w_row = pool_entry(gw, wv_e);
      store_entry(w_row, wv_e);
    }
  }
}

// ---------------------------------------------------------------------------------------------------------------
// prefill: grid = (n_q / 16) x n_chunks; a block covers `chunk_pools` pools for 16 queries
// ---------------------------------------------------------------------------------------------------------------
constexpr int SC_QW = 2;              // queries per wave
constexpr int SC_PWAVES = 8;          // waves per prefill block
constexpr int SC_PTHREADS = 64 * SC_PWAVES;
constexpr int SC_QG = SC_PWAVES * SC_QW;  // queries per block
constexpr int SC_MAXPG = 1024;        // page ids of one block's pool range held in LDS
constexpr int SC_PMAXCHUNK = 4096;    // pools per block
constexpr int SC_PT = 64;             // pools per tile: two 32-pool MFMA column blocks
constexpr int SC_NBUF = 4;            // LDS tile buffers: tiles t, t + 1 readable, t + 2, t + 3 landing

// LDS image of one 64-pool tile.  Pooled row r holds its 16-byte chunks at positions r * CPR + (c ^ (r & SWZ)):
// the XOR puts the rows that one B-operand read touches (one chunk of 32 consecutive rows) on distinct bank
// groups without padding, so each wave-wide direct global-to-LDS load fills 1 KiB of consecutive positions.
template <class T, int D>
struct PrefillTile {
  static constexpr int EPC = 16 / int(sizeof(T));
  static constexpr int CPR = D / EPC;                  // 16-byte chunks per pooled row
  static constexpr int TCH = SC_PT * CPR;              // chunks per tile
  static constexpr int CHT = (TCH + SC_PTHREADS - 1) / SC_PTHREADS;  // direct loads per thread per tile
  static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;  // XOR mask of a row's chunk positions
  static constexpr int BYTES = TCH * 16;
  static_assert(TCH % SC_PTHREADS == 0 || SC_PTHREADS % TCH == 0,
                "a tile is a whole number of block-wide loads, or part of one");
  static_assert((SC_PTHREADS / CPR) % (SWZ + 1) == 0, "a thread's chunk position is the same in all its loads");
};


template <class T, int D>
__global__ __launch_bounds__(SC_PTHREADS, 2) void score_prefill_kernel(
    const T* __restrict__ pooled, const int32_t* __restrict__ bt, int bt_stride, int log2_ppp,
    const T* __restrict__ q_idx, const float* __restrict__ w, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int n_q, int Hi, int P, float* __restrict__ scores, int64_t ld,
    int chunk_pools, int n_chunks) {
  using S = ScoreShape<T, D>;
  using PT = PrefillTile<T, D>;
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int CHT = PT::CHT;
  // separate arrays rather than one: the compiler tells separate LDS variables apart, so a read of one buffer
  // never waits for the direct loads still landing in another
  __shared__ __align__(16) char tiles0[PT::BYTES];
  __shared__ __align__(16) char tiles1[PT::BYTES];
  __shared__ __align__(16) char tiles2[PT::BYTES];
  __shared__ __align__(16) char tiles3[PT::BYTES];
  static_assert(SC_NBUF == 4, "one LDS array per buffer");
  auto tile_buf = [&](int buf) __attribute__((always_inline)) {
    return buf == 0 ? tiles0 : buf == 1 ? tiles1 : buf == 2 ? tiles2 : tiles3;
  };
  __shared__ int page_s[SC_MAXPG];
  __shared__ int seq_s[SC_QG];
  __shared__ int nc_s[SC_QG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same value, known to be wave-uniform
  const int n = lane & 31, g = lane >> 5;
  const int grp = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - grp * n_chunks;
  const int r0 = grp * SC_QG;
  if (tid < SC_QG) {
    const int row = r0 + tid;
    seq_s[tid] = row < n_q ? q_seq[row] : -1;
    nc_s[tid] = row < n_q ? int(min(int64_t((q_pos[row] + 1) / P), ld)) : 0;
  }
  F qa[SC_QW][S::STEPS];
  float wv[SC_QW][16];
#pragma unroll
  for (int r = 0; r < SC_QW; ++r) {
    const int row = r0 + wave * SC_QW + r;
    score_query_frags<T, D>(q_idx, w, row, row < n_q, Hi, n, g, qa[r], wv[r]);
  }
  // byte offset, within a tile, of lane (n, g)'s B operand at k-step s of the first 32-pool column block (the
  // second block lies 32 rows further; rows 32 apart share their XOR pattern)
  int koff[S::STEPS];
#pragma unroll
  for (int s = 0; s < S::STEPS; ++s) {
    const int e = g * (D / 2) + s * S::KPL, c = e / PT::EPC;
    koff[s] = (n * PT::CPR + (c ^ (n & PT::SWZ))) * 16 + (e % PT::EPC) * int(sizeof(T));
  }
  __syncthreads();

  unsigned pending = 0;
  for (int r = 0; r < SC_QG; ++r)
    if (seq_s[r] >= 0) pending |= 1u << r;
  const int p_begin = chunk * chunk_pools;
  const int ppp_mask = (1 << log2_ppp) - 1;

  while (pending) {
    const int seq = seq_s[__builtin_ctz(pending)];
    unsigned active = 0;
    int ncmax = 0;
    for (int r = 0; r < SC_QG; ++r)
      if (((pending >> r) & 1u) && seq_s[r] == seq) {
        active |= 1u << r;
        ncmax = max(ncmax, nc_s[r]);
      }
    pending &= ~active;
    const int p_end = min(p_begin + chunk_pools, ncmax);
    if (p_end <= p_begin) continue;
    const int ntile = (p_end - p_begin + SC_PT - 1) / SC_PT;
    const int pg0 = p_begin >> log2_ppp;
    const int npg = ((p_end - 1) >> log2_ppp) - pg0 + 1;
    __syncthreads();  // the previous sequence's page ids are no longer read
    for (int j = tid; j < npg; j += SC_PTHREADS) page_s[j] = bt[int64_t(seq) * bt_stride + pg0 + j];
    __syncthreads();

    // Each query row's scores go through a buffer resource sized to the pools this block may write for it
    // (below min(n_c, p_end); none for a row of another sequence): stores of masked lanes, of pools past the
    // range and of the pipeline's warm-up step fall outside it and are dropped by the hardware, without a
    // branch.
    __amdgpu_buffer_rsrc_t dst[SC_QW];
#pragma unroll
    for (int r = 0; r < SC_QW; ++r) {
      const int qr = wave_u * SC_QW + r;
      const int lim = ((active >> qr) & 1u) ? min(nc_s[qr], p_end) : 0;
      const uint64_t base = reinterpret_cast<uint64_t>(scores + int64_t(r0 + qr) * ld);
      const uint64_t base_u = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(base >> 32)))) << 32) |
                              uint32_t(__builtin_amdgcn_readfirstlane(int(base)));
      dst[r] = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<float*>(base_u), 0,
                                                 __builtin_amdgcn_readfirstlane(lim) * 4, 0x00020000);
    }
    // page ids of the rows this thread loads for tile t (a pool past the range re-reads the first pool)
    auto tile_pages = [&](int t, int(&pg)[CHT]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < CHT; ++i) {
        int pool = p_begin + t * SC_PT + min(i * SC_PTHREADS + tid, PT::TCH - 1) / PT::CPR;
        pool = pool < p_end ? pool : p_begin;
        pg[i] = page_s[(pool >> log2_ppp) - pg0];
      }
    };
    // tile t into LDS buffer `buf`: CHT wave-wide 16-byte loads straight into LDS per thread
    auto load_tile = [&](int t, int buf, const int(&pg)[CHT]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < CHT; ++i) {
        // a tile smaller than one block-wide load is filled by the first waves (a wave-uniform condition)
        if (PT::TCH < SC_PTHREADS && wave_u * 64 >= PT::TCH) break;
        const int q = i * SC_PTHREADS + tid, row = q / PT::CPR, c = (q % PT::CPR) ^ (row & PT::SWZ);
        int pool = p_begin + t * SC_PT + row;
        pool = pool < p_end ? pool : p_begin;
        const int64_t prow = (int64_t(pg[i]) << log2_ppp) + (pool & ppp_mask);
        const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(tile_buf(buf)));  // the LDS offset
        lds_dma16(pooled + prow * D + c * PT::EPC, lds + uint32_t((i * SC_PTHREADS + wave_u * 64) * 16));
      }
    };
    F kb[S::STEPS];  // B operands of the column block being computed
    // B operands of one 32-pool column block, read from LDS
    auto read_kb = [&](const char* kp, F(&kb)[S::STEPS]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < S::STEPS; ++s) kb[s] = *reinterpret_cast<const F*>(kp + koff[s]);
    };
    // One column block: its MFMAs (B operands in kb) interleaved, k-step by k-step, with the epilogue of the
    // previous block (accumulators `prev`, pools of tile t_prev, block u_prev), and each k-step's B registers
    // refilled from `next` (the following column block) right after its MFMAs are issued, so every read has a
    // whole block of MFMAs to land.  A scheduling barrier closes each k-step, which keeps this order.
    auto half = [&](f32x16(&acc)[SC_QW], const f32x16(&prev)[SC_QW], const char* next, int t_prev, int u_prev)
                    __attribute__((always_inline)) {
      constexpr int EPS = 16 / S::STEPS;  // epilogue elements per k-step
      float part[SC_QW];
#pragma unroll
      for (int s = 0; s < S::STEPS; ++s) {
#pragma unroll
        for (int r = 0; r < SC_QW; ++r) {
          acc[r] = mfma32(qa[r][s], kb[s], s == 0 ? f32x16{} : acc[r]);
#pragma unroll
          for (int i = s * EPS; i < (s + 1) * EPS; ++i) {  // ReLU as an integer max, as in score_reduce
            const float x = prev[r][i];
            const float y = __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
            part[r] = i == 0 ? wv[r][i] * y : part[r] + wv[r][i] * y;
          }
        }
        kb[s] = *reinterpret_cast<const F*>(next + koff[s]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the partner lane l ^ 32 holds the other 16 heads of the pool (as in score_reduce)
      float sc[SC_QW];
#pragma unroll
      for (int r = 0; r < SC_QW; ++r) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, part[r]), 0u, false, false);
        const uint32_t lo = sw[0], hi = sw[1];
        sc[r] = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
      }
      const int off =
          (g == 0 && t_prev >= 0) ? (p_begin + t_prev * SC_PT + u_prev * 32 + n) * 4 : int(0x80000000);
#pragma unroll
      for (int r = 0; r < SC_QW; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc[r]), dst[r], off, 0, 0);
    };
    auto epi = [&](int t, int u, const f32x16(&acc)[SC_QW]) __attribute__((always_inline)) {
      float sc[SC_QW];
      score_reduce<SC_QW>(acc, wv, sc);
      const int off = (g == 0 && t >= 0) ? (p_begin + t * SC_PT + u * 32 + n) * 4 : int(0x80000000);
#pragma unroll
      for (int r = 0; r < SC_QW; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc[r]), dst[r], off, 0, 0);
    };
    // Load pipeline.  Vector-memory operations complete in issue order, so "tile t + 2 has landed" is a count:
    // iteration t issues the loads of tile t + 3 first, then 2 * SC_QW score stores, and waits until at most
    // 4 * SC_QW + CHT operations are outstanding -- the previous iteration's stores, this iteration's loads and
    // stores -- before the barrier that publishes tile t + 2 to all waves.  Tile t + 1 is thus readable during
    // iteration t, whose second column block refills the B registers with its first.  Scheduling barriers keep
    // every vector-memory operation inside its part of the iteration (other instructions may cross them).
    constexpr int PIN = 0x38F;  // ALU, VALU, SALU, MFMA and LDS instructions may cross; vector memory may not
    int pg[CHT];
    f32x16 accA[SC_QW], accB[SC_QW];
#pragma unroll
    for (int r = 0; r < SC_QW; ++r) accA[r] = accB[r] = f32x16{};
    tile_pages(0, pg);
    load_tile(0, 0, pg);
    tile_pages(1, pg);
    load_tile(1, 1, pg);
    tile_pages(2, pg);
    load_tile(2, 2, pg);
    epi(-1, 0, accA);  // warm-up: the stores an iteration before the first would have issued (all dropped)
    epi(-1, 1, accB);
    tile_pages(3, pg);
    __builtin_amdgcn_sched_barrier(PIN);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(CHT + 2 * SC_QW));  // tiles 0 and 1
    __builtin_amdgcn_s_barrier();
    read_kb(tile_buf(0), kb);
    constexpr int HALF = 32 * PT::CPR * 16;  // byte offset of the second column block
    auto iter = [&](int t, int buf) __attribute__((always_inline)) {
      // buffer (buf + 3) % 4 was last read in iteration t - 1, which every wave has finished
      load_tile(t + 3, (buf + 3) % SC_NBUF, pg);
      __builtin_amdgcn_sched_barrier(PIN);
      tile_pages(t + 4, pg);
      __builtin_amdgcn_sched_barrier(0);
      half(accA, accB, tile_buf(buf) + HALF, t - 1, 1);
      half(accB, accA, tile_buf((buf + 1) % SC_NBUF), t, 0);
      __builtin_amdgcn_sched_barrier(PIN);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * SC_QW + CHT));  // tile t + 2
      __builtin_amdgcn_s_barrier();
    };
    // unrolled by the buffer count, so every LDS address offset is a constant
    for (int t = 0;;) {
      iter(t, 0);
      if (++t >= ntile) break;
      iter(t, 1);
      if (++t >= ntile) break;
      iter(t, 2);
      if (++t >= ntile) break;
      iter(t, 3);
      if (++t >= ntile) break;
    }
    epi(ntile - 1, 1, accB);
    // drain the loads still in flight into LDS before the buffers are reused
    __builtin_amdgcn_s_waitcnt(0);
  }
}

template <class T, int D>
static void launch_score_t(const ScoreLaunch& a, bool prefill, int chunk, int n_chunks, int n_groups,
                           int decode_blocks, const CompressLaunch* c, hipStream_t s) {
  if (prefill) {
    score_prefill_kernel<T, D><<<dim3(unsigned(int64_t(n_groups) * n_chunks)), dim3(SC_PTHREADS), 0, s>>>(
        (const T*)a.pooled, a.bt, a.bt_stride, a.log2_ppp, (const T*)a.q_idx, a.w, a.q_seq, a.q_pos, a.n_q, a.Hi,
        a.P, a.scores, a.ld, chunk, n_chunks);
  } else if (c) {
    const PendPools<T> pp{(const T*)c->keys, (const T*)c->gates, (const T*)c->ape, c->src, c->pool_seq,
                          c->pool_id, (T*)c->pooled, c->n_pools};
    score_decode_kernel<T, D, true><<<dim3(unsigned(decode_blocks)), dim3(256), 0, s>>>(
        (const T*)a.pooled, a.bt, a.bt_stride, a.log2_ppp, (const T*)a.q_idx, a.w, a.q_seq, a.q_pos, a.n_q, a.Hi,
        a.P, a.scores, a.ld, pp);
  } else {
    score_decode_kernel<T, D, false><<<dim3(unsigned(decode_blocks)), dim3(256), 0, s>>>(
        (const T*)a.pooled, a.bt, a.bt_stride, a.log2_ppp, (const T*)a.q_idx, a.w, a.q_seq, a.q_pos, a.n_q, a.Hi,
        a.P, a.scores, a.ld, PendPools<T>{});
  }
}

// compute units of the current device (looked up once per device)
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

// the decode kernel is the one that runs (the prefill kernel takes runs of >= 8 queries of one sequence)
static bool score_decode_shape(const ScoreLaunch& a) { return a.group < 8; }

// c: pools to pool in the same launch (decode kernel only; NULL for none)
static kp_status launch_score_impl(const ScoreLaunch& a, const CompressLaunch* c, hipStream_t s) {
  const int64_t ncmax = (int64_t(a.max_pos) + 1) / a.P;
  if (a.n_q == 0 || ncmax == 0) return KP_OK;
  const int64_t ppp = int64_t(1) << a.log2_ppp;
  // prefill shape when the caller promises runs of >= 8 queries of one sequence (a block takes 16)
  const bool prefill = !score_decode_shape(a);
  if (!prefill) {
    // persistent decode grid: SC_DBLOCKS_PER_CU blocks per compute unit, fewer when the tiles are few (about one
    // tile per wave, counted on the longest row: a small batch is latency-bound, and more waves in flight shorten
    // it -- one 32K-context query runs 1.3 us faster than with four tiles per wave)
    const int64_t tiles_ub = int64_t(a.n_q) * ((ncmax + 31) / 32);
    int64_t blocks = int64_t(SC_DBLOCKS_PER_CU) * cu_count();
    const int64_t few = (tiles_ub + 3) / 4;
    if (few < blocks) blocks = few < 1 ? 1 : few;
    if (a.dtype == KP_DTYPE_BF16) {
      if (a.D == 128) launch_score_t<bf16, 128>(a, false, 0, 0, 0, int(blocks), c, s);
      else launch_score_t<bf16, 32>(a, false, 0, 0, 0, int(blocks), c, s);
    } else {
      launch_score_t<float, 32>(a, false, 0, 0, 0, int(blocks), c, s);
    }
    return check_launch(c ? "dsa_compress_score" : "dsa_indexer_score");
  }
  const int64_t n_groups = (a.n_q + SC_QG - 1) / SC_QG;
  // pools per block: a multiple of 128 sized for about 1024 blocks, at most SC_PMAXCHUNK, and SC_MAXPG pages per
  // block
  int64_t chunk = (ncmax * n_groups + 1023) / 1024;
  chunk = ((chunk + 127) / 128) * 128;
  if (chunk < 128) chunk = 128;
  if (chunk > SC_PMAXCHUNK) chunk = SC_PMAXCHUNK;
  const int64_t cap = int64_t(SC_MAXPG - 1) * ppp;
  while (chunk > 128 && chunk > cap) chunk -= 128;
  if (chunk > cap) {
    set_error("dsa_indexer_score: pages of %lld pooled rows are too small", (long long)ppp);
    return KP_ERR_UNSUPPORTED;
  }
  const int64_t n_chunks = (ncmax + chunk - 1) / chunk;
  if (n_groups * n_chunks > 0x7fffffff) {
    set_error("dsa_indexer_score: grid of %lld blocks is too large", (long long)(n_groups * n_chunks));
    return KP_ERR_INVALID_ARG;
  }
  if (a.dtype == KP_DTYPE_BF16) {
    if (a.D == 128) launch_score_t<bf16, 128>(a, true, int(chunk), int(n_chunks), int(n_groups), 0, nullptr, s);
    else launch_score_t<bf16, 32>(a, true, int(chunk), int(n_chunks), int(n_groups), 0, nullptr, s);
  } else {
    launch_score_t<float, 32>(a, true, int(chunk), int(n_chunks), int(n_groups), 0, nullptr, s);
  }
  return check_launch("dsa_indexer_score");
}

kp_status launch_score(const ScoreLaunch& a, hipStream_t s) { return launch_score_impl(a, nullptr, s); }

// kpool_compress then dsa_indexer_score.  One launch when the decode kernel scores and the list has 1 ..
// SC_MAXPEND entries (the decode step's case: at most one completing pool per sequence); otherwise the two
// launches, in that order.
kp_status launch_compress_score(const CompressLaunch& c, const ScoreLaunch& a, hipStream_t s) {
  const bool scores = a.n_q > 0 && (int64_t(a.max_pos) + 1) / a.P > 0;
  if (c.n_pools > 0 && c.n_pools <= SC_MAXPEND && scores && score_decode_shape(a))
    return launch_score_impl(a, &c, s);
  const kp_status st = launch_compress(c, s);
  if (st != KP_OK) return st;
  return launch_score(a, s);
}

}  // namespace kp
