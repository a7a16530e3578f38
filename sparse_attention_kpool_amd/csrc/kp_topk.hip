// dsa_topk_select: causal top-k pools per query with the incomplete tail forced.
//
// [MAX glm5_next API page, index_kpool_always_select_tail]: the incomplete trailing pool is always visible.
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: the indexer always keeps
// the incomplete tail.  [GLM-5.3-Flash model card, "Raw config fields"]: index_topk 2048 (pools).  Ties go to
// the lower pool index (the layer's specification).
//
// Exact and deterministic, with no sort.  For one row of n scores and a budget b < n:
//   1. The row is read once into registers as order-preserving uint32 keys (-0 folded into +0): wave w owns a
//      contiguous range of the row and lane l holds its indices lo_w + 64 j + l.  Every later pass works on
//      these registers; LDS only holds a histogram and a few per-wave totals.
//   2. Radix select: the block's min and max key fix the common high bits; the varying bits below are resolved
//      11 at a time (at most three passes), finding the key T of the b-th largest score and how many copies of
//      T the budget still takes (need_eq).  Histograms are integer LDS atomics, so their order does not
//      matter.
//   3. Compaction in index order: every wave counts its range's keys > T and == T with ballots; one exchange of
//      the per-wave totals gives each wave its output offset and its share of the equal keys (the lowest
//      indices first -- exactly the lower-index tie-break); the kept ids come out already ascending, which is
//      the output format.
//   4. The tail pool tau (when (i+1) mod P != 0) is appended; it is larger than every complete pool id.
// A row takes one block, or two steps: every chunk of the row keeps its own top-b candidates (ascending), then
// one block selects the final b among the candidates.  Exact because an element in the row's top b (under score
// desc, index asc) is in the top b of its chunk.  Rows longer than 32768 pools (up to 16 chunks of at most
// 32768, 16 b <= 32768) always take two steps; so do rows of a small batch, whose chunks then spread over more
// blocks.
#include <type_traits>

#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_MAXN = 32768;          // keys of one block: 64 per lane
constexpr int TK_MAXCHUNKS = 16;        // chunks of a two-step row
static_assert(TK_THREADS * 4 == 2048, "every histogram bin has one owner thread");

// LDS state of one selection.
struct TkSync {
  uint32_t hist[2048];  // 11-bit digits; thread t of TK_THREADS owns bins 4t .. 4t+3
  uint32_t wa[TK_WAVES], wb[TK_WAVES];
  uint32_t digit, remaining;
};

// Keys held in registers: lane `lane` of wave w holds indices lo + 64 j + lane (j < NJ) of the row, valid below
// lo + cnt.  Wave ranges are multiples of 64 keys long, so ballot order is index order.
template <int NJ>
struct TkKeys {
  uint32_t k[NJ];
  int lo, cnt;
};

template <int NJ, class Load>
__device__ __forceinline__ void tk_load(TkKeys<NJ>& K, int n, Load load) {
  const int per = ((n + TK_WAVES * 64 - 1) / (TK_WAVES * 64)) * 64;  // <= 64 NJ by the caller's choice of NJ
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  K.lo = min(w * per, n);
  K.cnt = min(per, n - K.lo);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = 64 * j + lane;
    // unconditional (clamped) loads: every load is issued before the first is needed
    const uint32_t v = load(min(K.lo + i, n - 1));
    K.k[j] = i < K.cnt ? v : 0u;
  }
}

// Min and max over the wave (uniform results): within each row by DPP, then the four row values by readlane.
__device__ __forceinline__ void tk_wave_minmax(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp_u32<0xB1>(0xFFFFFFFFu, mn));
  mx = max(mx, dpp_u32<0xB1>(0u, mx));
  mn = min(mn, dpp_u32<0x4E>(0xFFFFFFFFu, mn));
  mx = max(mx, dpp_u32<0x4E>(0u, mx));
  mn = min(mn, dpp_u32<0x141>(0xFFFFFFFFu, mn));
  mx = max(mx, dpp_u32<0x141>(0u, mx));
  mn = min(mn, dpp_u32<0x140>(0xFFFFFFFFu, mn));
  mx = max(mx, dpp_u32<0x140>(0u, mx));
  mn = min(min(uint32_t(__builtin_amdgcn_readlane(int(mn), 0)), uint32_t(__builtin_amdgcn_readlane(int(mn), 16))),
           min(uint32_t(__builtin_amdgcn_readlane(int(mn), 32)), uint32_t(__builtin_amdgcn_readlane(int(mn), 48))));
  mx = max(max(uint32_t(__builtin_amdgcn_readlane(int(mx), 0)), uint32_t(__builtin_amdgcn_readlane(int(mx), 16))),
           max(uint32_t(__builtin_amdgcn_readlane(int(mx), 32)), uint32_t(__builtin_amdgcn_readlane(int(mx), 48))));
}

// Selects the `budget` largest of the block's n keys (0 < budget < n) and calls emit(out_pos, j, i, key) for each
// kept index i (held in the caller's register slot j), out_pos ascending with i.
template <int NJ, class Emit>
__device__ void tk_select(TkSync& sy, const TkKeys<NJ>& K, int budget, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto valid = [&](int j) __attribute__((always_inline)) { return 64 * j + lane < K.cnt; };
  // thread t owns bins 4t .. 4t+3: it zeroes them here and, after reading them, in every pass
  u32x4* own = reinterpret_cast<u32x4*>(sy.hist) + tid;
  *own = u32x4{0u, 0u, 0u, 0u};

  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    mn = min(mn, valid(j) ? K.k[j] : 0xFFFFFFFFu);
    mx = max(mx, K.k[j]);  // slots past cnt hold 0
  }
  tk_wave_minmax(mn, mx);
  if (lane == 0) {
    sy.wa[wv] = mn;
    sy.wb[wv] = mx;
  }
  __syncthreads();  // also orders the zeroing of the bins before the first pass's atomics
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    mn = min(mn, sy.wa[w]);
    mx = max(mx, sy.wb[w]);
  }
  // bits [0, lo) vary; bits at and above lo are common to every key and fixed in `prefix`
  int lo = (mn == mx) ? 0 : 32 - __clz(int(mn ^ mx));
  uint32_t mask = lo == 32 ? 0u : ~((1u << lo) - 1u);
  uint32_t prefix = mn & mask;
  uint32_t remaining = uint32_t(budget);
  // wa / wb are written next after a pass's first barrier, which every thread reaches after the reads above;
  // with no pass, the compaction writes them: wait for the reads here
  if (lo == 0) __syncthreads();
  // Each pass: histogram of the next (up to) 11 bits of the keys that match `prefix` (LDS integer atomics, so
  // their order does not matter); every thread reads its 4 bins and zeroes them for the next pass; a block-wide
  // prefix over the threads (thread order = digit order) finds the bin where the count from the top reaches
  // `remaining`.  Three barriers per pass: digit / remaining are written next two barriers later.  Slots past
  // cnt take part as keys of value 0: below every other key, they never move the budget-th largest key while
  // budget < cnt, and the compaction tells them apart when that key is 0.
  while (lo > 0) {
    const int width = min(11, lo);
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if ((K.k[j] & mask) == prefix) atomicAdd(&sy.hist[(K.k[j] >> shift) & dmask], 1u);
    __syncthreads();
    const bool owns = 4 * tid <= int(dmask);
    const u32x4 c = owns ? *own : u32x4{0u, 0u, 0u, 0u};
    if (owns) *own = u32x4{0u, 0u, 0u, 0u};
    const uint32_t mine = c[0] + c[1] + c[2] + c[3];
    uint32_t wtot;
    const uint32_t inc = wave_scan_u32(mine, wtot);
    if (lane == 0) sy.wa[wv] = wtot;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t t = sy.wa[w];
      before += (w < wv) ? t : 0u;
      total += t;
    }
    const uint32_t above = total - (before + inc);  // keys in higher bins than this thread's
    if (above < remaining && remaining <= above + mine) {
      uint32_t acc = above;
      int d = 3;
      if (acc + c[3] < remaining) {
        acc += c[3];
        d = 2;
        if (acc + c[2] < remaining) {
          acc += c[2];
          d = 1;
          if (acc + c[1] < remaining) {
            acc += c[1];
            d = 0;
          }
        }
      }
      sy.digit = uint32_t(4 * tid + d);
      sy.remaining = remaining - acc;
    }
    __syncthreads();
    prefix |= sy.digit << shift;
    mask |= dmask << shift;
    remaining = sy.remaining;
    lo = shift;
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = remaining;

  // compaction: per-wave counts of keys >= T and == T, one exchange, then each wave emits its range in index
  // order.  Slots past cnt hold 0, so they need telling apart only when T is 0.
  auto compact = [&](auto check) __attribute__((always_inline)) {
    constexpr bool CHECK = decltype(check)::value;
    auto in = [&](int j) __attribute__((always_inline)) { return CHECK ? valid(j) : true; };
    uint32_t ge = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      ge += uint32_t(__popcll(__ballot(in(j) && K.k[j] >= T)));
      eq += uint32_t(__popcll(__ballot(in(j) && K.k[j] == T)));
    }
    if (lane == 0) {
      sy.wa[wv] = ge;
      sy.wb[wv] = eq;
    }
    __syncthreads();
    uint32_t ge_before = 0, eq_before = 0, eq_total = 0;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t a = sy.wa[w], e = sy.wb[w];
      ge_before += (w < wv) ? a : 0u;
      eq_before += (w < wv) ? e : 0u;
      eq_total += e;
    }
    const uint64_t below = (uint64_t(1) << lane) - 1;
    if (NJ < 64 && need_eq == eq_total) {
      // every copy of T is kept: a key is kept iff it is >= T (blocks of 64 keys per lane have registers for one
      // emit loop only and always take the general one)
      uint32_t at = ge_before;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool take = in(j) && K.k[j] >= T;
        const uint64_t tm = __ballot(take);
        if (take) emit(int(at + uint32_t(__popcll(tm & below))), j, K.lo + 64 * j + lane, K.k[j]);
        at += uint32_t(__popcll(tm));
      }
    } else {
      // kept before this wave: all greater keys plus the first need_eq equal keys in index order
      uint32_t at = (ge_before - eq_before) + min(eq_before, need_eq);
      uint32_t eq_seen = eq_before;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool is_eq = in(j) && K.k[j] == T;
        const uint64_t eqm = __ballot(is_eq);
        const uint32_t eq_rank = eq_seen + uint32_t(__popcll(eqm & below));
        const bool take = K.k[j] > T || (is_eq && eq_rank < need_eq);  // a slot past cnt is never > T
        const uint64_t tm = __ballot(take);
        if (take) emit(int(at + uint32_t(__popcll(tm & below))), j, K.lo + 64 * j + lane, K.k[j]);
        at += uint32_t(__popcll(tm));
        eq_seen += uint32_t(__popcll(eqm));
      }
    }
  };
  if constexpr (NJ >= 64) {
    compact(std::true_type{});  // one form only, for the same reason
  } else {
    if (T == 0u) compact(std::true_type{});
    else compact(std::false_type{});
  }
  __syncthreads();
}

__device__ __forceinline__ void tk_geometry(int pos, int P, int k, int64_t ld, int& n_c, int& r, int& tau, int& b) {
  n_c = int(min(int64_t((pos + 1) / P), ld));  // ld bounds a row even if pos exceeds the promised max
  r = (pos + 1) % P;
  tau = pos / P;
  b = min(k - (r ? 1 : 0), n_c);
}

// Tail, -1 padding and the count, after `cnt` complete pools were written.
__device__ __forceinline__ void tk_finish(int32_t* out, int32_t* n_sel, int q, int k, int cnt, int r, int tau) {
  if (threadIdx.x == 0) {
    if (r) out[cnt] = tau;
    n_sel[q] = cnt + (r ? 1 : 0);
  }
  for (int j = cnt + (r ? 1 : 0) + threadIdx.x; j < k; j += TK_THREADS) out[j] = -1;
}

// One block per query row (rows of at most 64 NJ TK_WAVES pools).
template <int NJ>
__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                              const int32_t* __restrict__ q_pos, int P, int k,
                                                              int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ TkSync sy;
  const int q = blockIdx.x;
  int n_c, r, tau, b;
  tk_geometry(q_pos[q], P, k, ld, n_c, r, tau, b);
  const float* row = scores + int64_t(q) * ld;
  int32_t* out = sel + int64_t(q) * k;
  if (b >= n_c) {
    for (int p = threadIdx.x; p < n_c; p += TK_THREADS) out[p] = p;
  } else if (b > 0) {
    TkKeys<NJ> K;
    tk_load(K, n_c, [&](int i) __attribute__((always_inline)) { return score_key(row[i]); });
    tk_select(sy, K, b, [&](int at, int, int i, uint32_t) __attribute__((always_inline)) { out[at] = i; });
  }
  tk_finish(out, n_sel, q, k, max(b, 0), r, tau);
}

// Step 1 of a two-step row: chunk c of row q keeps min(b, chunk length) candidates (key, pool id), ascending.
template <int NJ>
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(const float* __restrict__ scores, int64_t ld,
                                                                const int32_t* __restrict__ q_pos, int P, int k,
                                                                int n_chunks, int chunk_len,
                                                                uint32_t* __restrict__ cand_key,
                                                                int32_t* __restrict__ cand_idx) {
  __shared__ TkSync sy;
  __shared__ __align__(16) uint32_t st_key[TK_MAXN / 2];  // b <= k <= TK_MAXN / 2 for a row of >= 2 chunks
  __shared__ __align__(16) uint32_t st_idx[TK_MAXN / 2];
  const int q = blockIdx.x / n_chunks;
  const int c = blockIdx.x - q * n_chunks;
  int n_c, r, tau, b;
  tk_geometry(q_pos[q], P, k, ld, n_c, r, tau, b);
  const int base = c * chunk_len;
  const int len = min(chunk_len, n_c - base);
  if (len <= 0 || b <= 0) return;
  const float* row = scores + int64_t(q) * ld + base;
  const int64_t cb = (int64_t(q) * n_chunks + c) * k;
  if (b >= len) {
    for (int i = threadIdx.x; i < len; i += TK_THREADS) {
      cand_key[cb + i] = score_key(row[i]);
      cand_idx[cb + i] = base + i;
    }
  } else {
    TkKeys<NJ> K;
    tk_load(K, len, [&](int i) __attribute__((always_inline)) { return score_key(row[i]); });
    // the kept candidates are staged in LDS and then written out with whole-row 16-byte stores
    tk_select(sy, K, b, [&](int at, int, int i, uint32_t key) __attribute__((always_inline)) {
      st_key[at] = key;
      st_idx[at] = base + i;
    });
    uint32_t* ok = cand_key + cb;
    uint32_t* oi = reinterpret_cast<uint32_t*>(cand_idx + cb);
    if ((cb & 3) == 0) {
      for (int i = 4 * threadIdx.x; i < b; i += 4 * TK_THREADS) {
        if (i + 4 <= b) {
          *reinterpret_cast<u32x4*>(ok + i) = *reinterpret_cast<const u32x4*>(st_key + i);
          *reinterpret_cast<u32x4*>(oi + i) = *reinterpret_cast<const u32x4*>(st_idx + i);
        } else {
          for (int e = i; e < b; ++e) {
            ok[e] = st_key[e];
            oi[e] = st_idx[e];
          }
        }
      }
    } else {
      for (int i = threadIdx.x; i < b; i += TK_THREADS) {
        ok[i] = st_key[i];
        oi[i] = st_idx[i];
      }
    }
  }
}

constexpr int TK_TREE_CAND = 8192;  // candidates one merge block takes when a row's chunks are merged in a tree

// Step 2 of a two-step row: the b best among chunk candidates, taken in chunk order (ascending ids).
//   FINAL   one block per row over all n_chunks chunks: writes the selection (sel, n_sel, tail, padding).
//   !FINAL  one block per (row, group of `group` consecutive chunks): writes that group's b best candidates
//           (key, pool id), ascending, in the chunk-candidate layout -- so a row of many chunks is merged as a
//           tree, and the final merge reads each group as one chunk of group * chunk_len pools.
// Exact: an element of the row's top b is in the top b of any subset of the row that holds it.
template <int NJ, bool FINAL>
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(const uint32_t* __restrict__ cand_key,
                                                                const int32_t* __restrict__ cand_idx, int64_t ld,
                                                                const int32_t* __restrict__ q_pos, int P, int k,
                                                                int n_chunks, int chunk_len, int group,
                                                                int32_t* __restrict__ sel,
                                                                int32_t* __restrict__ n_sel,
                                                                uint32_t* __restrict__ grp_key,
                                                                int32_t* __restrict__ grp_idx) {
  __shared__ TkSync sy;
  __shared__ int32_t kept[FINAL ? TK_MAXN / 2 : TK_TREE_CAND / 2];  // kept pool ids (or positions), in order
  __shared__ uint32_t kept_key[FINAL ? 1 : TK_TREE_CAND / 2];
  const int n_groups = FINAL ? 1 : (n_chunks + group - 1) / group;
  const int q = blockIdx.x / n_groups;
  const int G = blockIdx.x - q * n_groups;
  const int c0 = FINAL ? 0 : G * group;
  const int c1 = FINAL ? n_chunks : min(c0 + group, n_chunks);
  int n_c, r, tau, b;
  tk_geometry(q_pos[q], P, k, ld, n_c, r, tau, b);
  int32_t* out = sel + int64_t(q) * k;
  const int64_t ob = (int64_t(q) * n_groups + G) * k;  // !FINAL: this group's output candidates
  // Every chunk before the row's last non-empty one is longer than b (chunks hold at least 4k pools, or all
  // 32768) and kept exactly b candidates, so candidate i sits in chunk c0 + i / b at i % b.  (The quotient comes
  // from a float reciprocal, corrected to the exact one: i < 2^15, so the estimate is off by at most one.)
  const int bb = max(b, 1);
  int n2 = 0;
  for (int c = c0; c < c1; ++c) n2 += min(max(b, 0), max(0, min(chunk_len, n_c - c * chunk_len)));
  const int64_t rowc = (int64_t(q) * n_chunks + c0) * k;
  const float inv_bb = 1.f / float(bb);
  auto cand = [&](int i) __attribute__((always_inline)) -> int64_t {
    int c = int(float(i) * inv_bb);
    c -= (c * bb > i) ? 1 : 0;
    c += ((c + 1) * bb <= i) ? 1 : 0;
    return rowc + int64_t(c) * k + (i - c * bb);
  };
  if (b >= n2) {
    for (int i = threadIdx.x; i < n2; i += TK_THREADS) {
      if constexpr (FINAL) {
        out[i] = cand_idx[cand(i)];
      } else {
        grp_key[ob + i] = cand_key[cand(i)];
        grp_idx[ob + i] = cand_idx[cand(i)];
      }
    }
  } else if (b > 0) {
    TkKeys<NJ> K;  // straight from the candidates: every lane issues all its loads at once
    tk_load(K, n2, [&](int i) __attribute__((always_inline)) { return cand_key[cand(i)]; });
    if constexpr (NJ <= 32) {
      // the pool ids are loaded with the keys, so the kept ones go straight to LDS and leave in order with
      // coalesced stores
      TkKeys<NJ> Ix;
      tk_load(Ix, n2, [&](int i) __attribute__((always_inline)) { return uint32_t(cand_idx[cand(i)]); });
      tk_select(sy, K, b, [&](int at, int j, int, uint32_t key) __attribute__((always_inline)) {
        kept[at] = int32_t(Ix.k[j]);
        if constexpr (!FINAL) kept_key[at] = key;
      });
      for (int at = threadIdx.x; at < b; at += TK_THREADS) {
        if constexpr (FINAL) {
          out[at] = kept[at];
        } else {
          grp_key[ob + at] = kept_key[at];
          grp_idx[ob + at] = kept[at];
        }
      }
    } else {
      // no registers for the ids: the selection records positions, then the ids of all kept pools are read at
      // once
      tk_select(sy, K, b, [&](int at, int, int i, uint32_t key) __attribute__((always_inline)) {
        kept[at] = i;
        if constexpr (!FINAL) kept_key[at] = key;
      });
      for (int at = threadIdx.x; at < b; at += TK_THREADS) {
        if constexpr (FINAL) {
          out[at] = cand_idx[cand(kept[at])];
        } else {
          grp_key[ob + at] = kept_key[at];
          grp_idx[ob + at] = cand_idx[cand(kept[at])];
        }
      }
    }
  }
  if constexpr (FINAL) tk_finish(out, n_sel, q, k, max(b, 0), r, tau);
}

// Chunk length of the row split (a multiple of 256; n_chunks = 1 means one block per row).  A row longer than
// one block's registers is always split.  With few rows the split also spreads a row over several blocks
// (about 256 blocks in all), keeping chunks of at least 4k pools so that each chunk's top-k shrinks the merge's
// input.
static int tk_chunk_len(int P, int k, int n_q, int max_pos) {
  const int64_t ncmax = (int64_t(max_pos) + 1) / P;
  if (ncmax <= TK_MAXN && (n_q >= 192 || ncmax <= 4 * int64_t(k))) return TK_MAXN;
  const int64_t want = (256 + int64_t(n_q) - 1) / (n_q > 0 ? n_q : 1);
  int64_t len = (ncmax + want - 1) / want;
  if (len < 4 * int64_t(k)) len = 4 * int64_t(k);
  // never more chunks than the merge holds (TK_MAXCHUNKS, and chunks x k <= TK_MAXN)
  int64_t max_nch = TK_MAXN / (k > 0 ? k : 1);
  if (max_nch > TK_MAXCHUNKS) max_nch = TK_MAXCHUNKS;
  if (max_nch < 1) max_nch = 1;
  if (len < (ncmax + max_nch - 1) / max_nch) len = (ncmax + max_nch - 1) / max_nch;
  len = (len + 255) / 256 * 256;
  if (len > TK_MAXN) len = TK_MAXN;
  return int(len);
}

static int tk_chunks(int P, int k, int n_q, int max_pos) {
  const int64_t ncmax = (int64_t(max_pos) + 1) / P;
  const int len = tk_chunk_len(P, k, n_q, max_pos);
  return int((ncmax + len - 1) / len);
}

size_t topk_workspace(int P, int k, int n_q, int max_pos) {
  const int nch = tk_chunks(P, k, n_q, max_pos);
  if (nch <= 1) return 0;
  const int group = TK_TREE_CAND / (k > 0 ? k : 1);
  const int n_groups = (nch > group && group >= 2) ? (nch + group - 1) / group : 0;
  return size_t(n_q) * (nch + n_groups) * k * (sizeof(uint32_t) + sizeof(int32_t));
}

// keys per lane for n keys in one block: the smallest of 16, 32, 64 that holds them
static int tk_nj(int64_t n) { return n <= 16 * 64 * TK_WAVES ? 16 : n <= 32 * 64 * TK_WAVES ? 32 : 64; }

template <int NJ>
static kp_status launch_topk_nj(const TopkLaunch& a, int nch, int clen, int merge_nj, hipStream_t s) {
  // (nch, clen and merge_nj describe the merge input; a tree merge below replaces them with its groups')
  if (nch <= 1) {
    topk_row_kernel<NJ><<<dim3(unsigned(a.n_q)), dim3(TK_THREADS), 0, s>>>(a.scores, a.ld, a.q_pos, a.P, a.k, a.sel,
                                                                           a.n_sel);
    return check_launch("dsa_topk_select");
  }
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(a.ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(cand_key + size_t(a.n_q) * nch * a.k);
  topk_chunk_kernel<NJ><<<dim3(unsigned(int64_t(a.n_q) * nch)), dim3(TK_THREADS), 0, s>>>(
      a.scores, a.ld, a.q_pos, a.P, a.k, nch, clen, cand_key, cand_idx);
  kp_status st = check_launch("dsa_topk_select (chunks)");
  if (st != KP_OK) return st;
  // many chunks of a large k: merge groups of TK_TREE_CAND / k chunks first, then the groups
  const int group = TK_TREE_CAND / a.k;
  if (nch > group && group >= 2) {
    const int n_groups = (nch + group - 1) / group;
    uint32_t* grp_key = reinterpret_cast<uint32_t*>(cand_idx + size_t(a.n_q) * nch * a.k);
    int32_t* grp_idx = reinterpret_cast<int32_t*>(grp_key + size_t(a.n_q) * n_groups * a.k);
    topk_merge_kernel<16, false><<<dim3(unsigned(int64_t(a.n_q) * n_groups)), dim3(TK_THREADS), 0, s>>>(
        cand_key, cand_idx, a.ld, a.q_pos, a.P, a.k, nch, clen, group, nullptr, nullptr, grp_key, grp_idx);
    st = check_launch("dsa_topk_select (group merge)");
    if (st != KP_OK) return st;
    cand_key = grp_key;
    cand_idx = grp_idx;
    nch = n_groups;
    clen *= group;
    merge_nj = tk_nj(int64_t(nch) * a.k);
  }
  const dim3 grid(unsigned(a.n_q)), block(TK_THREADS);
  if (merge_nj == 16)
    topk_merge_kernel<16, true><<<grid, block, 0, s>>>(cand_key, cand_idx, a.ld, a.q_pos, a.P, a.k, nch, clen, 1,
                                                       a.sel, a.n_sel, nullptr, nullptr);
  else if (merge_nj == 32)
    topk_merge_kernel<32, true><<<grid, block, 0, s>>>(cand_key, cand_idx, a.ld, a.q_pos, a.P, a.k, nch, clen, 1,
                                                       a.sel, a.n_sel, nullptr, nullptr);
  else
    topk_merge_kernel<64, true><<<grid, block, 0, s>>>(cand_key, cand_idx, a.ld, a.q_pos, a.P, a.k, nch, clen, 1,
                                                       a.sel, a.n_sel, nullptr, nullptr);
  return check_launch("dsa_topk_select (merge)");
}

kp_status launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.n_q == 0) return KP_OK;
  const int nch = tk_chunks(a.P, a.k, a.n_q, a.max_pos);
  const int clen = tk_chunk_len(a.P, a.k, a.n_q, a.max_pos);
  if (nch > 1 && (nch > TK_MAXCHUNKS || int64_t(nch) * a.k > TK_MAXN)) {
    set_error("dsa_topk_select: %d pools per row with top-%d exceeds the two-step limit", (a.max_pos + 1) / a.P,
              a.k);
    return KP_ERR_UNSUPPORTED;
  }
  const int64_t ncmax = (int64_t(a.max_pos) + 1) / a.P;
  const int nj = tk_nj(nch <= 1 ? ncmax : clen);
  const int merge_nj = tk_nj(int64_t(nch) * a.k);
  if (nj == 16) return launch_topk_nj<16>(a, nch, clen, merge_nj, s);
  if (nj == 32) return launch_topk_nj<32>(a, nch, clen, merge_nj, s);
  return launch_topk_nj<64>(a, nch, clen, merge_nj, s);
}

}  // namespace kp
