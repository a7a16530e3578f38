// dsa_topk_select: causal top-k pools per query with the incomplete tail forced.
//
// [MAX glm5_next API page, index_kpool_always_select_tail]: the incomplete trailing pool is always visible.
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: the indexer always keeps
// the incomplete tail.  [GLM-5.3-Flash model card, "Raw config fields"]: index_topk 2048 (pools).  Ties go to
// the lower pool index (the layer's specification).
//
// Exact and deterministic, with no sort.  For one row of n scores and a budget b < n:
//   1. The row is copied once into LDS as order-preserving uint32 keys (-0 folded into +0).  Each wave owns a
//      contiguous range of it.
//   2. Radix select: the block's min and max key fix the common high bits; the varying bits below are resolved
//      11 at a time (at most three passes), finding the key T of the b-th largest score and how many copies of
//      T the budget still takes (need_eq).  Histograms are integer LDS atomics, so their order does not
//      matter.
//   3. Compaction in index order: every wave counts its range's keys > T and == T with ballots; one exchange of
//      the per-wave totals gives each wave its output offset and its share of the equal keys (the lowest
//      indices first -- exactly the lower-index tie-break); the kept ids come out already ascending, which is
//      the output format.
//   4. The tail pool tau (when (i+1) mod P != 0) is appended; it is larger than every complete pool id.
// Rows of at most 32768 pools take one block.  Longer rows (up to 16 x 32768) take two steps: every 32768-pool
// chunk keeps its own top-b candidates (ascending), then one block selects the final b among the candidates.
// Exact because an element in the row's top b (under score desc, index asc) is in the top b of its chunk.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_MAXN = 32768;          // keys held in LDS by one block
constexpr int TK_MAXCHUNKS = 16;        // chunks of a two-step row

struct TkShared {
  alignas(16) uint32_t keys[TK_MAXN];
  uint32_t hist[2048];
  uint32_t wa[TK_WAVES], wb[TK_WAVES];
  uint32_t digit, remaining;
};

// Each wave owns a contiguous range of the row: [wave_lo, wave_hi), a multiple of 256 keys long.
__device__ __forceinline__ void tk_wave_range(int n, int& lo, int& hi) {
  const int per = ((n + TK_WAVES * 256 - 1) / (TK_WAVES * 256)) * 256;
  const int w = threadIdx.x >> 6;
  lo = min(w * per, n);
  hi = min(lo + per, n);
}

// Selects the `budget` largest of keys[0..n) (0 < budget < n) and calls emit(out_pos, i) for each kept i,
// out_pos ascending with i.
//
// The radix passes only cover the bits in which the row's keys differ: a first pass takes the block min and
// max, their common high bits are fixed, and the varying bits below are resolved 11 at a time (at most three
// passes).  Digits of varying bits are spread, so plain LDS atomics seldom collide.  A row whose keys are all
// equal needs no pass at all.  Order-free passes read 16 bytes per lane from the wave's contiguous range; the
// compaction walks that range 64 keys per step with ballots, so only the per-wave totals cross waves.
template <class Emit>
__device__ void tk_select(TkShared& sh, int n, int budget, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int lo_i, hi_i;
  tk_wave_range(n, lo_i, hi_i);
  const uint4* k4 = reinterpret_cast<const uint4*>(sh.keys);

  // min / max (keys past n are skipped by index)
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int base = lo_i; base < hi_i; base += 256) {
    const int i = base + 4 * lane;
    if (i < hi_i) {
      const uint4 v = k4[i >> 2];
      const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j < hi_i) {
          mn = min(mn, e[j]);
          mx = max(mx, e[j]);
        }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, uint32_t(__shfl_xor(int(mn), off)));
    mx = max(mx, uint32_t(__shfl_xor(int(mx), off)));
  }
  if (lane == 0) {
    sh.wa[wv] = mn;
    sh.wb[wv] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    mn = min(mn, sh.wa[w]);
    mx = max(mx, sh.wb[w]);
  }
  __syncthreads();
  // bits [0, lo) vary; bits at and above lo are common to every key and fixed in `prefix`
  int lo = (mn == mx) ? 0 : 32 - __clz(int(mn ^ mx));
  uint32_t mask = lo == 32 ? 0u : ~((1u << lo) - 1u);
  uint32_t prefix = mn & mask;
  uint32_t remaining = uint32_t(budget);
  while (lo > 0) {
    const int width = min(11, lo);
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int j = tid; j < 2048; j += TK_THREADS) sh.hist[j] = 0;
    __syncthreads();
    for (int base = lo_i; base < hi_i; base += 256) {
      const int i = base + 4 * lane;
      if (i < hi_i) {
        const uint4 v = k4[i >> 2];
        const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i + j < hi_i && (e[j] & mask) == prefix) atomicAdd(&sh.hist[(e[j] >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    // thread t owns digits 4t .. 4t+3; `above` counts keys with a higher digit than its range
    uint32_t c[4], mine = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 4 * tid + j;
      c[j] = d <= int(dmask) ? sh.hist[d] : 0u;
      mine += c[j];
    }
    // inclusive prefix over threads (thread order = digit order), then count from the top
    uint32_t inc = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t u = uint32_t(__shfl_up(int(inc), off));
      if (lane >= off) inc += u;
    }
    if (lane == 63) sh.wa[wv] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
      before += (w < wv) ? sh.wa[w] : 0u;
      total += sh.wa[w];
    }
    const uint32_t above = total - (before + inc);
    if (above < remaining && remaining <= above + mine) {
      uint32_t acc = above;
      for (int j = 3; j >= 0; --j) {
        if (acc + c[j] >= remaining) {
          sh.digit = uint32_t(4 * tid + j);
          sh.remaining = remaining - acc;
          break;
        }
        acc += c[j];
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= dmask << shift;
    remaining = sh.remaining;
    lo = shift;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = remaining;

  // compaction: per-wave counts, one exchange, then each wave emits its range in index order
  uint32_t gt = 0, eq = 0;
  for (int base = lo_i; base < hi_i; base += 64) {
    const int i = base + lane;
    const uint32_t key = i < hi_i ? sh.keys[i] : 0u;
    gt += uint32_t(__popcll(__ballot(i < hi_i && key > T)));
    eq += uint32_t(__popcll(__ballot(i < hi_i && key == T)));
  }
  if (lane == 0) {
    sh.wa[wv] = gt;
    sh.wb[wv] = eq;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w)
    if (w < wv) {
      gt_before += sh.wa[w];
      eq_before += sh.wb[w];
    }
  // kept before this wave: all greater keys plus the first need_eq equal keys in index order
  uint32_t at = gt_before + min(eq_before, need_eq);
  uint32_t eq_seen = eq_before;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int base = lo_i; base < hi_i; base += 64) {
    const int i = base + lane;
    const uint32_t key = i < hi_i ? sh.keys[i] : 0u;
    const bool is_eq = i < hi_i && key == T;
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t eq_rank = eq_seen + uint32_t(__popcll(eqm & below));
    const bool take = (i < hi_i && key > T) || (is_eq && eq_rank < need_eq);
    const uint64_t tm = __ballot(take);
    if (take) emit(int(at + uint32_t(__popcll(tm & below))), i);
    at += uint32_t(__popcll(tm));
    eq_seen += uint32_t(__popcll(eqm));
  }
  __syncthreads();
}

// Copies n fp32 scores (16-byte aligned source) into LDS as keys.  Every thread issues all of its loads before
// its first LDS store (up to 16 float4 per thread per round), so the copy costs about one memory latency per
// round instead of one per element.
__device__ __forceinline__ void tk_load_keys(TkShared& sh, const float* __restrict__ src, int n) {
  constexpr int U = 16;
  const int n4 = n >> 2;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  uint4* k4 = reinterpret_cast<uint4*>(sh.keys);
  for (int base = 0; base < n4; base += U * TK_THREADS) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i4 = base + u * TK_THREADS + int(threadIdx.x);
      v[u] = s4[min(i4, max(n4 - 1, 0))];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i4 = base + u * TK_THREADS + int(threadIdx.x);
      if (i4 < n4)
        k4[i4] = make_uint4(score_key(v[u].x), score_key(v[u].y), score_key(v[u].z), score_key(v[u].w));
    }
  }
  for (int i = 4 * n4 + int(threadIdx.x); i < n; i += TK_THREADS) sh.keys[i] = score_key(src[i]);
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

// One block per query row (rows of at most TK_MAXN pools).
__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                              const int32_t* __restrict__ q_pos, int P, int k,
                                                              int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ TkShared sh;
  const int q = blockIdx.x;
  int n_c, r, tau, b;
  tk_geometry(q_pos[q], P, k, ld, n_c, r, tau, b);
  const float* row = scores + int64_t(q) * ld;
  int32_t* out = sel + int64_t(q) * k;
  if (b >= n_c) {
    for (int p = threadIdx.x; p < n_c; p += TK_THREADS) out[p] = p;
  } else if (b > 0) {
    tk_load_keys(sh, row, n_c);
    __syncthreads();
    tk_select(sh, n_c, b, [&](int at, int i) __attribute__((always_inline)) { out[at] = i; });
  }
  tk_finish(out, n_sel, q, k, max(b, 0), r, tau);
}

// Step 1 of a long row: chunk c of row q keeps min(b, chunk length) candidates (key, pool id), ascending.
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(const float* __restrict__ scores, int64_t ld,
                                                                const int32_t* __restrict__ q_pos, int P, int k,
                                                                int n_chunks, uint32_t* __restrict__ cand_key,
                                                                int32_t* __restrict__ cand_idx) {
  __shared__ TkShared sh;
  const int q = blockIdx.x / n_chunks;
  const int c = blockIdx.x - q * n_chunks;
  int n_c, r, tau, b;
  tk_geometry(q_pos[q], P, k, ld, n_c, r, tau, b);
  const int base = c * TK_MAXN;
  const int len = min(TK_MAXN, n_c - base);
  if (len <= 0 || b <= 0) return;
  const float* row = scores + int64_t(q) * ld + base;
  const int64_t cb = (int64_t(q) * n_chunks + c) * k;
  tk_load_keys(sh, row, len);
  __syncthreads();
  if (b >= len) {
    for (int i = threadIdx.x; i < len; i += TK_THREADS) {
      cand_key[cb + i] = sh.keys[i];
      cand_idx[cb + i] = base + i;
    }
  } else {
    tk_select(sh, len, b, [&](int at, int i) __attribute__((always_inline)) {
      cand_key[cb + at] = sh.keys[i];
      cand_idx[cb + at] = base + i;
    });
  }
}

// Step 2 of a long row: the final b among the chunks' candidates, taken in chunk order (ascending ids).
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(const uint32_t* __restrict__ cand_key,
                                                                const int32_t* __restrict__ cand_idx, int64_t ld,
                                                                const int32_t* __restrict__ q_pos, int P, int k,
                                                                int n_chunks, int32_t* __restrict__ sel,
                                                                int32_t* __restrict__ n_sel) {
  __shared__ TkShared sh;
  __shared__ int cstart[TK_MAXCHUNKS + 1];
  const int q = blockIdx.x;
  int n_c, r, tau, b;
  tk_geometry(q_pos[q], P, k, ld, n_c, r, tau, b);
  int32_t* out = sel + int64_t(q) * k;
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int c = 0; c < n_chunks; ++c) {
      cstart[c] = acc;
      const int len = max(0, min(TK_MAXN, n_c - c * TK_MAXN));
      acc += min(max(b, 0), len);
    }
    cstart[n_chunks] = acc;
  }
  __syncthreads();
  const int n2 = cstart[n_chunks];
  auto cand = [&](int i) __attribute__((always_inline)) -> int64_t {  // workspace offset of candidate i
    int c = 0;
    while (c + 1 < n_chunks && cstart[c + 1] <= i) ++c;
    return (int64_t(q) * n_chunks + c) * k + (i - cstart[c]);
  };
  if (b >= n2) {
    for (int i = threadIdx.x; i < n2; i += TK_THREADS) out[i] = cand_idx[cand(i)];
  } else if (b > 0) {
    for (int i = threadIdx.x; i < n2; i += TK_THREADS) sh.keys[i] = cand_key[cand(i)];
    __syncthreads();
    tk_select(sh, n2, b, [&](int at, int i) __attribute__((always_inline)) { out[at] = cand_idx[cand(i)]; });
  }
  tk_finish(out, n_sel, q, k, max(b, 0), r, tau);
}

static int tk_chunks(int P, int max_pos) {
  const int64_t ncmax = (int64_t(max_pos) + 1) / P;
  return int((ncmax + TK_MAXN - 1) / TK_MAXN);
}

size_t topk_workspace(int P, int k, int n_q, int max_pos) {
  const int nch = tk_chunks(P, max_pos);
  if (nch <= 1) return 0;
  return size_t(n_q) * nch * k * (sizeof(uint32_t) + sizeof(int32_t));
}

kp_status launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.n_q == 0) return KP_OK;
  const int nch = tk_chunks(a.P, a.max_pos);
  if (nch <= 1) {
    topk_row_kernel<<<dim3(unsigned(a.n_q)), dim3(TK_THREADS), 0, s>>>(a.scores, a.ld, a.q_pos, a.P, a.k, a.sel,
                                                                       a.n_sel);
    return check_launch("dsa_topk_select");
  }
  if (nch > TK_MAXCHUNKS || int64_t(nch) * a.k > TK_MAXN) {
    set_error("dsa_topk_select: %d pools per row with top-%d exceeds the two-step limit", (a.max_pos + 1) / a.P,
              a.k);
    return KP_ERR_UNSUPPORTED;
  }
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(a.ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(cand_key + size_t(a.n_q) * nch * a.k);
  topk_chunk_kernel<<<dim3(unsigned(int64_t(a.n_q) * nch)), dim3(TK_THREADS), 0, s>>>(
      a.scores, a.ld, a.q_pos, a.P, a.k, nch, cand_key, cand_idx);
  kp_status st = check_launch("dsa_topk_select (chunks)");
  if (st != KP_OK) return st;
  topk_merge_kernel<<<dim3(unsigned(a.n_q)), dim3(TK_THREADS), 0, s>>>(cand_key, cand_idx, a.ld, a.q_pos, a.P, a.k,
                                                                       nch, a.sel, a.n_sel);
  return check_launch("dsa_topk_select (merge)");
}

}  // namespace kp
