// dsa_topk_select: causal top-k pools per query with the incomplete tail forced.
//
// [MAX glm5_next API page, index_kpool_always_select_tail]: the incomplete trailing pool is always visible.
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: the indexer always keeps
// the incomplete tail.  [GLM-5.3-Flash model card, "Raw config fields"]: index_topk 2048 (pools).  Ties go to
// the lower pool index (the layer's specification).
//
// Algorithm (exact, deterministic, no sort):
//   1. Radix select on order-preserving uint32 keys of the fp32 scores (-0 folded into +0): four 8-bit
//      passes from the top digit find the key T of the budget-th largest score and how many copies of T the
//      budget still needs (need_eq).  Histograms are integer LDS atomics, so the result does not depend on
//      their order.
//   2. One pass in index order keeps every pool with key > T and the first need_eq pools with key == T.  A
//      pass in index order emits the kept pool ids already ascending, which is the output format, and taking
//      the first equal keys is exactly the lower-index tie-break.
//   3. The tail pool tau (when (i+1) mod P != 0) is appended; it is larger than every complete pool id.
// One 1024-thread block per query row.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

// Exclusive count of `flag` over the block in thread order; `total` receives the block-wide count.
__device__ __forceinline__ int block_excl_count(bool flag, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  const int rank = __popcll(b & ((uint64_t(1) << lane) - 1));
  if (lane == 0) wsum[wv] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < TK_WAVES; ++k) {
    const int c = wsum[k];
    before += (k < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + rank;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                          const int32_t* __restrict__ q_pos, int P, int k,
                                                          int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ uint32_t hist[256];
  __shared__ int wsum[TK_WAVES];
  __shared__ uint32_t sh_digit, sh_remaining;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int i = q_pos[q];
  const int n_c = int(min(int64_t((i + 1) / P), ld));  // ld bounds the row even if pos > max_pos
  const int r = (i + 1) % P;
  const int tau = i / P;
  const int budget = min(k - (r ? 1 : 0), n_c);
  const float* row = scores + int64_t(q) * ld;
  int32_t* out = sel + int64_t(q) * k;

  if (budget >= n_c) {
    for (int p = tid; p < n_c; p += TK_THREADS) out[p] = p;
  } else if (budget > 0) {
    uint32_t prefix = 0, mask = 0, remaining = uint32_t(budget);
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int p = tid; p < n_c; p += TK_THREADS) {
        const uint32_t key = score_key(row[p]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // wave 0: lane l owns digits 4l..4l+3; find the digit where the count from the top reaches `remaining`
        uint32_t c[4], mine = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[4 * tid + j];
          mine += c[j];
        }
        // inclusive suffix sum over lanes (lanes above hold higher digits)
        uint32_t suf = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t v = __shfl_down(suf, off);
          if (tid + off < 64) suf += v;
        }
        const uint32_t above = suf - mine;  // count of keys with a higher digit than this lane's range
        if (above < remaining && remaining <= suf) {
          uint32_t acc = above;
          for (int j = 3; j >= 0; --j) {
            if (acc + c[j] >= remaining) {
              sh_digit = uint32_t(4 * tid + j);
              sh_remaining = remaining - acc;
              break;
            }
            acc += c[j];
          }
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      mask |= 255u << shift;
      remaining = sh_remaining;
      __syncthreads();
    }
    const uint32_t T = prefix;
    const int need_eq = int(remaining);
    int base = 0, eq_base = 0;
    for (int p0 = 0; p0 < n_c; p0 += TK_THREADS) {
      const int p = p0 + tid;
      const uint32_t key = (p < n_c) ? score_key(row[p]) : 0u;
      const bool gt = (p < n_c) && key > T;
      const bool eq = (p < n_c) && key == T;
      int eq_tot, take_tot;
      const int eq_rank = eq_base + block_excl_count(eq, wsum, eq_tot);
      const bool take = gt || (eq && eq_rank < need_eq);
      const int at = base + block_excl_count(take, wsum, take_tot);
      if (take) out[at] = p;
      base += take_tot;
      eq_base += eq_tot;
    }
  }
  const int cnt = max(budget, 0);
  if (tid == 0) {
    if (r) out[cnt] = tau;
    n_sel[q] = cnt + (r ? 1 : 0);
  }
  for (int j = cnt + (r ? 1 : 0) + tid; j < k; j += TK_THREADS) out[j] = -1;
}

size_t topk_workspace(int, int, int, int) { return 0; }

kp_status launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.n_q == 0) return KP_OK;
  topk_kernel<<<dim3(unsigned(a.n_q)), dim3(TK_THREADS), 0, s>>>(a.scores, a.ld, a.q_pos, a.P, a.k, a.sel,
                                                                 a.n_sel);
  return check_launch("dsa_topk_select");
}

}  // namespace kp
