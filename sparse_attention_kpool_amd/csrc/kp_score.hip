// dsa_indexer_score: scores[q, p] = sum_h w[q, h] * ReLU(q_idx[q, h, :] . pooled[seq(q), p, :]), p < n_c(q).
//
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: the indexer scores pools
// of 4 tokens.  [GLM-5.3-Flash model card, "Raw config fields"]: 32 index heads of dim 128.  The weighted ReLU
// sum is the layer specification's definition.
//
// Mapping onto the matrix cores: for one query, [32 heads x D] . [D x 32 pools] is one 32x32 MFMA tile
// (32x32x16 bf16, or 32x32x2 f32), the index heads forming M.  Lane group g of the 32x32 layout carries the
// channels [g*D/2, (g+1)*D/2), so each lane streams one contiguous half-row (128 B for bf16 D = 128) of a
// pooled key.  The epilogue is in registers: each lane holds 16 heads of one pool, weights them with ReLU,
// sums in-lane, then adds its partner lane (l ^ 32) -- one cross-lane step per pool tile.
//
// Work split: grid x = (query group) x (pool chunk).  A query group is QW consecutive queries that the caller
// says share a sequence (a prefill chunk); each pooled-key tile loaded is then reused by QW queries.  If a
// group's queries turn out to belong to different sequences, the group is processed one sequence at a time,
// so the result never depends on that promise.  Within a block, the 4 waves take interleaved 32-pool tiles.
//
// Bound: decode is HBM-bound (the pooled-key stream, 256 B per pool at D = 128 bf16 for 32 x 128 MACs, i.e.
// 32 flop/B: above the VALU ridge, so the contraction runs on MFMA); prefill (many queries per sequence) is
// MFMA-bound.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

template <class T, int D, int QW>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ pooled, const int32_t* __restrict__ bt,
                                                    int bt_stride, int log2_ppp, const T* __restrict__ q_idx,
                                                    const float* __restrict__ w, const int32_t* __restrict__ q_seq,
                                                    const int32_t* __restrict__ q_pos, int n_q, int Hi, int P,
                                                    float* __restrict__ scores, int64_t ld, int chunk_pools,
                                                    int n_chunks) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int KPL = E::kpl;
  constexpr int STEPS = D / (2 * KPL);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;  // A row (head) and B column (pool) of this lane
  const int g = lane >> 5;  // k-group: channels [g*D/2, (g+1)*D/2)
  const int grp = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x - grp * n_chunks;
  const int r0 = grp * QW;

  int seqs[QW], ncs[QW];
  unsigned pending = 0;
#pragma unroll
  for (int r = 0; r < QW; ++r) {
    const int row = r0 + r;
    if (row < n_q) {
      seqs[r] = q_seq[row];
      ncs[r] = int(min(int64_t((q_pos[row] + 1) / P), ld));  // ld bounds the row even if pos > max_pos
      pending |= 1u << r;
    } else {
      seqs[r] = -1;
      ncs[r] = 0;
    }
  }

  // index-query fragments (A operand) and the head weights of the 16 D-rows this lane holds
  F qa[QW][STEPS];
  float wv[QW][16];
#pragma unroll
  for (int r = 0; r < QW; ++r) {
    const int row = (r0 + r < n_q) ? r0 + r : 0;
    const bool hv = (n < Hi) && (r0 + r < n_q);
    const T* qp = q_idx + (int64_t(row) * Hi + (hv ? n : 0)) * D + g * (D / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) qa[r][s] = hv ? E::frag_load(qp + s * KPL) : E::frag_zero();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = 8 * (i / 4) + 4 * g + (i % 4);
      wv[r][i] = (h < Hi && r0 + r < n_q) ? w[int64_t(row) * Hi + h] : 0.f;
    }
  }

  const int p_begin = chunk * chunk_pools;
  while (pending) {
    const int lead = __builtin_ctz(pending);
    const int seq = seqs[lead];
    unsigned active = 0;
    int ncmax = 0;
#pragma unroll
    for (int r = 0; r < QW; ++r)
      if (((pending >> r) & 1u) && seqs[r] == seq) {
        active |= 1u << r;
        ncmax = max(ncmax, ncs[r]);
      }
    pending &= ~active;
    const int p_end = min(p_begin + chunk_pools, ncmax);

    for (int t0 = p_begin + wave * 32; t0 < p_end; t0 += 4 * 32) {
      const int pool = t0 + n;
      F kb[STEPS];
      if (pool < p_end) {
        const int64_t row = paged_row(bt, bt_stride, seq, pool, log2_ppp);
        const T* kp = pooled + row * D + g * (D / 2);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) kb[s] = E::frag_load(kp + s * KPL);
      } else {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) kb[s] = E::frag_zero();
      }
#pragma unroll
      for (int r = 0; r < QW; ++r) {
        if (!((active >> r) & 1u)) continue;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < STEPS; ++s) acc = mfma32(qa[r][s], kb[s], acc);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part += wv[r][i] * fmaxf(acc[i], 0.f);
        part += __shfl_xor(part, 32);
        if (g == 0 && pool < ncs[r]) scores[int64_t(r0 + r) * ld + pool] = part;
      }
    }
  }
}

template <class T, int D>
static void launch_score_t(const ScoreLaunch& a, int qw, int chunk, int n_chunks, int n_groups, hipStream_t s) {
  const dim3 grid(unsigned(int64_t(n_groups) * n_chunks)), block(256);
  if (qw == 4)
    score_kernel<T, D, 4><<<grid, block, 0, s>>>((const T*)a.pooled, a.bt, a.bt_stride, a.log2_ppp,
                                                 (const T*)a.q_idx, a.w, a.q_seq, a.q_pos, a.n_q, a.Hi, a.P,
                                                 a.scores, a.ld, chunk, n_chunks);
  else
    score_kernel<T, D, 1><<<grid, block, 0, s>>>((const T*)a.pooled, a.bt, a.bt_stride, a.log2_ppp,
                                                 (const T*)a.q_idx, a.w, a.q_seq, a.q_pos, a.n_q, a.Hi, a.P,
                                                 a.scores, a.ld, chunk, n_chunks);
}

kp_status launch_score(const ScoreLaunch& a, hipStream_t s) {
  const int64_t ncmax = (int64_t(a.max_pos) + 1) / a.P;
  if (a.n_q == 0 || ncmax == 0) return KP_OK;
  const int qw = (a.group >= 4) ? 4 : 1;
  const int64_t n_groups = (a.n_q + qw - 1) / qw;
  // pools per block: a multiple of 4 waves x 32 pools, sized for about 2048 blocks in flight
  int64_t chunk = (ncmax * n_groups + 2047) / 2048;
  chunk = ((chunk + 127) / 128) * 128;
  if (chunk < 128) chunk = 128;
  if (chunk > 4096) chunk = 4096;
  const int64_t n_chunks = (ncmax + chunk - 1) / chunk;
  if (n_groups * n_chunks > 0x7fffffff) {
    set_error("dsa_indexer_score: grid of %lld blocks is too large", (long long)(n_groups * n_chunks));
    return KP_ERR_INVALID_ARG;
  }
  if (a.dtype == KP_DTYPE_BF16) {
    if (a.D == 128) launch_score_t<bf16, 128>(a, qw, int(chunk), int(n_chunks), int(n_groups), s);
    else launch_score_t<bf16, 32>(a, qw, int(chunk), int(n_chunks), int(n_groups), s);
  } else {
    launch_score_t<float, 32>(a, qw, int(chunk), int(n_chunks), int(n_groups), s);
  }
  return check_launch("dsa_indexer_score");
}

}  // namespace kp
