// sparse_mla_attn: nope-only absorbed MLA of each query over the tokens of its selected pools.
//
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: attention layers are
// nope-only MLA.  [MAX glm5_next API page, mla_use_nope / build_layers()]: no rotary embedding; the latent row is
// 576 wide, its last 64 (rotary) columns all zero.  [GLM-5.3-Flash model card, "Raw config fields"]:
// kv_lora_rank 512, 64 heads.  Absorbed MLA: the key of token t is its latent row, the value its first V
// columns; the zero rotary columns add nothing to q . latent and are not read.
//
// One block of 8 waves per (query, split of its selected tokens).  Token slots are taken 32 at a time: slot j
// is token P * sel[j / P] + j % P, valid while j < P * n_sel and the token is <= the query position (the tail
// pool is cut at the query itself).  At start the block turns its split's pool ids into cache-row bases (one
// block-table lookup per pool) in LDS, so no gathered load waits on another global load.
//
// The 8 waves form a two-stage pipeline over 32-slot blocks, one barrier per block:
//   load   bf16 rows of 512 value columns (attn_dma_kernel): each wave brings four whole 1 KiB rows per block
//          straight from global memory into LDS (one wave-wide 16-byte direct load per row, no register
//          staging), three blocks in flight in a ring of four buffers whose rows are XOR-swizzled so that both
//          products read them without bank conflicts.  Other shapes (attn_kernel): every thread keeps 16-byte
//          chunks of the rows in registers four blocks ahead and writes them to a 3-deep ring of padded LDS
//          buffers.
//   S      waves 0..3 (S waves), block j: wave w owns heads 16w..16w+15 and computes S^T = C . Q^T on
//          16x16x32 bf16 MFMA (tokens = M, heads = N, channels = K); its Q fragments stay in registers.  Online
//          softmax per head with a lazy running max (raised only when a block's max exceeds it by more than
//          2^64, far inside the fp32 / bf16 exponent range), so blocks practically never rescale.  P and the
//          rescale factor go to LDS.
//   O      waves 4..7 (O waves), block j-1 at the same time: wave w owns value channels (w-4)*V/4 .. +V/4 for
//          all heads: O^T += C^T . P^T.  The C^T operand is read from the same row-major buffer with the LDS
//          transpose read (ds_read_b64_tr_b16): in each 16-lane group, lane s points at 4 channels of token
//          8g + s/4 and lane i receives channel i of those 4 tokens.
// Each SIMD runs one S wave and one O wave, so the two products overlap on the matrix core.  S waves keep Q in
// the same register bank in which O waves keep their accumulators.  Without register staging (attn_dma_kernel)
// S waves keep twelve C-fragment reads in flight ahead of their MFMAs and O waves read a block's C^T fragments
// one iteration before they multiply them, so LDS latency stays off the MFMA chains.
// A query's selection is split over several blocks when the batch is small (split s takes every n_split-th
// selected pool from the s-th on).  Splits write unnormalised partials (O, running max, running sum) that a
// second kernel merges in split order, so results are deterministic.
//
// Bound: HBM (the gather of 1 KiB of bf16 value columns per token feeds 2 x 64 heads x 512 MACs: 128 flop/B,
// between the VALU and MFMA ridges, hence MFMA for both products).
#include <mutex>
#include <type_traits>

#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int AT_NT = 32;         // token slots per block
constexpr int AT_THREADS = 512;   // 4 S waves + 4 O waves
constexpr int AT_DEPTH = 4;       // blocks in flight from HBM (register-staged)
constexpr int AT_MAXSLOT = 8192 + 128;  // token slots of one split held in the LDS slot table (k pools + 1)
constexpr float LN2 = 0.69314718055994530942f;
// log2 headroom before the running max is raised: weights up to 2^64 stay far inside the fp32 / bf16 exponent
// range, so the accumulators are rescaled only when a later block's max beats the running one by 2^64.
constexpr float LAZY_MAX = 64.f;

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <class T, int V, int HT>
struct AttnShape {
  static constexpr int KPL = Elem<T>::kpl;
  static constexpr int EPC = 16 / int(sizeof(T));                     // elements per 16-byte chunk
  static constexpr int CPR = V / EPC;                                 // chunks per value row
  static constexpr int CHUNKS = AT_NT * CPR;                          // chunks per block
  static constexpr int CHT = (CHUNKS + AT_THREADS - 1) / AT_THREADS;  // chunks per thread per block
  static constexpr bool SWZ = sizeof(T) == 2 && CPR % 64 == 0;       // XOR-swizzled rows (see attn_swz)
  static constexpr int RS = SWZ ? V : V + EPC;                        // LDS row stride (else +16 B against conflicts)
  static constexpr int PS = AT_NT + EPC;                              // P row stride
  static constexpr int VW = V / 4;                                    // value channels per O wave
  static constexpr int MT = VW / 16;                                  // 16-channel tiles per O wave
  static constexpr int SK = V / (4 * KPL);                            // k-steps of the S product (K = V)
  static constexpr int OK = AT_NT / (4 * KPL);                        // k-steps of the O product (K = 32 tokens)
  static constexpr int QB = (SK * KPL * int(sizeof(T))) / 16;         // 16-byte units of one wave's Q fragments
  static constexpr int NB = (MT * HT > QB) ? MT * HT : QB;            // shared register bank (f32x4 units)
  static_assert(VW % 16 == 0, "value width must split into 16-channel tiles per O wave");
  static_assert((SK * KPL * int(sizeof(T))) % 16 == 0, "Q fragments fill whole 16-byte units");
};

// Position of chunk c in LDS row r of a swizzled block: c ^ attn_swz(r), with the permutation
// pi(r) = 2 (r mod 4) + 8 ((r >> 3) mod 2) + ((r >> 2) mod 2) of the row's last four bits.  Sixteen consecutive rows
// then put one chunk on sixteen distinct 4-bank groups (the S product's 16-byte reads), and the rows {0..3, 8..11}
// (or {4..7, 12..15}) that one half-wave's transposed 8-byte reads touch put an aligned 32-byte window on eight
// distinct 8-bank groups (the O product): both conflict-free in a 64-bank LDS, without padding.  With 1 KiB rows
// in 256-byte aligned buffers, each read address is a per-lane base XOR a constant.
__device__ __forceinline__ int attn_swz(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1) + ((r >> 2) & 1); }

// Two LDS transpose reads (ds_read_b64_tr_b16) joined into one 8-element MFMA fragment
__device__ __forceinline__ bf16x8 lds_tr_pair(uint32_t o1, uint32_t o2) {
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t(o1)));
  const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t(o2)));
  const uint2 u1 = __builtin_bit_cast(uint2, v1), u2 = __builtin_bit_cast(uint2, v2);
  return __builtin_bit_cast(bf16x8, make_uint4(u1.x, u1.y, u2.x, u2.y));
}

// 1 KiB of zeros: the source row of a slot with no token (past the split or past the query), so the O product
// multiplies its zero weight by zeros, never by whatever a cache row holds
__device__ __align__(16) uint32_t attn_zero_row[256];

// Pools a query attends from its selection row: the row's first n_row entries (n_row = min(n_sel, k), so a count
// beyond the row is never trusted) and, for a query that reads another query's row (an MTP draft sharing its
// target's selection), its own trailing pool tau = pos / P when that pool is incomplete ((pos + 1) mod P != 0) and
// the row lacks it.  The shared item is the target's top-k pick; the incomplete tail is not a pick but is always
// visible, so a draft always sees its own pending tokens -- itself included.  Returns the entry count; entry
// n_row, when present, is `extra`.  With `shared` set every thread of the block must call it (one barrier), as
// attn_own_tail (that tail pool, or -1 when the row holds it or it is complete).
__device__ __forceinline__ int attn_own_tail(const int32_t* __restrict__ row, int n_row, int pos, int log2P) {
  const int tau = pos >> log2P;
  int has = 0;
  for (int j = threadIdx.x; j < n_row; j += blockDim.x) has |= row[j] == tau ? 1 : 0;
  has = __syncthreads_or(has);
  return (has == 0 && ((pos + 1) & ((1 << log2P) - 1)) != 0) ? tau : -1;
}
__device__ __forceinline__ int attn_row_pools(const int32_t* __restrict__ row, int n_row, bool shared, int pos,
                                              int log2P, int& extra) {
  extra = shared ? attn_own_tail(row, n_row, pos, log2P) : -1;
  return n_row + (extra >= 0 ? 1 : 0);
}

// A-operand fragment of C^T (channels c0 .. c0+15 x tokens 8g .. 8g+7 of k-step s) from the row-major block.
template <class T, int RS>
__device__ __forceinline__ typename Elem<T>::frag ct_frag(const T* blk, int c0, int g, int l16, int s) {
  if constexpr (sizeof(T) == 2) {
    const int e = l16 >> 2, a = l16 & 3;
    const T* p1 = blk + (8 * g + e) * RS + c0 + 4 * a;   // tokens 8g .. 8g+3
    const T* p2 = p1 + 4 * RS;                           // tokens 8g+4 .. 8g+7
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p1));
    const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p2));
    const uint2 u1 = __builtin_bit_cast(uint2, v1), u2 = __builtin_bit_cast(uint2, v2);
    return __builtin_bit_cast(bf16x8, make_uint4(u1.x, u1.y, u2.x, u2.y));
  } else {
    return blk[(8 * g + s) * RS + c0 + l16];
  }
}

// O-wave epilogue: the output of the wave's channels for every head -- normalised (one split) or as an
// unnormalised partial with its running max and sum (several splits).  The accumulated O is multiplied by oscale
// on the way out (the scale of an fp8 latent cache; 1 otherwise).
template <class T, int V, int HT>
__device__ __forceinline__ void attn_write_out(const f32x4 (&bank)[AttnShape<T, V, HT>::NB], int qi, int sp,
                                               int n_split, int H, int wl, int l16, int g, const float* m_s,
                                               const float* l_s, T* __restrict__ out, float* __restrict__ lse,
                                               T* __restrict__ part_o, float* __restrict__ part_ml,
                                               float oscale = 1.f) {
  using S = AttnShape<T, V, HT>;
#pragma unroll
  for (int nt = 0; nt < HT; ++nt) {
    const int h = 16 * nt + l16;
    if (h >= H) continue;
    const float mh = m_s[h], lh = l_s[h];
    if (n_split == 1) {
      const float inv = oscale / lh;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const f32x4 o = bank[mt * HT + nt] * inv;
        T* op = out + (int64_t(qi) * H + h) * V + wl * S::VW + 16 * mt + 4 * g;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        } else {
          *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
      if (lse && wl == 0 && g == 0) lse[int64_t(qi) * H + h] = (mh + log2f(lh)) * LN2;
    } else {
      const int64_t base = int64_t(qi * n_split + sp) * H + h;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const f32x4 o = bank[mt * HT + nt] * oscale;
        T* pp = part_o + base * V + wl * S::VW + 16 * mt + 4 * g;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(pp) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        } else {
          *reinterpret_cast<float4*>(pp) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
      if (wl == 0 && g == 0) {
        part_ml[base * 2 + 0] = mh;
        part_ml[base * 2 + 1] = lh;
      }
    }
  }
}

template <class T, int V, int HT>
__global__ __launch_bounds__(AT_THREADS) void attn_kernel(
    const T* __restrict__ latent, int L, const int32_t* __restrict__ bt, int bt_stride, int log2_pt,
    const T* __restrict__ q, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, const int32_t* __restrict__ sel_row,
    int log2P, int k, int H, float scale_log2,
    int n_split, T* __restrict__ out, float* __restrict__ lse, T* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using S = AttnShape<T, V, HT>;
  using E = Elem<T>;
  using F = typename E::frag;
  __shared__ __align__(16) T crm[3][AT_NT * S::RS];
  __shared__ __align__(16) T ps[2][16 * HT * S::PS];
  __shared__ int32_t slot_tab[AT_MAXSLOT];
  __shared__ float alpha_s[2][64];
  __shared__ uint32_t resc_s[2];
  __shared__ float m_s[64];
  __shared__ float l_s[64];
  __shared__ uint32_t vmask_s[3];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const bool o_wave = wave >= 4;
  const int wl = wave & 3;  // index within the wave's role
  const int qi = blockIdx.x / n_split;
  const int srow = sel_row ? sel_row[qi] : qi;  // the selection row this query attends (shared by MTP drafts)
  const int sp = blockIdx.x - qi * n_split;
  const int seq = q_seq[qi];
  const int pos = q_pos[qi];
  const int P = 1 << log2P;
  // Split sp takes the selected pools sp, sp + n_split, sp + 2 n_split, ...: interleaved rather than
  // contiguous, so the blocks of one query read spread-out parts of its (ascending) selection at a time.
  const int n_row = min(n_sel[srow], k);
  int extra;
  const int ns_pools = attn_row_pools(sel + int64_t(srow) * k, n_row, sel_row != nullptr, pos, log2P, extra);
  const int my_pools = ns_pools > sp ? (ns_pools - sp + n_split - 1) / n_split : 0;
  const int s_begin = 0;
  const int s_end = my_pools * P;

  if (s_begin >= s_end) {  // an empty split (this query selected fewer tokens)
    if (n_split > 1) {
      for (int h = tid; h < H; h += AT_THREADS) {
        part_ml[(int64_t(qi * n_split + sp) * H + h) * 2 + 0] = -INFINITY;
        part_ml[(int64_t(qi * n_split + sp) * H + h) * 2 + 1] = 0.f;
      }
    } else {
      for (int64_t e = tid; e < int64_t(H) * V; e += AT_THREADS) out[int64_t(qi) * H * V + e] = E::from_f32(0.f);
      if (lse)
        for (int h = tid; h < H; h += AT_THREADS) lse[int64_t(qi) * H + h] = -INFINITY;
    }
    return;
  }
  const int nsl = s_end - s_begin;  // slots of this split (a whole number of pools)
  const int nblk = (nsl + AT_NT - 1) / AT_NT;

  // Slot table: cache row of every slot of the split, -1 for a slot past the query (the cut tail pool).  One
  // block-table lookup per pool, done once; in the loop a slot's row is then a single LDS read.
  {
    const int32_t* qsel = sel + int64_t(srow) * k + sp;
    const int pt_mask = (1 << log2_pt) - 1;
    for (int j = tid; j < (nsl >> log2P); j += AT_THREADS) {
      const int gj = sp + j * n_split;  // entry of the row
      const int p = gj < n_row ? qsel[int64_t(j) * n_split] : extra;
      int nt = 0, row = 0;
      if (p >= 0) {
        const int first = p << log2P;
        nt = min(P, pos - first + 1);
        if (nt > 0) row = bt[int64_t(seq) * bt_stride + (first >> log2_pt)] * (pt_mask + 1) + (first & pt_mask);
      }
      for (int w = 0; w < P; ++w) slot_tab[(j << log2P) + w] = w < nt ? row + w : -1;
    }
  }

  // Register bank: an S wave keeps the Q^T fragments of its 16 heads there (B operand of S^T = C . Q^T; lane
  // holds head 16*wl + l16, channels g*(V/4) + s*KPL .. +KPL for k-step s); an O wave keeps its accumulators
  // O^T[16 channels x 16 heads] tiles at bank[mt * HT + nt].
  f32x4 bank[S::NB];
#pragma unroll
  for (int b = 0; b < S::NB; ++b) bank[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool s_active = !o_wave && wl < HT;
  if (s_active) {
    const int h = 16 * wl + l16;
    const bool hv = h < H;
    const T* qp = q + (int64_t(qi) * H + (hv ? h : 0)) * L + g * (V / 4);
    if (hv) {
#pragma unroll
      for (int s = 0; s < S::SK; ++s) {
        if constexpr (sizeof(T) == 2) bank[s] = __builtin_bit_cast(f32x4, E::frag_load(qp + s * S::KPL));
        else bank[s >> 2][s & 3] = qp[s];
      }
    }
  }
  auto qfrag = [&](int s) __attribute__((always_inline)) -> F {
    if constexpr (sizeof(T) == 2) return __builtin_bit_cast(bf16x8, bank[s]);
    else return bank[s >> 2][s & 3];
  };
  // S waves: running max of the lane's head (the same in all four lanes of a head) and the lane's own part of
  // the running sum (its 8 slots of each block; the four parts are added once at the end)
  float m_run = -INFINITY, l_run = 0.f;

  __syncthreads();  // slot table ready

  // table entry of slot t (0..31) of block b: its cache row, or -1 (past the split or past the query)
  auto slot_entry = [&](int b, int t) __attribute__((always_inline)) -> int {
    const int rel = b * AT_NT + t;
    const int e = slot_tab[min(rel, AT_MAXSLOT - 1)];
    return rel < nsl ? e : -1;
  };

  // Slot (row of the block) of a thread's i-th chunk c: with one value row per wave instruction, wave w takes
  // the CHT consecutive slots w*CHT .. (w+1)*CHT-1 (one whole pool at P = CHT = 4); otherwise c / CPR.
  auto slot_of = [&](int c, int i) __attribute__((always_inline)) -> int {
    if constexpr (S::CPR == 64 && S::CHUNKS % AT_THREADS == 0) return (tid >> 6) * S::CHT + i;
    else return c / S::CPR;
  };

  // Loads are unconditional (an invalid slot reads row 0 of the cache and is zeroed when stored): branch-free
  // loads let the compiler wait for exactly the block it needs instead of draining every load in flight.  With
  // one whole value row per wave instruction the row is wave-uniform and its address is computed on the
  // scalar unit.
  auto load_block = [&](int b, u32x4(&R)[S::CHT], bool(&vrow)[S::CHT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::CHT; ++i) {
      if constexpr (S::CPR == 64 && S::CHUNKS % AT_THREADS == 0) {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const int e = __builtin_amdgcn_readfirstlane(slot_entry(b, wv * S::CHT + i));
        const T* rp = latent + int64_t(max(e, 0)) * L;
        R[i] = *reinterpret_cast<const u32x4*>(rp + lane * S::EPC);
        vrow[i] = e >= 0;
      } else {
        const int c = min(tid + AT_THREADS * i, S::CHUNKS - 1);
        const int e = slot_entry(b, c / S::CPR);
        R[i] = *reinterpret_cast<const u32x4*>(latent + int64_t(max(e, 0)) * L + (c % S::CPR) * S::EPC);
        vrow[i] = e >= 0;
      }
    }
  };

  auto s_phase = [&](int j) __attribute__((always_inline)) {
    const T* blk = crm[j % 3];
    f32x4 sa[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sa[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sa[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* ap = blk + (16 * t + l16) * S::RS + g * (V / 4);
#pragma unroll
      for (int s = 0; s < S::SK; ++s) sa[t][s & 1] = mfma16(E::frag_load(ap + s * S::KPL), qfrag(s), sa[t][s & 1]);
    }
    // lane holds head 16*wl + l16, slots 16t + 4g + i
    const uint32_t vm = vmask_s[j % 3];
    float x[2][4];
    float lmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 16 * t + 4 * g + i;
        x[t][i] = ((vm >> slot) & 1u) ? (sa[t][0][i] + sa[t][1][i]) * scale_log2 : -INFINITY;
        lmax = fmaxf(lmax, x[t][i]);
      }
    // The running max is raised only for a head whose block max beats it by more than LAZY_MAX; no lane over
    // that bound means no head is raised, so the cross-lane max is needed only on the (rare) raising blocks.
    float alpha = 1.f;
    const bool raise = __ballot(lmax > m_run + LAZY_MAX) != 0;
    if (raise) {
      float bmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = (bmax > m_run + LAZY_MAX) ? bmax : m_run;
      alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      if (g == 0) alpha_s[j & 1][16 * wl + l16] = alpha;
    }
    float rsum = 0.f;
    float pv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[t][i] = (x[t][i] == -INFINITY) ? 0.f : fast_exp2(x[t][i] - m_run);
        rsum += pv[t][i];
      }
    l_run = l_run * alpha + rsum;
    T* prow = ps[j & 1] + (16 * wl + l16) * S::PS;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(prow + 16 * t + 4 * g) =
            make_uint2(pack_bf16x2(pv[t][0], pv[t][1]), pack_bf16x2(pv[t][2], pv[t][3]));
      } else {
        *reinterpret_cast<float4*>(prow + 16 * t + 4 * g) = make_float4(pv[t][0], pv[t][1], pv[t][2], pv[t][3]);
      }
    }
    if (lane == 0) reinterpret_cast<uint8_t*>(&resc_s[j & 1])[wl] = raise ? 1 : 0;
  };

  auto o_phase = [&](int j) __attribute__((always_inline)) {
    const T* blk = crm[j % 3];
    const T* pb = ps[j & 1];
    // rescale only the head tiles whose running max moved
    const uint32_t rf = resc_s[j & 1];
    if (rf) {
#pragma unroll
      for (int nt = 0; nt < HT; ++nt) {
        if ((rf >> (8 * nt)) & 0xffu) {
          const float a = alpha_s[j & 1][16 * nt + l16];
#pragma unroll
          for (int mt = 0; mt < S::MT; ++mt) bank[mt * HT + nt] *= a;
        }
      }
    }
    // O^T[channels of this wave][heads] += C^T . P^T; k-slot (group g, step s, element e) = token 8g + s*KPL + e
#pragma unroll
    for (int s = 0; s < S::OK; ++s) {
      F bq[HT];
#pragma unroll
      for (int nt = 0; nt < HT; ++nt) bq[nt] = E::frag_load(pb + (16 * nt + l16) * S::PS + 8 * g + s * S::KPL);
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const F av = ct_frag<T, S::RS>(blk, wl * S::VW + 16 * mt, g, l16, s);
#pragma unroll
        for (int nt = 0; nt < HT; ++nt) bank[mt * HT + nt] = mfma16(av, bq[nt], bank[mt * HT + nt]);
      }
    }
  };

  // iteration j: store block j into the ring, start loading block j+AT_DEPTH, then S(j) on S waves and O(j-1) on
  // O waves.  Buffer j % 3 was last read by O(j-3) in iteration j-2, two barriers ago.
  // Stores and loads are unconditional, also for blocks past the end (all slots invalid: zeros are stored,
  // row 0 is read): with no load or store under a branch the compiler's wait counts stay exact, and a wave
  // waits only for the block it stores, never for the one loaded after it.
  auto iter = [&](int j, u32x4(&R)[S::CHT], bool(&vrow)[S::CHT]) __attribute__((always_inline)) {
    T* blk = crm[j % 3];
#pragma unroll
    for (int i = 0; i < S::CHT; ++i) {
      const int c = tid + AT_THREADS * i;
      if (S::CHUNKS % AT_THREADS == 0 || c < S::CHUNKS)
        *reinterpret_cast<u32x4*>(blk + slot_of(c, i) * S::RS + (c % S::CPR) * S::EPC) =
            vrow[i] ? R[i] : u32x4{0, 0, 0, 0};
    }
    if (wave == 0) {
      const uint32_t vm = uint32_t(__ballot(lane < AT_NT && slot_entry(j, lane & (AT_NT - 1)) >= 0));
      if (lane == 0) vmask_s[j % 3] = vm;
    }
    load_block(j + AT_DEPTH, R, vrow);
    __syncthreads();
    if (o_wave) {
      if (j >= 1 && j - 1 < nblk) o_phase(j - 1);
    } else if (s_active && j < nblk) {
      s_phase(j);
    }
  };

  u32x4 R[AT_DEPTH][S::CHT];
  bool vr[AT_DEPTH][S::CHT];
#pragma unroll
  for (int d = 0; d < AT_DEPTH; ++d) load_block(d, R[d], vr[d]);
  // iterations 0 .. nblk (the last one runs O of block nblk - 1), in whole rounds of AT_DEPTH: the up to
  // AT_DEPTH - 1 iterations past nblk compute nothing and only re-read row 0
  for (int j = 0; j <= nblk; j += AT_DEPTH) {
#pragma unroll
    for (int d = 0; d < AT_DEPTH; ++d) iter(j + d, R[d], vr[d]);
  }

  if (s_active) {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (g == 0) {
      m_s[16 * wl + l16] = m_run;
      l_s[16 * wl + l16] = l_run;
    }
  }
  __syncthreads();
  if (!o_wave) return;
  attn_write_out<T, V, HT>(bank, qi, sp, n_split, H, wl, l16, g, m_s, l_s, out, lse, part_o, part_ml);
}

// ---------------------------------------------------------------------------------------------------------------
// bf16 latent rows of V = 512 value columns: the same split, slots and two-role pipeline as attn_kernel, with the
// value rows going straight from global memory into LDS (one wave-wide 16-byte direct load per 1 KiB row, no
// register staging), three blocks in flight in a ring of four swizzled 32 KiB buffers.  The registers this frees
// let the S waves keep twelve C-fragment reads in flight ahead of their MFMAs, and the O waves read a block's C^T
// fragments one iteration before they multiply them.
// ---------------------------------------------------------------------------------------------------------------
constexpr int AD_NBUF = 4;        // LDS block buffers: blocks j .. j + 2 land or are read, j + 3 is refilled
constexpr int AD_MAXPOOL = 2048 + 16;  // pools of one split held in the LDS pool table (k pools + 1)
constexpr int AD_DIST = 12;       // S waves: C-fragment reads in flight ahead of the MFMAs

// FP8: the latent cache holds OCP E4M3 codes (1 byte per element; value = code value * its scale).  Then every wave
// loads its 4 rows (512 B each, one 1 KiB wave load per 2 rows) of each block into registers three blocks ahead,
// converts every code to bf16 once -- exactly: E4M3 values are bf16 values -- and writes the same swizzled bf16
// block the direct loads produce, two blocks ahead of the S phase, so the S and O phases are unchanged.  The cache
// scale is folded into the softmax scale and applied to O on the way out.
//
// MTP (verification runs): queries come in runs of two consecutive entries -- a target and its draft -- that attend
// selection row `run` (one row per run), each cut at its own position plus its own incomplete trailing pool when
// the row lacks it (see attn_own_tail).  A block takes (run, split, head half hb): its 64 score / output rows are 32
// heads (hb * 32 ..) of each of the two queries -- S waves 0, 1 the target's, 2, 3 the draft's -- over ONE list of
// gathered rows: the row's pools and the queries' added tails, each row with one validity mask per query.  When
// the two queries belong to different sequences the list is the two queries' pools one after the other (each row
// attended by one query only).  The two head-half blocks of a (run, split) are launched 8 apart, so they run on
// one XCD at about the same time and the second reads each row from that XCD's L2.
template <int HT, bool FP8, bool MTP = false>
__global__ __launch_bounds__(AT_THREADS) void attn_dma_kernel(
    const void* __restrict__ latent_v, int L, const int32_t* __restrict__ bt, int bt_stride, int log2_pt,
    const bf16* __restrict__ q, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, const int32_t* __restrict__ sel_row,
    int log2P, int k, int H, float scale_log2,
    int n_split, bf16* __restrict__ out, float* __restrict__ lse, bf16* __restrict__ part_o,
    float* __restrict__ part_ml, float oscale, int n_q) {
  static_assert(!MTP || (!FP8 && HT == 4), "MTP runs: bf16 latent rows, 64 score rows per block");
  using T = bf16;
  // S waves: C-fragment reads in flight ahead of the MFMAs (fewer with fp8: the staging registers take the rest)
  constexpr int DIST = FP8 ? 6 : AD_DIST;
  const bf16* latent = static_cast<const bf16*>(latent_v);
  const uint8_t* latent8 = static_cast<const uint8_t*>(latent_v);
  constexpr int V = 512;
  using S = AttnShape<T, V, HT>;
  using E = Elem<T>;
  using F = typename E::frag;
  static_assert(S::SWZ && S::RS == V && S::CPR == 64 && S::CHUNKS == 4 * AT_THREADS && S::OK == 1,
                "one 1 KiB swizzled row per wave instruction, four rows per wave and block");
  __shared__ __align__(1024) T crm[AD_NBUF][AT_NT * V];
  __shared__ __align__(16) T ps[2][16 * HT * S::PS];
  __shared__ int32_t prow_s[AD_MAXPOOL];  // cache row of each pool's first token
  __shared__ uint8_t pnt_s[AD_MAXPOOL];   // tokens of the pool at or before the query (0: none)
  __shared__ float alpha_s[2][64];
  __shared__ uint32_t resc_s[2];
  __shared__ float m_s[64];
  __shared__ float l_s[64];
  __shared__ uint32_t vmask_s[MTP ? 2 : 1][AT_MAXSLOT / AT_NT];  // valid-slot mask of every block, per query

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same value, known to be wave-uniform
  const int l16 = lane & 15, g = lane >> 4;
  const bool o_wave = wave >= 4;
  const int wl = wave & 3;  // index within the wave's role
  const int P = 1 << log2P;
  int qi, sp, hb = 0, srow;
  if constexpr (MTP) {
    // block b: unit u = run * n_split + split, head half hb; units go 8 to a group, a group's head halves 8 apart
    const int nhb = (H + 31) >> 5;
    const int per = 8 * nhb, b = int(blockIdx.x);
    const int u = (b / per) * 8 + (b % per) % 8;
    hb = (b % per) / 8;
    if (u >= ((n_q + 1) >> 1) * n_split) return;  // launch padding: the whole block leaves before any barrier
    srow = u / n_split;
    sp = u - srow * n_split;
    qi = 2 * srow;
  } else {
    qi = blockIdx.x / n_split;
    sp = blockIdx.x - qi * n_split;
    srow = sel_row ? sel_row[qi] : qi;  // the selection row this query attends (shared by MTP drafts)
  }
  const int seq = q_seq[qi];
  const int pos = q_pos[qi];
  // the run's draft (MTP), when present
  const bool has_b = MTP && qi + 1 < n_q;
  const int seq_b = has_b ? q_seq[qi + 1] : seq;
  const int pos_b = has_b ? q_pos[qi + 1] : -1;
  // split sp takes the entries sp, sp + n_split, sp + 2 n_split, ... of the pool list (as attn_kernel)
  // The first selection entry of each thread is loaded right away, with the selection count rather than after
  // it (an entry past the count is read but not used; every index stays inside the row of k entries).
  const int32_t* rowp = sel + int64_t(srow) * k;
  const int32_t* qsel = rowp + sp;
  const int kq = (k - sp + n_split - 1) / n_split;  // entries of the row this split strides over
  const int p_first = tid < kq ? qsel[int64_t(tid) * n_split] : -1;
  const int n_row = min(n_sel[srow], k);
  // Pool list: the row's n_row pools and the added tails.  One query: entry n_row is `extra` when present.  MTP
  // (tail_a, tail_b: each query's own added tail, or -1): one sequence -- the row, then tail_a, then tail_b unless
  // it is the same pool (ex_b); two sequences -- the target's row and tail_a (n_a entries), then the draft's row
  // and tail_b.
  int extra = -1, tail_a = -1, tail_b = -1, ex_b = -1, n_a = 0, ns_pools;
  bool one_seq = true;
  if constexpr (MTP) {
    tail_a = attn_own_tail(rowp, n_row, pos, log2P);
    if (has_b) tail_b = attn_own_tail(rowp, n_row, pos_b, log2P);
    one_seq = !has_b || seq_b == seq;
    n_a = n_row + (tail_a >= 0 ? 1 : 0);
    if (one_seq) {
      ex_b = tail_b != tail_a ? tail_b : -1;
      ns_pools = n_a + (ex_b >= 0 ? 1 : 0);
    } else {
      ns_pools = n_a + n_row + (tail_b >= 0 ? 1 : 0);
    }
  } else {
    ns_pools = attn_row_pools(rowp, n_row, sel_row != nullptr, pos, log2P, extra);
  }
  const int my_pools = ns_pools > sp ? (ns_pools - sp + n_split - 1) / n_split : 0;
  const int nsl = my_pools * P;  // slots of this split

  // Output row r of the block (0 .. 63): query and head, and whether it exists.  One query: row r is head r.  MTP:
  // rows 0 .. 31 are heads hb * 32 .. of the target, rows 32 .. 63 the same heads of the draft.
  auto row_dest = [&](int r, int& qd, int& hd) __attribute__((always_inline)) -> bool {
    if constexpr (MTP) {
      qd = qi + (r >> 5);
      hd = hb * 32 + (r & 31);
      return hd < H && (r < 32 || has_b);
    } else {
      qd = qi;
      hd = r;
      return r < H;
    }
  };
  constexpr int NROW = MTP ? 64 : 16 * HT;  // output rows of the block (rows past H are never written)

  if (nsl == 0) {  // an empty split (these queries selected fewer tokens)
    for (int r = tid; r < NROW; r += AT_THREADS) {
      int qd, hd;
      if (!row_dest(r, qd, hd)) continue;
      if (n_split > 1) {
        part_ml[(int64_t(qd * n_split + sp) * H + hd) * 2 + 0] = -INFINITY;
        part_ml[(int64_t(qd * n_split + sp) * H + hd) * 2 + 1] = 0.f;
      } else if (lse) {
        lse[int64_t(qd) * H + hd] = -INFINITY;
      }
    }
    if (n_split == 1) {
      for (int i = tid; i < NROW * (V / 8); i += AT_THREADS) {
        int qd, hd;
        if (!row_dest(i / (V / 8), qd, hd)) continue;
        *reinterpret_cast<u32x4*>(out + (int64_t(qd) * H + hd) * V + (i % (V / 8)) * 8) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }
  const int nblk = (nsl + AT_NT - 1) / AT_NT;

  // Register bank, as in attn_kernel: Q^T fragments on an S wave (bank[0 .. QB)), accumulators on an O wave.  The
  // Q loads go out before the pool table's dependent ones.
  f32x4 bank[S::NB];
#pragma unroll
  for (int b = 0; b < S::NB; ++b) bank[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // S wave wl: query s_q, heads s_h = 16 wl + l16 (MTP: waves 0, 1 the target's heads hb * 32 .., 2, 3 the draft's)
  const int s_member = MTP ? (wl >> 1) : 0;
  const int s_q = qi + s_member;
  const int s_h = MTP ? hb * 32 + 16 * (wl & 1) + l16 : 16 * wl + l16;
  const bool s_active = !o_wave && (MTP ? (s_member == 0 || has_b) : wl < HT);
  if (s_active) {
    if (s_h < H) {
      const T* qp = q + (int64_t(s_q) * H + s_h) * L + g * (V / 4);
#pragma unroll
      for (int s = 0; s < S::SK; ++s) bank[s] = __builtin_bit_cast(f32x4, E::frag_load(qp + s * S::KPL));
    }
  }
  // Pool table: cache row of every pool's first token and how many of its tokens the query sees (the tail pool is
  // cut at the query), one block-table lookup per pool; and the valid-slot mask of every block, OR-ed over the
  // 32 / P consecutive lanes that hold the block's pools (no LDS round trip).  MTP: a pool counts the tokens that
  // either query sees (the rows the block loads), and each query has its own mask.
  {
    const int pt_mask = (1 << log2_pt) - 1;
    const int ppb = AT_NT >> log2P;  // pools per block (P <= 32)
    for (int j0 = 0; j0 < my_pools; j0 += AT_THREADS) {
      const int j = j0 + tid;
      const bool valid = j < my_pools;
      const int gj = sp + j * n_split;  // entry of the pool list
      int p = -1, eseq = seq;
      bool att_a = true, att_b = false;  // which queries attend the entry
      auto row_entry = [&](int e) __attribute__((always_inline)) {
        return (j0 == 0 && e == gj) ? p_first : rowp[e];
      };
      if constexpr (MTP) {
        if (valid) {
          if (one_seq) {
            if (gj < n_row) {
              p = row_entry(gj);
              att_b = has_b;
            } else {
              p = (gj == n_row && tail_a >= 0) ? tail_a : ex_b;
              att_a = p == tail_a;
              att_b = has_b && p == tail_b;
            }
          } else if (gj < n_a) {
            p = gj < n_row ? row_entry(gj) : tail_a;
          } else {
            const int e2 = gj - n_a;
            p = e2 < n_row ? rowp[e2] : tail_b;
            eseq = seq_b;
            att_a = false;
            att_b = true;
          }
        }
      } else {
        p = gj >= n_row ? (valid ? extra : -1) : j0 == 0 ? p_first : qsel[int64_t(j) * n_split];
      }
      int nt = 0, nt_b = 0, row = 0;
      if (valid && p >= 0) {
        const int first = p << log2P;
        if (att_a) nt = max(min(P, pos - first + 1), 0);
        if (att_b) nt_b = max(min(P, pos_b - first + 1), 0);
        if (max(nt, nt_b) > 0)
          row = bt[int64_t(eseq) * bt_stride + (first >> log2_pt)] * (pt_mask + 1) + (first & pt_mask);
      }
      if (valid) {
        prow_s[j] = row;
        pnt_s[j] = uint8_t(max(nt, nt_b));
      }
      uint32_t bits = (nt >= 32 ? 0xffffffffu : (1u << nt) - 1u) << ((j & (ppb - 1)) << log2P);
      for (int o = 1; o < ppb; o <<= 1) bits |= uint32_t(__shfl_xor(int(bits), o));
      if (valid && (j & (ppb - 1)) == 0) vmask_s[0][j / ppb] = bits;
      if constexpr (MTP) {
        uint32_t bb = (nt_b >= 32 ? 0xffffffffu : (1u << nt_b) - 1u) << ((j & (ppb - 1)) << log2P);
        for (int o = 1; o < ppb; o <<= 1) bb |= uint32_t(__shfl_xor(int(bb), o));
        if (valid && (j & (ppb - 1)) == 0) vmask_s[1][j / ppb] = bb;
      }
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();  // pool table and masks ready

  // cache row of slot t (0..31) of block b, or -1 (past the split or past the query)
  auto slot_entry = [&](int b, int t) __attribute__((always_inline)) -> int {
    const int rel = b * AT_NT + t;
    const int pool = min(rel >> log2P, AD_MAXPOOL - 1), w = rel & (P - 1);
    return (rel < nsl && w < int(pnt_s[pool])) ? prow_s[pool] + w : -1;
  };
  __builtin_amdgcn_s_waitcnt(0);  // every prologue load is in: only block loads are in flight from here
  // rows of the slots this wave loads for block b, one per lane (lane i < CHT: slot CHT w + i), read a whole
  // iteration before their loads so the table lookups never delay them
  auto block_rows = [&](int b) __attribute__((always_inline)) -> int {
    return slot_entry(b, wave_u * S::CHT + (lane & (S::CHT - 1)));
  };
  // Block b into buffer b % 4: wave w brings slots 4w .. 4w+3, one row per instruction; lane l takes chunk
  // l ^ attn_swz(slot) of the row, so LDS position l holds it (see attn_swz).  An invalid slot reads the zero row.
  auto load_block = [&](int b, int rows) __attribute__((always_inline)) {
    const uint32_t base = lds_off(crm[b % AD_NBUF]);
#pragma unroll
    for (int i = 0; i < S::CHT; ++i) {
      const int slot = wave_u * S::CHT + i;
      const int e = __builtin_amdgcn_readlane(rows, i);
      const int c = lane ^ attn_swz(slot);
      const void* src = e >= 0 ? static_cast<const void*>(latent + int64_t(e) * L + c * S::EPC)
                               : static_cast<const void*>(attn_zero_row + 4 * lane);
      lds_dma16(src, base + uint32_t(slot * V * int(sizeof(T))));
    }
  };

  auto s_phase = [&](int j) __attribute__((always_inline)) {
    const T* blk = crm[j % AD_NBUF];
    f32x4 sa[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) sa[t][0] = sa[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragment f = t * SK + s: row 16t + l16, chunk g * CPR/4 + s, at byte (row base + g * CPR/4 * 16 +
    // 16 attn_swz(l16)) ^ (16 s) (rows 16t + l16 share their last four bits with l16)
    const uint32_t a0 = lds_off(blk + l16 * S::RS + g * (V / 4)) + 16 * attn_swz(l16);
    auto rd = [&](int f) __attribute__((always_inline)) -> F {
      return lds_load<F>((a0 + (f / S::SK) * 16 * S::RS * int(sizeof(T))) ^ (16 * (f % S::SK)));
    };
    F cf[DIST];
#pragma unroll
    for (int f = 0; f < DIST; ++f) cf[f] = rd(f);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead: the scheduler would sink them to their uses
#pragma unroll
    for (int f = 0; f < 2 * S::SK; ++f) {
      const int t = f / S::SK, s = f % S::SK;
      sa[t][s & 1] = mfma16(cf[f % DIST], __builtin_bit_cast(F, bank[s]), sa[t][s & 1]);
      if (f + DIST < 2 * S::SK) cf[f % DIST] = rd(f + DIST);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds score row 16*wl + l16, slots 16t + 4g + i
    const uint32_t vm = vmask_s[s_member][j];
    float x[2][4];
    float lmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 16 * t + 4 * g + i;
        x[t][i] = ((vm >> slot) & 1u) ? (sa[t][0][i] + sa[t][1][i]) * scale_log2 : -INFINITY;
        lmax = fmaxf(lmax, x[t][i]);
      }
    // lazy running max, as in attn_kernel
    float alpha = 1.f;
    const bool raise = __ballot(lmax > m_run + LAZY_MAX) != 0;
    if (raise) {
      float bmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = (bmax > m_run + LAZY_MAX) ? bmax : m_run;
      alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      if (g == 0) alpha_s[j & 1][16 * wl + l16] = alpha;
    }
    float rsum = 0.f;
    float pv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[t][i] = (x[t][i] == -INFINITY) ? 0.f : fast_exp2(x[t][i] - m_run);
        rsum += pv[t][i];
      }
    l_run = l_run * alpha + rsum;
    T* prow = ps[j & 1] + (16 * wl + l16) * S::PS;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      *reinterpret_cast<uint2*>(prow + 16 * t + 4 * g) =
          make_uint2(pack_bf16x2(pv[t][0], pv[t][1]), pack_bf16x2(pv[t][2], pv[t][3]));
    if (lane == 0) reinterpret_cast<uint8_t*>(&resc_s[j & 1])[wl] = raise ? 1 : 0;
  };

  // the transposed reads of tokens r1 = 8g + l16/4 and r2 = r1 + 4 at channels c0 + 4a (a = l16 mod 4,
  // c0 = wl * VW + 16 mt) sit at byte base_i ^ (32 mt) of a block, base_i fixed per lane (see attn_swz)
  uint32_t tb1, tb2;
  {
    const int e = l16 >> 2, a = l16 & 3;
    const int r1 = 8 * g + e, r2 = r1 + 4, x1 = attn_swz(r1), x2 = attn_swz(r2);
    const uint32_t b = wl * S::VW * 2 + 8 * (a & 1);
    tb1 = b + r1 * S::RS * 2 + 32 * (x1 >> 1) + 16 * ((a >> 1) ^ (x1 & 1));
    tb2 = b + r2 * S::RS * 2 + 32 * (x2 >> 1) + 16 * ((a >> 1) ^ (x2 & 1));
  }
  // O waves read a block's C^T fragments in the iteration that publishes it (beside S on the same block) and
  // multiply them one iteration later, so a block's buffer is free one iteration earlier than if O read it itself
  auto o_read = [&](int j, F(&av)[S::MT]) __attribute__((always_inline)) {
    const uint32_t blk = lds_off(crm[j % AD_NBUF]);
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt) av[mt] = lds_tr_pair((blk + tb1) ^ (32 * mt), (blk + tb2) ^ (32 * mt));
  };
  auto o_mma = [&](int j, const F(&av)[S::MT]) __attribute__((always_inline)) {
    const T* pb = ps[j & 1];
    // rescale only the head tiles whose running max moved
    const uint32_t rf = resc_s[j & 1];
    if (rf) {
#pragma unroll
      for (int nt = 0; nt < HT; ++nt) {
        if ((rf >> (8 * nt)) & 0xffu) {
          const float a = alpha_s[j & 1][16 * nt + l16];
#pragma unroll
          for (int mt = 0; mt < S::MT; ++mt) bank[mt * HT + nt] *= a;
        }
      }
    }
    F bq[HT];
#pragma unroll
    for (int nt = 0; nt < HT; ++nt) bq[nt] = E::frag_load(pb + (16 * nt + l16) * S::PS + 8 * g);
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < HT; ++nt) bank[mt * HT + nt] = mfma16(av[mt], bq[nt], bank[mt * HT + nt]);
  };
  auto o_phase = [&](int j) __attribute__((always_inline)) {
    const uint32_t blk = lds_off(crm[j % AD_NBUF]);
    const T* pb = ps[j & 1];
    // rescale only the head tiles whose running max moved
    const uint32_t rf = resc_s[j & 1];
    if (rf) {
#pragma unroll
      for (int nt = 0; nt < HT; ++nt) {
        if ((rf >> (8 * nt)) & 0xffu) {
          const float a = alpha_s[j & 1][16 * nt + l16];
#pragma unroll
          for (int mt = 0; mt < S::MT; ++mt) bank[mt * HT + nt] *= a;
        }
      }
    }
    // O^T[channels of this wave][heads] += C^T . P^T over the block's 32 tokens: all fragments first
    F bq[HT];
#pragma unroll
    for (int nt = 0; nt < HT; ++nt) bq[nt] = E::frag_load(pb + (16 * nt + l16) * S::PS + 8 * g);
    F av[S::MT];
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt) av[mt] = lds_tr_pair((blk + tb1) ^ (32 * mt), (blk + tb2) ^ (32 * mt));
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < HT; ++nt) bank[mt * HT + nt] = mfma16(av[mt], bq[nt], bank[mt * HT + nt]);
  };

  // Iteration j: wait for this wave's loads of block j (those of blocks j + 1 and j + 2, when they exist, stay in
  // flight), publish it with the barrier -- after which every wave is past iteration j - 1, so buffer (j + 3) % 4, last read in
  // iteration j - 1 (by S(j - 1) and by the O waves' fragment reads), is free -- start block j + 3, then S(j) on S
  // waves; O waves read block j's C^T fragments and multiply block j - 1's (read in iteration j - 1).  Three blocks
  // stay in flight from HBM per compute unit.  (The barrier's release fence waits for each
  // wave's LDS reads, so no read of a buffer is still pending when its next block is started.)
  if constexpr (!FP8) {
    // Blocks past the end are never loaded, so the last iterations wait for fewer blocks in flight (the wait
    // counts stay exact: a wave's loads complete in issue order).
    load_block(0, block_rows(0));
    if (nblk > 1) load_block(1, block_rows(1));
    if (nblk > 2) load_block(2, block_rows(2));
    int rows_next = block_rows(3);
    auto publish = [&](int j) __attribute__((always_inline)) {
      if (j + 2 < nblk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * S::CHT));
      else if (j + 1 < nblk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(S::CHT));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      if (j + 3 < nblk) load_block(j + 3, rows_next);
      rows_next = block_rows(j + 4);
    };
    // One loop per role (the role is wave-uniform and both loops pass the same barriers), so the O waves' two
    // fragment sets and the S waves' read-ahead never hold registers at the same time.
    if (o_wave) {
      F avA[S::MT], avB[S::MT];
      // unrolled by two, so each fragment set keeps its registers
      for (int j = 0;;) {
        publish(j);
        if (j < nblk) o_read(j, avA);
        if (j >= 1) o_mma(j - 1, avB);
        if (++j > nblk) break;
        publish(j);
        if (j < nblk) o_read(j, avB);
        o_mma(j - 1, avA);
        if (++j > nblk) break;
      }
    } else {
      for (int j = 0; j <= nblk; ++j) {
        publish(j);
        if (s_active && j < nblk) s_phase(j);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load may land in LDS after the block ends
  } else {
    // Wave w brings slots 4w .. 4w + 3 of each block (as the direct loads do): load i covers slot 4w + 2i (lanes
    // 0..31) and 4w + 2i + 1 (lanes 32..63), lane l taking the 16 codes of channels 16 (l % 32) .. + 15.
    // Lane j < 4 of fp8_rows(b) holds the cache row of slot 4w + j of block b (-1: none).
    auto fp8_rows = [&](int b) __attribute__((always_inline)) -> int {
      return slot_entry(b, 4 * wave_u + (lane & 3));
    };
    auto load8 = [&](int rows, u32x4(&R)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int e0 = __builtin_amdgcn_readlane(rows, 2 * i), e1 = __builtin_amdgcn_readlane(rows, 2 * i + 1);
        const int e = lane < 32 ? e0 : e1;
        const uint8_t* src = e >= 0 ? latent8 + int64_t(e) * L + 16 * (lane & 31)
                                    : reinterpret_cast<const uint8_t*>(attn_zero_row) + 16 * (lane & 31);
        R[i] = *reinterpret_cast<const u32x4*>(src);
      }
    };
    // codes -> bf16 into buffer b % 4: the 16 codes of lane l are bf16 chunks 2 (l % 32) and 2 (l % 32) + 1 of
    // its slot's row, stored at chunk position c ^ attn_swz(slot) as the direct loads place them
    auto store8 = [&](int b, const u32x4(&R)[2]) __attribute__((always_inline)) {
      T* blk = crm[b % AD_NBUF];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int slot = 4 * wave_u + 2 * i + (lane >> 5);
        const int c = 2 * (lane & 31);
        uint32_t h[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(R[i][d]), false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(R[i][d]), true);
          h[2 * d] = pack_bf16x2(lo[0], lo[1]);
          h[2 * d + 1] = pack_bf16x2(hi[0], hi[1]);
        }
        T* row = blk + slot * V;
        *reinterpret_cast<u32x4*>(row + ((c ^ attn_swz(slot)) * S::EPC)) = u32x4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<u32x4*>(row + (((c + 1) ^ attn_swz(slot)) * S::EPC)) = u32x4{h[4], h[5], h[6], h[7]};
      }
    };
    // blocks in flight, block b in R[b % 3] (a fourth would not fit the registers beside the S and O state)
    u32x4 R0[2], R1[2], R2[2];
    load8(fp8_rows(0), R0);
    load8(fp8_rows(1), R1);
    load8(fp8_rows(2), R2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    store8(0, R0);
    load8(fp8_rows(3), R0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
    store8(1, R1);
    load8(fp8_rows(4), R1);
    // Iteration j: the barrier publishes block j + 1 (written in iteration j - 1); after it every wave is past
    // iteration j - 1, so buffer (j + 2) % 4, last read by S(j - 2) and O(j - 2), is free: each wave writes its
    // rows of block j + 2 into it from registers and loads block j + 5 in their place, then O waves run O(j - 1)
    // and S waves S(j).  Loads are unconditional (a block past the end reads the zero row), so the wait for the
    // oldest block is exact.
    auto iter = [&](int j, u32x4(&R)[2]) __attribute__((always_inline)) {
      __syncthreads();
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
      store8(j + 2, R);
      load8(fp8_rows(j + 5), R);
      if (o_wave) {
        if (j >= 1) o_phase(j - 1);
      } else if (s_active && j < nblk) {
        s_phase(j);
      }
    };
    // unrolled by the register ring, so every register index is a constant (a block in flight must stay in its
    // registers: moving them would wait for its loads); the scheduling barriers keep the copies apart
    for (int j = 0;;) {
      iter(j, R2);
      __builtin_amdgcn_sched_barrier(0);
      if (++j > nblk) break;
      iter(j, R0);
      __builtin_amdgcn_sched_barrier(0);
      if (++j > nblk) break;
      iter(j, R1);
      __builtin_amdgcn_sched_barrier(0);
      if (++j > nblk) break;
    }
    __builtin_amdgcn_s_waitcnt(0);
  }

  if (s_active) {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (g == 0) {
      m_s[16 * wl + l16] = m_run;
      l_s[16 * wl + l16] = l_run;
    }
  }
  __syncthreads();
  // Write-out through LDS (the ring is free now): O waves store their scaled O as bf16 rows of 1040 B (1 KiB of
  // channels plus 16 B, which keeps the 16 heads of one store on distinct banks); then all threads copy the rows
  // out with 16-byte stores.  A (query, split)'s H x V outputs are contiguous, so the copy is one 64 KiB run.
  constexpr int SROW = V + 8;  // staging row stride, elements
  static_assert(64 * SROW * int(sizeof(T)) <= AD_NBUF * AT_NT * V * int(sizeof(T)), "staging fits the ring");
  T* stg = &crm[0][0];  // the whole ring, as one array
  if (o_wave) {
#pragma unroll
    for (int nt = 0; nt < HT; ++nt) {
      const int r = 16 * nt + l16;
      int qd, hd;
      if (!row_dest(r, qd, hd)) continue;
      // (a query that sees no token of this block's list -- possible for one query of an MTP run -- has l = 0)
      const float f = n_split == 1 ? (l_s[r] > 0.f ? oscale / l_s[r] : 0.f) : oscale;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const f32x4 o = bank[mt * HT + nt] * f;
        *reinterpret_cast<uint2*>(stg + r * SROW + wl * S::VW + 16 * mt + 4 * g) =
            make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < NROW * (V / S::EPC); i += AT_THREADS) {
    const int r = i / (V / S::EPC), c = i % (V / S::EPC);
    int qd, hd;
    if (!row_dest(r, qd, hd)) continue;
    T* dst = n_split == 1 ? out + (int64_t(qd) * H + hd) * V : part_o + (int64_t(qd * n_split + sp) * H + hd) * V;
    *reinterpret_cast<u32x4*>(dst + c * S::EPC) = *reinterpret_cast<const u32x4*>(stg + r * SROW + c * S::EPC);
  }
  if (tid < NROW) {
    int qd, hd;
    if (row_dest(tid, qd, hd)) {
      if (n_split == 1) {
        if (lse) lse[int64_t(qd) * H + hd] = l_s[tid] > 0.f ? (m_s[tid] + log2f(l_s[tid])) * LN2 : -INFINITY;
      } else {
        const int64_t base = int64_t(qd * n_split + sp) * H + hd;
        part_ml[base * 2 + 0] = m_s[tid];
        part_ml[base * 2 + 1] = l_s[tid];
      }
    }
  }
}

// Merge of the split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s per (query, head), with
// M the max of m_s over non-empty splits, both sums taken in split order.  Each split's O is stored in the cache
// dtype (rounded once, as the output is), its (m, l) in fp32.  A group of TPC adjacent threads merges 16 bytes of
// channels (8 bf16 or 4 fp32) of one head, each thread PER of its splits; 256 threads per block.  Every thread
// issues the loads of all its splits' partial O and (m, l) at once (an empty split's O was never written, so its
// value is dropped by a select) and computes its head's weights itself: no LDS, no barrier, one wait on memory.
constexpr int CB_THREADS = 256;
constexpr int CB_MAXSPLIT = 64;  // attn_splits never returns more

// PER: splits per thread (registers for each); TPC: threads per 16-byte output chunk (1, 2, 4 or 8 adjacent lanes),
// each merging its own PER splits against the group's common maximum, the group's sums added across its lanes
// (one DPP exchange per value and lane bit) and written by the first lane.  More lanes per chunk spread a few
// queries' many splits over more compute units: each holds fewer loads in flight.
template <class T, int PER, int TPC>
__global__ __launch_bounds__(CB_THREADS) void attn_combine_kernel(const T* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml, int n_split,
                                                                  int n_q, int H, int V, T* __restrict__ out,
                                                                  float* __restrict__ lse) {
  static_assert(PER * TPC <= CB_MAXSPLIT && (TPC == 1 || TPC == 2 || TPC == 4 || TPC == 8), "splits per thread");
  constexpr int EPT = 16 / int(sizeof(T));  // channels per thread
  const int tph = TPC * (V / EPT);          // threads per head (a head may span blocks)
  // thread t of the grid: query t / (H tph), head (t mod H tph) / tph, lane group (t mod tph) / TPC
  const int64_t gt = int64_t(blockIdx.x) * CB_THREADS + threadIdx.x, per_q = int64_t(H) * tph;
  const int qi = int(gt / per_q);
  const int rem = int(gt - int64_t(qi) * per_q);
  const int h = rem / tph;
  const int c = ((rem % tph) / TPC) * EPT;
  const int part = rem & (TPC - 1);  // which PER splits this thread merges (TPC divides tph)
  const int64_t mls = int64_t(H) * 2, pos_ = int64_t(H) * V;
  if (qi >= n_q) return;  // past the last query (a group's lanes are adjacent: groups leave whole)
  const int64_t row = int64_t(qi) * n_split * H + h;  // split s: O at part_o + (row + s * H) * V, (m, l) likewise
  const int s0 = part * PER, n_mine = min(PER, n_split - s0);
  const T* po = part_o + (row + int64_t(s0) * H) * V + c;
  const float* pm = part_ml + (row + int64_t(s0) * H) * 2;
  u32x4 o[PER];
  float2 ml[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (u < n_mine) {
      o[u] = *reinterpret_cast<const u32x4*>(po + u * pos_);
      ml[u] = *reinterpret_cast<const float2*>(pm + u * mls);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (u < n_mine && ml[u].y > 0.f) M = fmaxf(M, ml[u].x);
  // the group's lanes: lane ^ 1 (quad_perm 1, 0, 3, 2), lane ^ 2 (quad_perm 2, 3, 0, 1), then the other quad of
  // the 8 (row_half_mirror: each quad already holds its quad's value)
  auto group = [&](float v, auto op) __attribute__((always_inline)) {
    if constexpr (TPC >= 2) v = op(v, __uint_as_float(dpp_u32<0xB1>(0u, __float_as_uint(v))));
    if constexpr (TPC >= 4) v = op(v, __uint_as_float(dpp_u32<0x4E>(0u, __float_as_uint(v))));
    if constexpr (TPC >= 8) v = op(v, __uint_as_float(dpp_u32<0x141>(0u, __float_as_uint(v))));
    return v;
  };
  auto fmax2 = [](float a, float b) { return fmaxf(a, b); };
  auto fadd2 = [](float a, float b) { return a + b; };
  M = group(M, fmax2);
  float wsum = 0.f;
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if (u < n_mine && ml[u].y > 0.f) {
      const float w = exp2f(ml[u].x - M);
      wsum += ml[u].y * w;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float v;
        if constexpr (sizeof(T) == 2) {
          const uint32_t d = o[u][e / 2];
          v = __uint_as_float((e & 1) ? (d & 0xffff0000u) : (d << 16));
        } else {
          v = __uint_as_float(o[u][e]);
        }
        acc[e] += w * v;
      }
    }
  }
  if constexpr (TPC > 1) {
    wsum = group(wsum, fadd2);
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = group(acc[e], fadd2);
    if (part) return;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;  // a query that attends no token: zeros, lse -inf
  u32x4 r;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __float_as_uint(acc[e] * inv);
  }
  *reinterpret_cast<u32x4*>(out + (int64_t(qi) * H + h) * V + c) = r;
  if (lse && c == 0) lse[int64_t(qi) * H + h] = wsum > 0.f ? (M + log2f(wsum)) * LN2 : -INFINITY;
}

int attn_splits(int P, int k, int n_q) {
  // about one block per CU (256), at most CB_MAXSPLIT splits, at least one pool per split, and few enough pools per
  // split (ceil((k + 1) / splits) <= AT_MAXSLOT / P, and <= AD_MAXPOOL) for the LDS slot and pool tables -- a
  // row shared by an MTP draft may carry the draft's own tail pool beyond its k entries
  int64_t want = (256 + int64_t(n_q) - 1) / (n_q > 0 ? n_q : 1);
  if (want > k) want = k;
  if (want > CB_MAXSPLIT) want = CB_MAXSPLIT;
  const int64_t per_split = AT_MAXSLOT / P < AD_MAXPOOL ? AT_MAXSLOT / P : AD_MAXPOOL;
  const int64_t min_splits = (int64_t(k) + 1 + per_split - 1) / per_split;
  if (want < min_splits) want = min_splits;
  return want < 1 ? 1 : int(want);
}

int attn_splits_mtp(int P, int k, int n_q, int H) {
  // about 256 blocks over the runs' head halves, at most 32 splits, and few enough list entries per split for the
  // LDS tables: a run of two sequences lists both queries' pools, 2 (k + 1) entries
  const int64_t units = int64_t((n_q + 1) / 2) * ((H + 31) / 32);
  int64_t want = (256 + units - 1) / (units > 0 ? units : 1);
  if (want > k) want = k;
  if (want > 32) want = 32;
  const int64_t per_split = AT_MAXSLOT / P < AD_MAXPOOL ? AT_MAXSLOT / P : AD_MAXPOOL;
  const int64_t min_splits = (2 * (int64_t(k) + 1) + per_split - 1) / per_split;
  if (want < min_splits) want = min_splits;
  return want < 1 ? 1 : int(want);
}

size_t attn_workspace_mtp(int P, int k, int H, int V, int n_q, int esize) {
  const int ns = attn_splits_mtp(P, k, n_q, H);
  if (ns <= 1) return 0;
  return size_t(n_q) * ns * H * (size_t(V) * esize + 2 * sizeof(float));
}

size_t attn_workspace(int P, int k, int H, int V, int n_q, int esize) {
  const int ns = attn_splits(P, k, n_q);
  if (ns <= 1) return 0;
  // partial O in the cache dtype, then (m, l) in fp32 (n_q * ns * H * V * esize is a multiple of 8: V is even)
  return size_t(n_q) * ns * H * (size_t(V) * esize + 2 * sizeof(float));
}

// Split-KV partials of sparse_mla_attn_noalloc: one array per device, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a device address); it uses the address
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[KP_NOALLOC_SCRATCH_BYTES];

kp_status attn_noalloc_scratch(void** ptr) {
  constexpr int MAXDEV = 64;
  static void* addr[MAXDEV] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= MAXDEV) {
    set_error("sparse_mla_attn_noalloc: no usable current device (%s)", hipGetErrorString(e));
    return KP_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("sparse_mla_attn_noalloc: scratch address lookup failed on device %d: %s", dev, hipGetErrorString(e));
      return KP_ERR_LAUNCH;
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return KP_OK;
}

// Split merge of n_q queries' partials (ns splits each) into out / lse.
template <class T>
static kp_status launch_combine(const AttnLaunch& a, int ns, const T* part_o, const float* part_ml, hipStream_t s) {
  const int tpc = ns <= 8 ? 1 : ns <= 16 ? 2 : ns <= 32 ? 4 : 8;  // threads per 16-byte output chunk, 8 splits each
  const int64_t threads = int64_t(a.n_q) * a.H * tpc * (a.V / (16 / int(sizeof(T))));
  const dim3 grid(unsigned((threads + CB_THREADS - 1) / CB_THREADS)), block(CB_THREADS);
  if (tpc == 1)
    attn_combine_kernel<T, 8, 1><<<grid, block, 0, s>>>(part_o, part_ml, ns, a.n_q, a.H, a.V, (T*)a.out, a.lse);
  else if (tpc == 2)
    attn_combine_kernel<T, 8, 2><<<grid, block, 0, s>>>(part_o, part_ml, ns, a.n_q, a.H, a.V, (T*)a.out, a.lse);
  else if (tpc == 4)
    attn_combine_kernel<T, 8, 4><<<grid, block, 0, s>>>(part_o, part_ml, ns, a.n_q, a.H, a.V, (T*)a.out, a.lse);
  else
    attn_combine_kernel<T, 8, 8><<<grid, block, 0, s>>>(part_o, part_ml, ns, a.n_q, a.H, a.V, (T*)a.out, a.lse);
  return check_launch("sparse_mla_attn (split merge)");
}

// MTP runs (sparse_mla_attn_mtp): bf16 rows of 512 value columns, 64 heads at most.  Blocks: every (run, split)
// unit once per head half, the units 8 to a group and a group's head halves 8 blocks apart (one XCD).
static kp_status launch_attn_mtp(const AttnLaunch& a, hipStream_t s) {
  const int ns = attn_splits_mtp(a.P, a.k, a.n_q, a.H);
  bf16* part_o = nullptr;
  float* part_ml = nullptr;
  if (ns > 1) {
    part_o = reinterpret_cast<bf16*>(a.ws);
    part_ml = reinterpret_cast<float*>(part_o + size_t(a.n_q) * ns * a.H * a.V);
  }
  const int64_t units = int64_t((a.n_q + 1) / 2) * ns;
  const int64_t blocks = (units + 7) / 8 * 8 * ((a.H + 31) / 32);
  if (blocks > 0x7fffffff) {
    set_error("sparse_mla_attn_mtp: too many queries for one launch");
    return KP_ERR_INVALID_ARG;
  }
  attn_dma_kernel<4, false, true><<<dim3(unsigned(blocks)), dim3(AT_THREADS), 0, s>>>(
      a.latent, a.L, a.bt, a.bt_stride, a.log2_pt, (const bf16*)a.q, a.q_seq, a.q_pos, a.sel, a.n_sel, nullptr,
      ilog2(a.P), a.k, a.H, a.scale * 1.4426950408889634f, ns, (bf16*)a.out, a.lse, part_o, part_ml, 1.f, a.n_q);
  kp_status st = check_launch("sparse_mla_attn_mtp");
  if (st != KP_OK || ns == 1) return st;
  return launch_combine<bf16>(a, ns, part_o, part_ml, s);
}

template <class T, int V, int HT>
static kp_status launch_attn_t(const AttnLaunch& a, hipStream_t s) {
  const int ns = attn_splits(a.P, a.k, a.n_q);
  T* part_o = nullptr;
  float* part_ml = nullptr;
  if (ns > 1) {
    part_o = reinterpret_cast<T*>(a.ws);
    part_ml = reinterpret_cast<float*>(part_o + size_t(a.n_q) * ns * a.H * a.V);
  }
  const float scale_log2 = a.scale * 1.4426950408889634f;
  if constexpr (std::is_same<T, bf16>::value && V == 512) {
    if (a.latent_fp8)  // the cache scale multiplies every logit and the output
      attn_dma_kernel<HT, true><<<dim3(unsigned(int64_t(a.n_q) * ns)), dim3(AT_THREADS), 0, s>>>(
          a.latent, a.L, a.bt, a.bt_stride, a.log2_pt, (const T*)a.q, a.q_seq, a.q_pos, a.sel, a.n_sel, a.sel_row,
          ilog2(a.P), a.k, a.H, scale_log2 * a.kv_scale, ns, (T*)a.out, a.lse, part_o, part_ml, a.kv_scale,
          a.n_q);
    else
      attn_dma_kernel<HT, false><<<dim3(unsigned(int64_t(a.n_q) * ns)), dim3(AT_THREADS), 0, s>>>(
          a.latent, a.L, a.bt, a.bt_stride, a.log2_pt, (const T*)a.q, a.q_seq, a.q_pos, a.sel, a.n_sel, a.sel_row,
          ilog2(a.P), a.k, a.H, scale_log2, ns, (T*)a.out, a.lse, part_o, part_ml, 1.f, a.n_q);
  } else

    attn_kernel<T, V, HT><<<dim3(unsigned(int64_t(a.n_q) * ns)), dim3(AT_THREADS), 0, s>>>(
        (const T*)a.latent, a.L, a.bt, a.bt_stride, a.log2_pt, (const T*)a.q, a.q_seq, a.q_pos, a.sel, a.n_sel,
        a.sel_row,
        ilog2(a.P), a.k, a.H, scale_log2, ns, (T*)a.out, a.lse, part_o, part_ml);
  kp_status st = check_launch("sparse_mla_attn");
  if (st != KP_OK || ns == 1) return st;
  return launch_combine<T>(a, ns, part_o, part_ml, s);
}

kp_status launch_attn(const AttnLaunch& a, hipStream_t s) {
  if (a.n_q == 0) return KP_OK;
  if (a.mtp) {
    if (!(a.dtype == KP_DTYPE_BF16 && a.V == 512 && !a.latent_fp8 && a.H <= 64)) {
      set_error("sparse_mla_attn_mtp: built for bf16 with v_dim 512 and at most 64 heads");
      return KP_ERR_UNSUPPORTED;
    }
    if (attn_splits_mtp(a.P, a.k, a.n_q, a.H) > CB_MAXSPLIT) {
      set_error("sparse_mla_attn_mtp: topk %d pools of %d tokens needs more than %d splits per query", a.k, a.P,
                CB_MAXSPLIT);
      return KP_ERR_UNSUPPORTED;
    }
    return launch_attn_mtp(a, s);
  }
  if (a.latent_fp8 && !(a.dtype == KP_DTYPE_BF16 && a.V == 512)) {
    set_error("sparse_mla_attn_fp8: built for bf16 queries with v_dim 512 only");
    return KP_ERR_UNSUPPORTED;
  }
  if (attn_splits(a.P, a.k, a.n_q) > CB_MAXSPLIT) {
    set_error("sparse_mla_attn: topk %d pools of %d tokens needs more than %d splits per query", a.k, a.P,
              CB_MAXSPLIT);
    return KP_ERR_UNSUPPORTED;
  }
  if (int64_t(a.n_q) * attn_splits(a.P, a.k, a.n_q) > 0x7fffffff) {
    set_error("sparse_mla_attn: too many queries for one launch");
    return KP_ERR_INVALID_ARG;
  }
  // 16-head tiles: 1 (H <= 16), 2 (H <= 32) or 4 (H <= 64)
  const int ht = a.H <= 16 ? 1 : a.H <= 32 ? 2 : 4;
  if (a.dtype == KP_DTYPE_BF16) {
    if (a.V == 512) {
      if (ht == 4) return launch_attn_t<bf16, 512, 4>(a, s);
      if (ht == 2) return launch_attn_t<bf16, 512, 2>(a, s);
      return launch_attn_t<bf16, 512, 1>(a, s);
    }
    if (ht == 4) return launch_attn_t<bf16, 64, 4>(a, s);
    if (ht == 2) return launch_attn_t<bf16, 64, 2>(a, s);
    return launch_attn_t<bf16, 64, 1>(a, s);
  }
  if (ht == 4) return launch_attn_t<float, 64, 4>(a, s);
  if (ht == 2) return launch_attn_t<float, 64, 2>(a, s);
  return launch_attn_t<float, 64, 1>(a, s);
}

}  // namespace kp
