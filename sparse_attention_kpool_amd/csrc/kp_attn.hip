// sparse_mla_attn: nope-only absorbed MLA of each query over the tokens of its selected pools.
//
// [llama.cpp PR "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: attention layers are
// nope-only MLA.  [MAX glm5_next API page, mla_use_nope / build_layers()]: no rotary embedding; the latent row is
// 576 wide, its last 64 (rotary) columns all zero.  [GLM-5.3-Flash model card, "Raw config fields"]:
// kv_lora_rank 512, 64 heads.  Absorbed MLA: the key of token t is its latent row, the value its first V
// columns; the zero rotary columns add nothing to q . latent and are not read.
//
// One block (4 waves) per (query, split of its selected tokens).  Token slots are taken 32 at a time: slot j
// is token P * sel[j / P] + j % P, valid while j < P * n_sel and the token is <= the query position (the tail
// pool is cut at the query itself).  Per 32-slot block:
//   load   every thread gathers 16-byte chunks of the V-wide value rows (8 threads cover 128 contiguous bytes
//          of a row) into registers one block ahead, then writes them to LDS twice: row-major (token x
//          channel) and transposed (channel x token).
//   S      wave w owns heads 16w..16w+15 and computes S^T = C . Q^T on 16x16x32 bf16 MFMA (tokens = M,
//          heads = N, channels = K).  Its Q fragments stay in registers for the whole call; C comes from the
//          row-major copy with one 16-byte read per lane per k-step.  Online softmax per head: each lane holds
//          one head, so the row max / sum take two cross-lane steps (xor 16, xor 32).
//   O      wave w owns value channels w*V/4 .. (w+1)*V/4 for all heads: O^T += C^T . P^T, with C^T from the
//          transposed copy and P (stored by the S waves in LDS) as B.  Its accumulators (V/4 x 64 heads fp32)
//          stay in registers; each head's rescale factor is one scalar per lane.
// Splits write unnormalised partials (O, running max, running sum) that a second kernel merges in split
// order, so results are deterministic.
//
// Bound: HBM (the gather of 1 KiB of bf16 value columns per token feeds 2 x 64 heads x 512 MACs: 128 flop/B,
// between the VALU and MFMA ridges, hence MFMA for both products).
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int AT_NT = 32;  // token slots per block
constexpr float LN2 = 0.69314718055994530942f;

template <class T, int V>
struct AttnShape {
  static constexpr int KPL = Elem<T>::kpl;
  static constexpr int EPC = 16 / int(sizeof(T));   // elements per 16-byte chunk
  static constexpr int CPR = V / EPC;               // chunks per value row
  static constexpr int UNITS = 8 * CPR;             // (4-token group, chunk) load units per block
  static constexpr int UPT = (UNITS + 255) / 256;   // units per thread
  static constexpr int RS = V + EPC;                // row-major LDS stride (elements), +16 B against conflicts
  static constexpr int TS = AT_NT + EPC;            // transposed LDS stride
  static constexpr int PS = AT_NT + EPC;            // P stride
  static constexpr int VW = V / 4;                  // value channels per wave in the O product
  static constexpr int MT = VW / 16;                // 16-channel tiles per wave
  static constexpr int SK = V / (4 * KPL);          // k-steps of the S product (K = V channels)
  static constexpr int OK = AT_NT / (4 * KPL);      // k-steps of the O product (K = 32 tokens)
  static_assert(CPR % 8 == 0, "value row must be a multiple of 128 bytes");
  static_assert(VW % 16 == 0, "value width must split into 16-channel tiles per wave");
};

template <class T>
__device__ __forceinline__ uint32_t chunk_elem_bits(const uint4& v, int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
  } else {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  }
}

template <class T, int V>
__global__ __launch_bounds__(256) void attn_kernel(
    const T* __restrict__ latent, int L, const int32_t* __restrict__ bt, int bt_stride, int log2_pt,
    const T* __restrict__ q, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, int log2P, int k, int H, float scale_log2,
    int n_split, int blocks_per_split, T* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using S = AttnShape<T, V>;
  using E = Elem<T>;
  using F = typename E::frag;
  __shared__ __align__(16) T crm[AT_NT * S::RS];
  __shared__ __align__(16) T ct[V * S::TS];
  __shared__ __align__(16) T ps[64 * S::PS];
  __shared__ float alpha_s[64];
  __shared__ float m_s[64];
  __shared__ float l_s[64];
  __shared__ uint32_t vmask_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int qi = blockIdx.x / n_split;
  const int sp = blockIdx.x - qi * n_split;
  const int seq = q_seq[qi];
  const int pos = q_pos[qi];
  const int P = 1 << log2P;
  const int n_slots = n_sel[qi] * P;
  const int s_begin = sp * blocks_per_split * AT_NT;
  const int s_end = min(s_begin + blocks_per_split * AT_NT, n_slots);
  const int32_t* qsel = sel + int64_t(qi) * k;

  if (s_begin >= s_end) {  // an empty split (this query selected fewer tokens)
    if (n_split > 1) {
      for (int h = tid; h < H; h += 256) {
        part_ml[(int64_t(qi * n_split + sp) * H + h) * 2 + 0] = -INFINITY;
        part_ml[(int64_t(qi * n_split + sp) * H + h) * 2 + 1] = 0.f;
      }
    } else {
      for (int64_t e = tid; e < int64_t(H) * V; e += 256) out[int64_t(qi) * H * V + e] = E::from_f32(0.f);
      if (lse)
        for (int h = tid; h < H; h += 256) lse[int64_t(qi) * H + h] = -INFINITY;
    }
    return;
  }
  const int nblk = (s_end - s_begin + AT_NT - 1) / AT_NT;

  // Q^T fragments of this wave's 16 heads (B operand of S^T = C . Q^T): lane holds head 16*wave + l16,
  // channels g*(V/4) + s*KPL .. +KPL for k-step s
  const bool s_wave = 16 * wave < H;
  F qf[S::SK];
  {
    const int h = 16 * wave + l16;
    const bool hv = h < H;
    const T* qp = q + (int64_t(qi) * H + (hv ? h : 0)) * L + g * (V / 4);
#pragma unroll
    for (int s = 0; s < S::SK; ++s) qf[s] = hv ? E::frag_load(qp + s * S::KPL) : E::frag_zero();
  }

  f32x4 oacc[S::MT][4];
#pragma unroll
  for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 buf[S::UPT][4];
  uint32_t vmask = 0;

  // token of slot `slot`, or -1 when the slot is past this split or past the query (causal tail)
  auto slot_token = [&](int slot) -> int {
    if (slot >= s_end) return -1;
    const int p = qsel[slot >> log2P];
    if (p < 0) return -1;
    const int t = (p << log2P) + (slot & (P - 1));
    return t <= pos ? t : -1;
  };

  auto load_block = [&](int b) {
    const int slot0 = s_begin + b * AT_NT;
#pragma unroll
    for (int j = 0; j < S::UPT; ++j) {
      const int u = tid + 256 * j;
      const int c = ((u >> 6) << 3) | (u & 7);
      const int pg = (u >> 3) & 7;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = (u < S::UNITS) ? slot_token(slot0 + 4 * pg + t) : -1;
        if (tok >= 0) {
          const int64_t row = paged_row(bt, bt_stride, seq, tok, log2_pt);
          buf[j][t] = *reinterpret_cast<const uint4*>(latent + row * L + c * S::EPC);
        } else {
          buf[j][t] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    if (wave == 0) {
      const bool v = lane < AT_NT && slot_token(slot0 + lane) >= 0;
      vmask = uint32_t(__ballot(v));
    }
  };

  auto store_block = [&]() {
#pragma unroll
    for (int j = 0; j < S::UPT; ++j) {
      const int u = tid + 256 * j;
      if (u >= S::UNITS) continue;
      const int c = ((u >> 6) << 3) | (u & 7);
      const int pg = (u >> 3) & 7;
#pragma unroll
      for (int t = 0; t < 4; ++t) *reinterpret_cast<uint4*>(&crm[(4 * pg + t) * S::RS + c * S::EPC]) = buf[j][t];
#pragma unroll
      for (int e = 0; e < S::EPC; ++e) {
        T* dst = &ct[(c * S::EPC + e) * S::TS + 4 * pg];
        if constexpr (sizeof(T) == 2) {
          const uint32_t lo = chunk_elem_bits<T>(buf[j][0], e) | (chunk_elem_bits<T>(buf[j][1], e) << 16);
          const uint32_t hi = chunk_elem_bits<T>(buf[j][2], e) | (chunk_elem_bits<T>(buf[j][3], e) << 16);
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<uint4*>(dst) =
              make_uint4(chunk_elem_bits<T>(buf[j][0], e), chunk_elem_bits<T>(buf[j][1], e),
                         chunk_elem_bits<T>(buf[j][2], e), chunk_elem_bits<T>(buf[j][3], e));
        }
      }
    }
    if (tid == 0) vmask_s = vmask;
  };

  load_block(0);
  for (int b = 0; b < nblk; ++b) {
    __syncthreads();  // every wave is done reading the previous block from LDS
    store_block();
    __syncthreads();
    if (b + 1 < nblk) load_block(b + 1);  // in flight while this block is computed
    const uint32_t vm = vmask_s;

    if (s_wave) {
      // S^T tiles for tokens 0..15 and 16..31 of the block
      f32x4 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const T* ap = &crm[(16 * t + l16) * S::RS + g * (V / 4)];
#pragma unroll
        for (int s = 0; s < S::SK; ++s) sacc[t] = mfma16(E::frag_load(ap + s * S::KPL), qf[s], sacc[t]);
      }
      // lane holds head 16*wave + l16, tokens 16t + 4g + i
      float x[2][4];
      float bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 16 * t + 4 * g + i;
          x[t][i] = ((vm >> slot) & 1u) ? sacc[t][i] * scale_log2 : -INFINITY;
          bmax = fmaxf(bmax, x[t][i]);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
      float rsum = 0.f;
      float pv[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[t][i] = (x[t][i] == -INFINITY) ? 0.f : exp2f(x[t][i] - m_new);
          rsum += pv[t][i];
        }
      rsum += __shfl_xor(rsum, 16);
      rsum += __shfl_xor(rsum, 32);
      l_run = l_run * alpha + rsum;
      m_run = m_new;
      T* prow = &ps[(16 * wave + l16) * S::PS];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (sizeof(T) == 2) {
          const uint32_t lo = uint32_t(f32_to_bf16(pv[t][0])) | (uint32_t(f32_to_bf16(pv[t][1])) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16(pv[t][2])) | (uint32_t(f32_to_bf16(pv[t][3])) << 16);
          *reinterpret_cast<uint2*>(prow + 16 * t + 4 * g) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(prow + 16 * t + 4 * g) = make_float4(pv[t][0], pv[t][1], pv[t][2], pv[t][3]);
        }
      }
      if (g == 0) alpha_s[16 * wave + l16] = alpha;
    }
    __syncthreads();

    // O^T[channels of this wave][heads] += C^T . P^T; slot for (group g, step s, element e) = 8g + s*KPL + e
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (16 * nt >= H) break;
      const float a = alpha_s[16 * nt + l16];
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) oacc[mt][nt] *= a;
    }
#pragma unroll
    for (int s = 0; s < S::OK; ++s) {
      F bq[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bq[nt] = (16 * nt < H) ? E::frag_load(&ps[(16 * nt + l16) * S::PS + 8 * g + s * S::KPL]) : E::frag_zero();
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const F av = E::frag_load(&ct[(wave * S::VW + 16 * mt + l16) * S::TS + 8 * g + s * S::KPL]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (16 * nt < H) oacc[mt][nt] = mfma16(av, bq[nt], oacc[mt][nt]);
      }
    }
  }

  if (s_wave && g == 0) {
    m_s[16 * wave + l16] = m_run;
    l_s[16 * wave + l16] = l_run;
  }
  __syncthreads();

#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int h = 16 * nt + l16;
    if (16 * nt >= H) break;
    if (h >= H) continue;
    const float mh = m_s[h], lh = l_s[h];
    if (n_split == 1) {
      const float inv = 1.f / lh;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const int ch0 = wave * S::VW + 16 * mt + 4 * g;
        T* op = out + (int64_t(qi) * H + h) * V + ch0;
        if constexpr (sizeof(T) == 2) {
          const uint32_t lo = uint32_t(f32_to_bf16(oacc[mt][nt][0] * inv)) |
                              (uint32_t(f32_to_bf16(oacc[mt][nt][1] * inv)) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16(oacc[mt][nt][2] * inv)) |
                              (uint32_t(f32_to_bf16(oacc[mt][nt][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(op) = make_float4(oacc[mt][nt][0] * inv, oacc[mt][nt][1] * inv,
                                                       oacc[mt][nt][2] * inv, oacc[mt][nt][3] * inv);
        }
      }
      if (lse && wave == 0 && g == 0) lse[int64_t(qi) * H + h] = (mh + log2f(lh)) * LN2;
    } else {
      const int64_t base = int64_t(qi * n_split + sp) * H + h;
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) {
        const int ch0 = wave * S::VW + 16 * mt + 4 * g;
        *reinterpret_cast<float4*>(part_o + base * V + ch0) =
            make_float4(oacc[mt][nt][0], oacc[mt][nt][1], oacc[mt][nt][2], oacc[mt][nt][3]);
      }
      if (wave == 0 && g == 0) {
        part_ml[base * 2 + 0] = mh;
        part_ml[base * 2 + 1] = lh;
      }
    }
  }
}

// Merge of the split partials of one (query, head): out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <class T>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, int n_split, int H,
                                                           int V, T* __restrict__ out, float* __restrict__ lse) {
  const int qh = blockIdx.x;
  const int qi = qh / H, h = qh - qi * H;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) {
    const int64_t b = (int64_t(qi * n_split + s) * H + h) * 2;
    if (part_ml[b + 1] > 0.f) M = fmaxf(M, part_ml[b]);
  }
  float wsum = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const int64_t b = (int64_t(qi * n_split + s) * H + h) * 2;
    const float l = part_ml[b + 1];
    if (l > 0.f) wsum += l * exp2f(part_ml[b] - M);
  }
  const float inv = 1.f / wsum;
  for (int c = threadIdx.x; c < V; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const int64_t b = int64_t(qi * n_split + s) * H + h;
      const float l = part_ml[b * 2 + 1];
      if (l > 0.f) acc += part_o[b * V + c] * exp2f(part_ml[b * 2] - M);
    }
    out[int64_t(qh) * V + c] = Elem<T>::from_f32(acc * inv);
  }
  if (lse && threadIdx.x == 0) lse[qh] = (M + log2f(wsum)) * LN2;
}

int attn_splits(int P, int k, int n_q) {
  const int64_t blocks = (int64_t(k) * P + AT_NT - 1) / AT_NT;
  int64_t want = (512 + int64_t(n_q) - 1) / (n_q > 0 ? n_q : 1);
  if (want > blocks) want = blocks;
  if (want > 32) want = 32;
  return want < 1 ? 1 : int(want);
}

size_t attn_workspace(int P, int k, int H, int V, int n_q) {
  const int ns = attn_splits(P, k, n_q);
  if (ns <= 1) return 0;
  return size_t(n_q) * ns * H * (size_t(V) + 2) * sizeof(float);
}

template <class T, int V>
static kp_status launch_attn_t(const AttnLaunch& a, hipStream_t s) {
  const int ns = attn_splits(a.P, a.k, a.n_q);
  const int64_t blocks = (int64_t(a.k) * a.P + AT_NT - 1) / AT_NT;
  const int bps = int((blocks + ns - 1) / ns);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (ns > 1) {
    part_o = reinterpret_cast<float*>(a.ws);
    part_ml = part_o + size_t(a.n_q) * ns * a.H * a.V;
  }
  const float scale_log2 = a.scale * 1.4426950408889634f;
  attn_kernel<T, V><<<dim3(unsigned(int64_t(a.n_q) * ns)), dim3(256), 0, s>>>(
      (const T*)a.latent, a.L, a.bt, a.bt_stride, a.log2_pt, (const T*)a.q, a.q_seq, a.q_pos, a.sel, a.n_sel,
      ilog2(a.P), a.k, a.H, scale_log2, ns, bps, (T*)a.out, a.lse, part_o, part_ml);
  kp_status st = check_launch("sparse_mla_attn");
  if (st != KP_OK || ns == 1) return st;
  attn_combine_kernel<T><<<dim3(unsigned(int64_t(a.n_q) * a.H)), dim3(256), 0, s>>>(part_o, part_ml, ns, a.H, a.V,
                                                                                     (T*)a.out, a.lse);
  return check_launch("sparse_mla_attn (split merge)");
}

kp_status launch_attn(const AttnLaunch& a, hipStream_t s) {
  if (a.n_q == 0) return KP_OK;
  if (int64_t(a.n_q) * attn_splits(a.P, a.k, a.n_q) > 0x7fffffff) {
    set_error("sparse_mla_attn: too many queries for one launch");
    return KP_ERR_INVALID_ARG;
  }
  if (a.dtype == KP_DTYPE_BF16) {
    if (a.V == 512) return launch_attn_t<bf16, 512>(a, s);
    return launch_attn_t<bf16, 64>(a, s);
  }
  return launch_attn_t<float, 64>(a, s);
}

}  // namespace kp
