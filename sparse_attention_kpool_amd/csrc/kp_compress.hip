// kpool_compress: one pooled index key per complete pool.
//
// [MAX glm5_next API page, index_kpool_compress]: the pooled key is a learned weighted average of the pool's
// tokens, the weights coming from gate logits plus an intra-pool position embedding.  [llama.cpp PR "add
// GLM-5.3-Flash (GLM5-Next) support", soft_max crash report]: the softmax runs over each pool's tokens, per
// channel.  One thread per (pool, channel); consecutive threads take consecutive channels, so every key, gate
// and output row is read and written as one coalesced run.  The pool axis is folded into grid x only.
//
// Bound: HBM.  Per pool it moves 2*P*D stored values in and D out -- negligible next to scoring, because a
// decode step completes at most one pool per sequence.
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

template <class T>
__global__ __launch_bounds__(256) void compress_kernel(const T* __restrict__ keys, const T* __restrict__ gates,
                                                       const int32_t* __restrict__ src, const T* __restrict__ ape,
                                                       const int32_t* __restrict__ pool_seq,
                                                       const int32_t* __restrict__ pool_id, T* __restrict__ pooled,
                                                       const int32_t* __restrict__ bt, int bt_stride, int log2_ppp,
                                                       int n_pools, int P, int D) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t i = gid / D;
  const int c = int(gid - i * D);
  if (i >= n_pools) return;
  const int64_t s = src ? src[i] : i;
  const float v = pool_channel<T>(keys + s * P * D + c, gates ? gates + s * P * D + c : nullptr, ape ? ape + c : nullptr,
                                  P, D);
  const int64_t row = paged_row(bt, bt_stride, pool_seq[i], pool_id[i], log2_ppp);
  pooled[row * D + c] = Elem<T>::from_f32(v);
}

kp_status launch_compress(const CompressLaunch& a, hipStream_t s) {
  if (a.n_pools == 0) return KP_OK;
  const int64_t threads = int64_t(a.n_pools) * a.D;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) {
    set_error("kpool_compress: %lld pools x %d channels exceed the grid", (long long)a.n_pools, a.D);
    return KP_ERR_INVALID_ARG;
  }
  if (a.dtype == KP_DTYPE_BF16) {
    compress_kernel<bf16><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(
        (const bf16*)a.keys, (const bf16*)a.gates, a.src, (const bf16*)a.ape, a.pool_seq, a.pool_id,
        (bf16*)a.pooled, a.bt, a.bt_stride, a.log2_ppp, a.n_pools, a.P, a.D);
  } else {
    compress_kernel<float><<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(
        (const float*)a.keys, (const float*)a.gates, a.src, (const float*)a.ape, a.pool_seq, a.pool_id,
        (float*)a.pooled, a.bt, a.bt_stride, a.log2_ppp, a.n_pools, a.P, a.D);
  }
  return check_launch("kpool_compress");
}

}  // namespace kp
