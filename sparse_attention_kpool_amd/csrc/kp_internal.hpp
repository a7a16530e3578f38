// Host-side declarations shared between the C entry points (kp_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kpool.h"

namespace kp {

// Records the message returned by kp_last_error() on this thread.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Checks hipGetLastError() after a launch; KP_ERR_LAUNCH with the message on failure.
kp_status check_launch(const char* what);

inline int ilog2(int64_t v) {
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

struct CompressLaunch {
  int dtype, P, D, n_pools, log2_ppp, bt_stride;
  const void* keys;
  const void* gates;
  const int32_t* src;
  const void* ape;
  const int32_t* pool_seq;
  const int32_t* pool_id;
  void* pooled;
  const int32_t* bt;
};
kp_status launch_compress(const CompressLaunch& a, hipStream_t s);

struct ScoreLaunch {
  int dtype, P, D, Hi, n_q, max_pos, group, log2_ppp, bt_stride;
  const void* pooled;
  const int32_t* bt;
  const void* q_idx;
  const float* w;
  const int32_t* q_seq;
  const int32_t* q_pos;
  float* scores;
  int64_t ld;
};
kp_status launch_score(const ScoreLaunch& a, hipStream_t s);
// launch_compress(c) then launch_score(a), in one launch where the decode scorer can pool c's entries itself
kp_status launch_compress_score(const CompressLaunch& c, const ScoreLaunch& a, hipStream_t s);

struct TopkLaunch {
  int P, k, n_q, max_pos;
  const float* scores;
  int64_t ld;
  const int32_t* q_pos;
  int32_t* sel;
  int32_t* n_sel;
  void* ws;
  size_t ws_bytes;
};
size_t topk_workspace(int P, int k, int n_q, int max_pos);
kp_status launch_topk(const TopkLaunch& a, hipStream_t s);

struct AttnLaunch {
  int dtype, P, H, L, V, k, n_q, max_pos, log2_pt, bt_stride;
  float scale;
  int latent_fp8;   // latent cache of E4M3 codes (bf16 queries and output, V = 512)
  float kv_scale;   // its scale (value = code value * kv_scale)
  const void* latent;
  const int32_t* bt;
  const void* q;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* sel;
  const int32_t* n_sel;
  const int32_t* sel_row;  // query i attends selection row sel_row[i] (NULL: row i)
  int mtp;                 // runs of a target and its draft attending selection row i / 2 (sparse_mla_attn_mtp)
  void* out;
  float* lse;
  void* ws;
  size_t ws_bytes;
};
// Number of split-KV partitions per query for a call shape (a pure function of its arguments).
int attn_splits(int P, int k, int n_q);
size_t attn_workspace(int P, int k, int H, int V, int n_q, int esize);
// The same for sparse_mla_attn_mtp's launch (n_q queries in runs of two).
int attn_splits_mtp(int P, int k, int n_q, int H);
size_t attn_workspace_mtp(int P, int k, int H, int V, int n_q, int esize);
kp_status launch_attn(const AttnLaunch& a, hipStream_t s);
// Device address of the current device's static split-KV scratch (KP_NOALLOC_SCRATCH_BYTES), looked up on the
// first call per device.
kp_status attn_noalloc_scratch(void** ptr);

kp_status launch_read_rows(const void* base, int64_t row_stride, int32_t row_bytes, const int32_t* rows,
                           int64_t n_rows, int blocks, hipStream_t s);

struct LinearLaunch {
  int batch, M, N, K, c_dtype;
  const void* A;
  int64_t lda, sa;
  const void* W;
  int64_t ldw, sw;
  void* C;
  int64_t ldc, sc;
  float alpha;
};
// up to 8 products in one launch (plus one split-K reduce launch); one tile shape for all, by the largest M
size_t linear_group_workspace(const LinearLaunch* probs, int n);
kp_status launch_linear_group(const LinearLaunch* probs, int n, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace kp
