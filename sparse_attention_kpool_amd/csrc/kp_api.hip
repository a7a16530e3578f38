// The extern "C" entry points declared in include/kpool.h: argument validation, then one launcher per call.
// Nothing here touches device memory or synchronises; a validation failure launches nothing.
#include <stdarg.h>
#include <math.h>
#include <stdio.h>

#include "kp_internal.hpp"

namespace kp {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

kp_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return KP_ERR_LAUNCH;
  }
  return KP_OK;
}

static bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
static bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define KP_REQUIRE(cond, code, ...) \
  do {                              \
    if (!(cond)) {                  \
      set_error(__VA_ARGS__);       \
      return code;                  \
    }                               \
  } while (0)

static kp_status check_dims(const kp_dims* d, const char* fn) {
  KP_REQUIRE(d, KP_ERR_INVALID_ARG, "%s: dims is NULL", fn);
  KP_REQUIRE(d->dtype == KP_DTYPE_F32 || d->dtype == KP_DTYPE_BF16, KP_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn,
             d->dtype);
  KP_REQUIRE(pow2(d->pool) && d->pool <= 32, KP_ERR_INVALID_ARG, "%s: pool must be a power of two in 1..32 (got %d)",
             fn, d->pool);
  KP_REQUIRE(d->idx_dim >= 1 && d->idx_heads >= 1 && d->heads >= 1, KP_ERR_INVALID_ARG,
             "%s: idx_dim, idx_heads and heads must be >= 1", fn);
  KP_REQUIRE(d->topk >= 1, KP_ERR_INVALID_ARG, "%s: topk must be >= 1 (got %d)", fn, d->topk);
  KP_REQUIRE(d->v_dim >= 1 && d->v_dim <= d->latent_dim, KP_ERR_INVALID_ARG,
             "%s: need 1 <= v_dim <= latent_dim (got %d, %d)", fn, d->v_dim, d->latent_dim);
  KP_REQUIRE(pow2(d->page_tokens) && d->page_tokens % d->pool == 0, KP_ERR_INVALID_ARG,
             "%s: page_tokens must be a power of two and a multiple of pool (got %d, pool %d)", fn, d->page_tokens,
             d->pool);
  return KP_OK;
}

static kp_status check_cache(const kp_cache* c, bool need_latent, bool need_pooled, const char* fn) {
  KP_REQUIRE(c, KP_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  KP_REQUIRE(c->block_table, KP_ERR_INVALID_ARG, "%s: block_table is NULL", fn);
  KP_REQUIRE(c->bt_stride >= 1, KP_ERR_INVALID_ARG, "%s: bt_stride must be >= 1", fn);
  if (need_latent) KP_REQUIRE(c->latent && aligned(c->latent), KP_ERR_INVALID_ARG, "%s: latent NULL or misaligned", fn);
  if (need_pooled) KP_REQUIRE(c->pooled && aligned(c->pooled), KP_ERR_INVALID_ARG, "%s: pooled NULL or misaligned", fn);
  return KP_OK;
}

static kp_status check_queries(const kp_queries* q, const char* fn) {
  KP_REQUIRE(q, KP_ERR_INVALID_ARG, "%s: queries is NULL", fn);
  KP_REQUIRE(q->n_q >= 0, KP_ERR_INVALID_ARG, "%s: n_q < 0", fn);
  if (q->n_q == 0) return KP_OK;
  KP_REQUIRE(q->seq && q->pos, KP_ERR_INVALID_ARG, "%s: queries seq/pos NULL", fn);
  KP_REQUIRE(q->max_pos >= 0, KP_ERR_INVALID_ARG, "%s: max_pos < 0", fn);
  return KP_OK;
}

static bool score_built(const kp_dims* d) {
  return (d->dtype == KP_DTYPE_BF16 && (d->idx_dim == 128 || d->idx_dim == 32)) ||
         (d->dtype == KP_DTYPE_F32 && d->idx_dim == 32);
}

static bool attn_built(const kp_dims* d) {
  return (d->dtype == KP_DTYPE_BF16 && (d->v_dim == 512 || d->v_dim == 64)) ||
         (d->dtype == KP_DTYPE_F32 && d->v_dim == 64);
}

static size_t elem_size(const kp_dims* d) { return d->dtype == KP_DTYPE_BF16 ? 2 : 4; }

}  // namespace kp

using namespace kp;

extern "C" {

int32_t kp_abi_version(void) { return 7; }

const char* kp_last_error(void) { return g_err; }

// Validation and launch record of kpool_compress (KP_OK with a.n_pools == 0: nothing to pool).
static kp_status compress_prepare(const char* fn, const kp_dims* dims, const kp_cache* cache, int32_t n_pools,
                                  const void* keys, const void* gates, const int32_t* src, const void* ape,
                                  const int32_t* pool_seq, const int32_t* pool_id, CompressLaunch& a) {
  a = CompressLaunch{};
  kp_status st = check_dims(dims, fn);
  if (st != KP_OK) return st;
  st = check_cache(cache, false, true, fn);
  if (st != KP_OK) return st;
  KP_REQUIRE(n_pools >= 0, KP_ERR_INVALID_ARG, "%s: n_pools < 0", fn);
  if (n_pools == 0) return KP_OK;
  KP_REQUIRE(keys && pool_seq && pool_id, KP_ERR_INVALID_ARG, "%s: NULL input", fn);
  KP_REQUIRE(aligned(keys) && (!gates || aligned(gates)) && (!ape || aligned(ape)), KP_ERR_INVALID_ARG,
             "%s: misaligned input", fn);
  a.dtype = dims->dtype;
  a.P = dims->pool;
  a.D = dims->idx_dim;
  a.n_pools = n_pools;
  a.log2_ppp = ilog2(dims->page_tokens / dims->pool);
  a.bt_stride = cache->bt_stride;
  a.keys = keys;
  a.gates = gates;
  a.src = src;
  a.ape = ape;
  a.pool_seq = pool_seq;
  a.pool_id = pool_id;
  a.pooled = cache->pooled;
  a.bt = cache->block_table;
  return KP_OK;
}

// Validation and launch record of dsa_indexer_score (KP_OK with a.n_q == 0: nothing to score).
static kp_status score_prepare(const char* fn, const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                               const void* q_idx, const float* w, float* scores, int64_t ld_scores, ScoreLaunch& a) {
  a = ScoreLaunch{};
  kp_status st = check_dims(dims, fn);
  if (st != KP_OK) return st;
  st = check_queries(queries, fn);
  if (st != KP_OK) return st;
  if (queries->n_q == 0) return KP_OK;
  st = check_cache(cache, false, true, fn);
  if (st != KP_OK) return st;
  KP_REQUIRE(score_built(dims), KP_ERR_UNSUPPORTED, "%s: idx_dim %d with dtype %d is not built (bf16: 32, 128; f32: 32)",
             fn, dims->idx_dim, dims->dtype);
  KP_REQUIRE(dims->idx_heads <= 32, KP_ERR_UNSUPPORTED, "%s: idx_heads %d > 32", fn, dims->idx_heads);
  KP_REQUIRE(q_idx && w && scores, KP_ERR_INVALID_ARG, "%s: NULL q_idx, w or scores", fn);
  KP_REQUIRE(aligned(q_idx) && aligned(w) && aligned(scores), KP_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  const int64_t need = (int64_t(queries->max_pos) + 1) / dims->pool;
  KP_REQUIRE(ld_scores >= need && ld_scores >= 1, KP_ERR_INVALID_ARG, "%s: ld_scores %lld < %lld visible pools", fn,
             (long long)ld_scores, (long long)need);
  KP_REQUIRE(ld_scores % 4 == 0, KP_ERR_INVALID_ARG, "%s: ld_scores %lld is not a multiple of 4", fn,
             (long long)ld_scores);
  a.dtype = dims->dtype;
  a.P = dims->pool;
  a.D = dims->idx_dim;
  a.Hi = dims->idx_heads;
  a.n_q = queries->n_q;
  a.max_pos = queries->max_pos;
  a.group = queries->group;
  a.log2_ppp = ilog2(dims->page_tokens / dims->pool);
  a.bt_stride = cache->bt_stride;
  a.pooled = cache->pooled;
  a.bt = cache->block_table;
  a.q_idx = q_idx;
  a.w = w;
  a.q_seq = queries->seq;
  a.q_pos = queries->pos;
  a.scores = scores;
  a.ld = ld_scores;
  return KP_OK;
}

kp_status kpool_compress(const kp_dims* dims, const kp_cache* cache, int32_t n_pools, const void* keys,
                         const void* gates, const int32_t* src, const void* ape, const int32_t* pool_seq,
                         const int32_t* pool_id, void* stream) {
  CompressLaunch a;
  const kp_status st = compress_prepare("kpool_compress", dims, cache, n_pools, keys, gates, src, ape, pool_seq,
                                        pool_id, a);
  if (st != KP_OK || a.n_pools == 0) return st;
  return launch_compress(a, (hipStream_t)stream);
}

kp_status dsa_indexer_score(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                            const void* q_idx, const float* w, float* scores, int64_t ld_scores, void* stream) {
  ScoreLaunch a;
  const kp_status st = score_prepare("dsa_indexer_score", dims, cache, queries, q_idx, w, scores, ld_scores, a);
  if (st != KP_OK || a.n_q == 0) return st;
  return launch_score(a, (hipStream_t)stream);
}

kp_status dsa_compress_score(const kp_dims* dims, const kp_cache* cache, int32_t n_pools, const void* keys,
                             const void* gates, const int32_t* src, const void* ape, const int32_t* pool_seq,
                             const int32_t* pool_id, const kp_queries* queries, const void* q_idx, const float* w,
                             float* scores, int64_t ld_scores, void* stream) {
  const char* fn = "dsa_compress_score";
  CompressLaunch c;
  kp_status st = compress_prepare(fn, dims, cache, n_pools, keys, gates, src, ape, pool_seq, pool_id, c);
  if (st != KP_OK) return st;
  ScoreLaunch a;
  st = score_prepare(fn, dims, cache, queries, q_idx, w, scores, ld_scores, a);
  if (st != KP_OK) return st;
  if (a.n_q == 0) return c.n_pools ? launch_compress(c, (hipStream_t)stream) : KP_OK;
  if (c.n_pools == 0) return launch_score(a, (hipStream_t)stream);
  return launch_compress_score(c, a, (hipStream_t)stream);
}

size_t dsa_topk_workspace_size(const kp_dims* dims, const kp_queries* queries) {
  if (!dims || !queries) return 0;
  return topk_workspace(dims->pool, dims->topk, queries->n_q, queries->max_pos);
}

kp_status dsa_topk_select(const kp_dims* dims, const kp_queries* queries, const float* scores, int64_t ld_scores,
                          int32_t* sel, int32_t* n_sel, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "dsa_topk_select";
  kp_status st = check_dims(dims, fn);
  if (st != KP_OK) return st;
  st = check_queries(queries, fn);
  if (st != KP_OK) return st;
  if (queries->n_q == 0) return KP_OK;
  KP_REQUIRE(scores && sel && n_sel, KP_ERR_INVALID_ARG, "%s: NULL scores, sel or n_sel", fn);
  KP_REQUIRE(aligned(scores) && aligned(sel) && aligned(n_sel), KP_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  const int64_t need = (int64_t(queries->max_pos) + 1) / dims->pool;
  KP_REQUIRE(ld_scores >= need && ld_scores >= 1, KP_ERR_INVALID_ARG, "%s: ld_scores %lld < %lld visible pools", fn,
             (long long)ld_scores, (long long)need);
  KP_REQUIRE(ld_scores % 4 == 0, KP_ERR_INVALID_ARG, "%s: ld_scores %lld is not a multiple of 4", fn,
             (long long)ld_scores);
  const size_t ws_need = topk_workspace(dims->pool, dims->topk, queries->n_q, queries->max_pos);
  KP_REQUIRE(ws_bytes >= ws_need && (ws_need == 0 || workspace), KP_ERR_WORKSPACE,
             "%s: workspace of %zu bytes < %zu required", fn, ws_bytes, ws_need);
  TopkLaunch a{};
  a.P = dims->pool;
  a.k = dims->topk;
  a.n_q = queries->n_q;
  a.max_pos = queries->max_pos;
  a.scores = scores;
  a.ld = ld_scores;
  a.q_pos = queries->pos;
  a.sel = sel;
  a.n_sel = n_sel;
  a.ws = workspace;
  a.ws_bytes = ws_bytes;
  return launch_topk(a, (hipStream_t)stream);
}

size_t sparse_mla_workspace_size(const kp_dims* dims, const kp_queries* queries) {
  if (!dims || !queries || queries->n_q <= 0 || dims->pool < 1 || dims->topk < 1) return 0;
  return attn_workspace(dims->pool, dims->topk, dims->heads, dims->v_dim, queries->n_q, int(elem_size(dims)));
}

size_t sparse_mla_mtp_workspace_size(const kp_dims* dims, const kp_queries* queries) {
  if (!dims || !queries || queries->n_q <= 0 || dims->pool < 1 || dims->topk < 1 || dims->heads < 1) return 0;
  return attn_workspace_mtp(dims->pool, dims->topk, dims->heads, dims->v_dim, queries->n_q, int(elem_size(dims)));
}

// Shared body of the attention calls (fp8: latent rows of latent_dim E4M3 codes; mtp: runs of a target and its
// draft attending selection row i / 2).
static kp_status attn_call(const char* fn, bool fp8, float kv_scale, const kp_dims* dims, const kp_cache* cache,
                           const kp_queries* queries, const void* q, const int32_t* sel, const int32_t* n_sel,
                           const int32_t* sel_row, void* out, float* lse, void* workspace, size_t ws_bytes,
                           void* stream, bool mtp = false) {
  kp_status st = check_dims(dims, fn);
  if (st != KP_OK) return st;
  st = check_queries(queries, fn);
  if (st != KP_OK) return st;
  if (queries->n_q == 0) return KP_OK;
  st = check_cache(cache, true, false, fn);
  if (st != KP_OK) return st;
  if (fp8) {
    KP_REQUIRE(dims->dtype == KP_DTYPE_BF16 && dims->v_dim == 512, KP_ERR_UNSUPPORTED,
               "%s: built for bf16 queries and output with v_dim 512 (got dtype %d, v_dim %d)", fn, dims->dtype,
               dims->v_dim);
    KP_REQUIRE(kv_scale > 0.f && kv_scale < INFINITY, KP_ERR_INVALID_ARG, "%s: kv_scale must be finite and > 0",
               fn);
  } else {
    KP_REQUIRE(attn_built(dims), KP_ERR_UNSUPPORTED,
               "%s: v_dim %d with dtype %d is not built (bf16: 512, 64; f32: 64)", fn, dims->v_dim, dims->dtype);
  }
  KP_REQUIRE(dims->heads <= 64, KP_ERR_UNSUPPORTED, "%s: heads %d > 64", fn, dims->heads);
  if (mtp)
    KP_REQUIRE(dims->dtype == KP_DTYPE_BF16 && dims->v_dim == 512, KP_ERR_UNSUPPORTED,
               "%s: built for bf16 with v_dim 512 (got dtype %d, v_dim %d)", fn, dims->dtype, dims->v_dim);
  const int64_t lat_es = fp8 ? 1 : int64_t(elem_size(dims));
  KP_REQUIRE((int64_t(dims->latent_dim) * lat_es) % 16 == 0, KP_ERR_INVALID_ARG,
             "%s: latent rows must be a multiple of 16 bytes (latent_dim %d)", fn, dims->latent_dim);
  KP_REQUIRE(q && sel && n_sel && out, KP_ERR_INVALID_ARG, "%s: NULL q, sel, n_sel or out", fn);
  KP_REQUIRE(aligned(q) && aligned(sel) && aligned(n_sel) && aligned(out) && (!lse || aligned(lse)) &&
                 (!sel_row || aligned(sel_row)),
             KP_ERR_INVALID_ARG, "%s: misaligned buffer", fn);
  const size_t ws_need =
      mtp ? attn_workspace_mtp(dims->pool, dims->topk, dims->heads, dims->v_dim, queries->n_q, int(elem_size(dims)))
          : attn_workspace(dims->pool, dims->topk, dims->heads, dims->v_dim, queries->n_q, int(elem_size(dims)));
  KP_REQUIRE(ws_bytes >= ws_need && (ws_need == 0 || (workspace && aligned(workspace))), KP_ERR_WORKSPACE,
             "%s: workspace of %zu bytes < %zu required", fn, ws_bytes, ws_need);
  AttnLaunch a{};
  a.mtp = mtp ? 1 : 0;
  a.dtype = dims->dtype;
  a.P = dims->pool;
  a.H = dims->heads;
  a.L = dims->latent_dim;
  a.V = dims->v_dim;
  a.k = dims->topk;
  a.n_q = queries->n_q;
  a.max_pos = queries->max_pos;
  a.log2_pt = ilog2(dims->page_tokens);
  a.bt_stride = cache->bt_stride;
  a.scale = dims->scale;
  a.latent_fp8 = fp8 ? 1 : 0;
  a.kv_scale = fp8 ? kv_scale : 1.f;
  a.latent = cache->latent;
  a.bt = cache->block_table;
  a.q = q;
  a.q_seq = queries->seq;
  a.q_pos = queries->pos;
  a.sel = sel;
  a.n_sel = n_sel;
  a.sel_row = sel_row;
  a.out = out;
  a.lse = lse;
  a.ws = workspace;
  a.ws_bytes = ws_bytes;
  return launch_attn(a, (hipStream_t)stream);
}

kp_status sparse_mla_attn(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries, const void* q,
                          const int32_t* sel, const int32_t* n_sel, void* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream) {
  return attn_call("sparse_mla_attn", false, 1.f, dims, cache, queries, q, sel, n_sel, nullptr, out, lse, workspace,
                   ws_bytes, stream);
}

kp_status sparse_mla_attn_shared(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                                 const void* q, const int32_t* sel, const int32_t* n_sel, const int32_t* sel_row,
                                 void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  KP_REQUIRE(sel_row || !queries || queries->n_q == 0, KP_ERR_INVALID_ARG, "sparse_mla_attn_shared: NULL sel_row");
  return attn_call("sparse_mla_attn_shared", false, 1.f, dims, cache, queries, q, sel, n_sel, sel_row, out, lse,
                   workspace, ws_bytes, stream);
}

kp_status sparse_mla_attn_mtp(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries, const void* q,
                              const int32_t* sel, const int32_t* n_sel, void* out, float* lse, void* workspace,
                              size_t ws_bytes, void* stream) {
  return attn_call("sparse_mla_attn_mtp", false, 1.f, dims, cache, queries, q, sel, n_sel, nullptr, out, lse,
                   workspace, ws_bytes, stream, true);
}

kp_status sparse_mla_attn_noalloc(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                                  const void* q, const int32_t* sel, const int32_t* n_sel, void* out, float* lse,
                                  void* stream) {
  const char* fn = "sparse_mla_attn_noalloc";
  kp_status st = check_dims(dims, fn);
  if (st != KP_OK) return st;
  st = check_queries(queries, fn);
  if (st != KP_OK) return st;
  if (queries->n_q == 0) return KP_OK;
  const size_t need =
      attn_workspace(dims->pool, dims->topk, dims->heads, dims->v_dim, queries->n_q, int(elem_size(dims)));
  KP_REQUIRE(need <= size_t(KP_NOALLOC_SCRATCH_BYTES), KP_ERR_WORKSPACE,
             "%s: this call needs %zu bytes of split-KV scratch, more than the %zu bytes held per device "
             "(use sparse_mla_attn with a workspace)",
             fn, need, size_t(KP_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0) {
    st = attn_noalloc_scratch(&ws);
    if (st != KP_OK) return st;
  }
  return attn_call(fn, false, 1.f, dims, cache, queries, q, sel, n_sel, nullptr, out, lse, ws, need, stream);
}

kp_status sparse_mla_attn_fp8(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries, const void* q,
                              const int32_t* sel, const int32_t* n_sel, float kv_scale, void* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream) {
  return attn_call("sparse_mla_attn_fp8", true, kv_scale, dims, cache, queries, q, sel, n_sel, nullptr, out, lse,
                   workspace, ws_bytes, stream);
}

}  // extern "C"

// validation of one product and its launch descriptor
static kp_status linear_prepare(const kp_linear_problem& q, const char* fn, LinearLaunch& a) {
  KP_REQUIRE(q.batch >= 0 && q.M >= 0 && q.N >= 0, KP_ERR_INVALID_ARG, "%s: negative batch, M or N", fn);
  a = LinearLaunch{};
  a.batch = q.batch;
  a.M = q.M;
  a.N = q.N;
  a.K = q.K;
  if (q.batch == 0 || q.M == 0 || q.N == 0) {  // empty: nothing is read or written
    a.batch = a.M = a.N = 0;
    return KP_OK;
  }
  KP_REQUIRE(q.K >= 64 && q.K % 64 == 0, KP_ERR_UNSUPPORTED, "%s: K = %d is not a positive multiple of 64", fn, q.K);
  KP_REQUIRE(q.c_dtype == KP_DTYPE_BF16 || q.c_dtype == KP_DTYPE_F32, KP_ERR_INVALID_ARG, "%s: bad c_dtype", fn);
  KP_REQUIRE(q.A && q.W && q.C, KP_ERR_INVALID_ARG, "%s: NULL operand", fn);
  KP_REQUIRE(aligned(q.A) && aligned(q.W) && aligned(q.C), KP_ERR_INVALID_ARG, "%s: misaligned operand", fn);
  KP_REQUIRE(q.lda >= q.K && q.ldw >= q.K && q.ldc >= q.N, KP_ERR_INVALID_ARG, "%s: leading dimension below K or N",
             fn);
  KP_REQUIRE(q.lda % 8 == 0 && q.ldw % 8 == 0 && q.stride_a % 8 == 0 && q.stride_w % 8 == 0 && q.stride_a >= 0 &&
                 q.stride_w >= 0,
             KP_ERR_INVALID_ARG, "%s: A / W row and batch strides must be non-negative multiples of 8", fn);
  KP_REQUIRE(q.ldc % 4 == 0 && q.stride_c % 4 == 0 && q.stride_c >= 0, KP_ERR_INVALID_ARG,
             "%s: C row and batch strides must be non-negative multiples of 4", fn);
  KP_REQUIRE(isfinite(q.alpha), KP_ERR_INVALID_ARG, "%s: alpha is not finite", fn);
  a.c_dtype = q.c_dtype;
  a.A = q.A;
  a.lda = q.lda;
  a.sa = q.stride_a;
  a.W = q.W;
  a.ldw = q.ldw;
  a.sw = q.stride_w;
  a.C = q.C;
  a.ldc = q.ldc;
  a.sc = q.stride_c;
  a.alpha = q.alpha;
  return KP_OK;
}

static kp_status linear_group_prepare(int32_t n, const kp_linear_problem* problems, const char* fn,
                                      LinearLaunch (&a)[8]) {
  KP_REQUIRE(n >= 0 && n <= 8, KP_ERR_INVALID_ARG, "%s: %d products (1..8 per call)", fn, n);
  KP_REQUIRE(n == 0 || problems, KP_ERR_INVALID_ARG, "%s: NULL problem list", fn);
  for (int i = 0; i < n; ++i) {
    const kp_status st = linear_prepare(problems[i], fn, a[i]);
    if (st != KP_OK) return st;
  }
  return KP_OK;
}

extern "C" {

size_t kp_linear_group_workspace_size(int32_t n, const kp_linear_problem* problems) {
  LinearLaunch a[8];
  if (linear_group_prepare(n, problems, "kp_linear_group_workspace_size", a) != KP_OK) return 0;
  return linear_group_workspace(a, n);
}

kp_status kp_linear_group(int32_t n, const kp_linear_problem* problems, void* workspace, size_t ws_bytes,
                          void* stream) {
  const char* fn = "kp_linear_group";
  LinearLaunch a[8];
  const kp_status st = linear_group_prepare(n, problems, fn, a);
  if (st != KP_OK) return st;
  KP_REQUIRE(!workspace || aligned(workspace), KP_ERR_INVALID_ARG, "%s: misaligned workspace", fn);
  return launch_linear_group(a, n, workspace, workspace ? ws_bytes : 0, (hipStream_t)stream);
}

static kp_linear_problem one_problem(int32_t batch, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                                     int64_t stride_a, const void* W, int64_t ldw, int64_t stride_w, void* C,
                                     int64_t ldc, int64_t stride_c, int32_t c_dtype, float alpha) {
  kp_linear_problem q;
  q.batch = batch;
  q.M = M;
  q.N = N;
  q.K = K;
  q.A = A;
  q.lda = lda;
  q.stride_a = stride_a;
  q.W = W;
  q.ldw = ldw;
  q.stride_w = stride_w;
  q.C = C;
  q.ldc = ldc;
  q.stride_c = stride_c;
  q.c_dtype = c_dtype;
  q.alpha = alpha;
  return q;
}

kp_status kp_read_rows(const void* base, int64_t row_stride, int32_t row_bytes, const int32_t* rows, int64_t n_rows,
                       int32_t blocks_per_cu, void* stream) {
  const char* fn = "kp_read_rows";
  KP_REQUIRE(n_rows >= 0, KP_ERR_INVALID_ARG, "%s: n_rows < 0", fn);
  if (n_rows == 0) return KP_OK;
  KP_REQUIRE(base && rows && aligned(base), KP_ERR_INVALID_ARG, "%s: NULL or misaligned base / rows", fn);
  KP_REQUIRE(row_bytes == 1024 || row_bytes == 4096, KP_ERR_INVALID_ARG,
             "%s: row_bytes must be 1024 (a value row) or 4096 (a page of pooled keys), got %d", fn, row_bytes);
  KP_REQUIRE(row_stride >= row_bytes && row_stride % 16 == 0, KP_ERR_INVALID_ARG,
             "%s: row_stride must be >= row_bytes and a multiple of 16", fn);
  KP_REQUIRE(blocks_per_cu >= 1 && blocks_per_cu <= 8, KP_ERR_INVALID_ARG, "%s: blocks_per_cu in 1..8", fn);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus <= 0)
    cus = 256;
  return launch_read_rows(base, row_stride, row_bytes, rows, n_rows, cus * blocks_per_cu, (hipStream_t)stream);
}

size_t kp_linear_workspace_size(int32_t batch, int32_t M, int32_t N, int32_t K) {
  // only the shape matters: stand-in operands that pass validation
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  const kp_linear_problem q = one_problem(batch, M, N, K, dummy, K, 0, dummy, K, 0, (void*)dummy, N + (4 - N % 4) % 4,
                                          0, KP_DTYPE_F32, 1.f);
  return kp_linear_group_workspace_size(1, &q);
}

kp_status kp_linear(int32_t batch, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int64_t stride_a,
                    const void* W, int64_t ldw, int64_t stride_w, void* C, int64_t ldc, int64_t stride_c,
                    int32_t c_dtype, float alpha, void* workspace, size_t ws_bytes, void* stream) {
  const kp_linear_problem q =
      one_problem(batch, M, N, K, A, lda, stride_a, W, ldw, stride_w, C, ldc, stride_c, c_dtype, alpha);
  const char* fn = "kp_linear";
  LinearLaunch a;
  const kp_status st = linear_prepare(q, fn, a);
  if (st != KP_OK) return st;
  KP_REQUIRE(!workspace || aligned(workspace), KP_ERR_INVALID_ARG, "%s: misaligned workspace", fn);
  return launch_linear_group(&a, 1, workspace, workspace ? ws_bytes : 0, (hipStream_t)stream);
}

}  // extern "C"
