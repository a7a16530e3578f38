/*
 * kpool.h -- C ABI of the KPool-DSA sparse-attention layer (GLM-5.3-Flash) for AMD Instinct MI355X (gfx950).
 *
 * The layer runs in four calls, each a hand-written HIP kernel enqueued on the caller's stream:
 *
 *   kpool_compress     pools of P consecutive tokens -> one pooled index key per complete pool
 *   dsa_indexer_score  head-weighted ReLU scores of the complete pools each query may see
 *   dsa_topk_select    causal top-k pools per query, the incomplete tail pool always kept
 *   sparse_mla_attn    nope-only absorbed MLA of each query over the tokens of its selected pools
 *
 * and, beside them, kp_linear: the dense projections that feed and follow the path (indexer query, head
 * weights and key | gate; the MLA query absorb and output un-absorb).  dsa_compress_score runs the first two
 * calls as one (one launch for a decode batch).
 *
 * Sources (page title, section):
 *   [MAX "max.pipelines.architectures.glm5_next" API page]: fields index_kpool (tokens per scoring pool),
 *     index_kpool_always_select_tail, index_kpool_compress (gate logits plus a learned intra-pool position
 *     embedding weight each pool's tokens), mla_use_nope (no rotary embedding), build_layers() (576-wide latent
 *     carrying 64 rotary columns that are all zero), mla_head_dim.
 *   [llama.cpp pull request "add GLM-5.3-Flash (GLM5-Next) support", "What I implemented new"]: pools of 4
 *     consecutive tokens are scored and the incomplete tail is always kept; the indexer cache holds key and gate
 *     per token; attention layers are nope-only MLA.  Same page, soft_max crash report: the pooling softmax is
 *     over each pool's 4 tokens per channel, and a launch that put the pool axis on grid y failed beyond 65,535
 *     pools -- here no grid axis other than x ever scales with pools, tokens or queries.
 *   [GLM-5.3-Flash model card, "Raw config fields"]: index_head_dim 128, index_n_heads 32, index_kpool 4,
 *     index_topk 2048, kv_lora_rank 512, num_attention_heads 64, qk_head_dim 256.
 *   The layer's specification fixes what the pages leave open: pooling = softmax over (gate + position term)
 *   within the pool, then a weighted sum of the keys; score = sum_h w_h * ReLU(q_h . k_pool); ties toward the
 *   lower pool index.
 *
 * Conventions shared by every call
 *   - Ownership: the caller owns every buffer.  The library allocates no device memory and keeps no state
 *     between calls; scratch comes in through the workspace arguments, sized by the *_workspace_size queries.
 *   - Pointers: "device" pointers are HIP device memory; "host" pointers are read during the call only.
 *     Device buffers must be 16-byte aligned.
 *   - Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the null stream) with no host or device
 *     synchronisation.  Calls on different streams are safe when their outputs do not overlap.
 *   - Errors: each call returns a kp_status.  On a validation failure nothing is launched and kp_last_error()
 *     (thread-local) says why.  KP_ERR_LAUNCH reports the HIP launch error.  Faults inside a kernel surface at
 *     the caller's next synchronisation.  The library never aborts the process.
 *   - Data contract (not checked): positions lie within the caches' filled extent, block-table entries that a
 *     query can reach are valid pages, the rotary columns v_dim..latent_dim-1 of q and of the latent cache are
 *     zero, values are finite, every queries->pos[i] <= queries->max_pos.
 *   - Positions: a query at absolute position i (0-based) sees the complete pools p < n_c = (i+1) / P; its
 *     trailing pool tau = i / P is incomplete when r = (i+1) mod P != 0 and then holds tokens P*tau .. i.
 *   - Paging: both caches share one block table of physical page ids.  A page holds `page_tokens` latent rows
 *     and `page_tokens / pool` pooled-key rows; page_tokens is a power of two and a multiple of `pool`, so no
 *     pool straddles a page.  A contiguous cache is a block table 0, 1, 2, ...
 *   - Widths: pool ids, positions and counts are int32; all byte offsets are computed in 64 bits.
 */
#ifndef KPOOL_H
#define KPOOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KP_OK = 0,
  KP_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misaligned buffer, inconsistent dims           */
  KP_ERR_UNSUPPORTED = -2,   /* valid but not built: dtype / head dim / value width combination       */
  KP_ERR_WORKSPACE = -3,     /* workspace missing or smaller than the matching *_workspace_size query */
  KP_ERR_LAUNCH = -4         /* the HIP launch failed; kp_last_error() holds hipGetErrorString         */
} kp_status;

typedef enum { KP_DTYPE_F32 = 0, KP_DTYPE_BF16 = 1 } kp_dtype;

/* Layer dimensions (host struct, read during the call only). */
typedef struct {
  int32_t pool;        /* P: tokens per pool (index_kpool = 4); power of two, 1..32                         */
  int32_t idx_dim;     /* D: index head dim (128); built: 32, 128                                            */
  int32_t idx_heads;   /* Hi: index heads (32); 1..32                                                        */
  int32_t topk;        /* k: pools kept per query, the forced tail included (2048); >= 1                     */
  int32_t heads;       /* H: MLA heads (64); 1..64                                                           */
  int32_t latent_dim;  /* L: latent row width (576 = 512 + 64 zero rotary columns); >= v_dim                */
  int32_t v_dim;       /* V: value / nope width (512); built: 512, 64 (64 also for f32)                      */
  int32_t page_tokens; /* tokens per cache page; power of two, multiple of pool                              */
  int32_t dtype;       /* kp_dtype: storage type of keys, gates, ape, q_idx, q, both caches and out          */
  float scale;         /* attention softmax scale (1/sqrt(qk_head_dim) = 1/16 for the model)                 */
} kp_dims;

/* The two paged caches of one layer (host struct; the pointers are device memory). */
typedef struct {
  void* latent;                /* [n_pages, page_tokens, latent_dim] storage dtype                           */
  void* pooled;                /* [n_pages, page_tokens / pool, idx_dim] storage dtype                       */
  const int32_t* block_table;  /* [n_seq, bt_stride] physical page ids                                       */
  int32_t bt_stride;           /* entries per block-table row                                                */
} kp_cache;

/* A batch of queries (host struct; seq and pos are device arrays). */
typedef struct {
  int32_t n_q;                 /* number of queries; 0 is a valid empty call                                 */
  const int32_t* seq;          /* [n_q] block-table row of each query's sequence                             */
  const int32_t* pos;          /* [n_q] absolute 0-based position of each query                              */
  int32_t max_pos;             /* host: an upper bound of pos[]; sizes the grids without a device sync       */
  int32_t group;               /* host hint: runs of `group` consecutive queries that share a sequence (a
                                  prefill chunk); 1 = no promise.  Results never depend on it: a run that
                                  breaks the promise is processed one query at a time.                       */
} kp_queries;

/*
 * kpool_compress -- pooled index keys of complete pools.
 *   [MAX glm5_next API page, index_kpool_compress]; [llama.cpp PR, "What I implemented new"; soft_max crash
 *   report: softmax over a pool's tokens per channel]; formula per the layer's specification.
 *   For pool i (0 <= i < n_pools), channel c < D and token j < P of the pool:
 *     z_j = gate[j, c] + ape[j, c];  a = softmax_j(z);  pooled[c] = sum_j a_j * key[j, c]
 *   computed in fp32 as key[0,c] + sum_j a_j * (key[j,c] - key[0,c]) (equal in exact arithmetic; it makes a
 *   constant key pool to exactly that key), rounded once (nearest-even) to the storage dtype and written to
 *   row pool_id[i] of sequence pool_seq[i] of the pooled cache.
 *   keys, gates: device [n_src, P, D]; pool i reads source row src[i] (src NULL: row i).  A decode step passes
 *     its per-sequence ring of pending key/gate rows directly, with src = the sequences whose pool completes.
 *   ape: device [P, D].  pool_seq, pool_id: device [n_pools].
 *   gates and ape may each be NULL, meaning zero gate logits / a zero position term.  Both NULL is the
 *     non-learned pooling [MAX glm5_next API page, index_kpool_compress off]: the plain mean of the pool's keys.
 *   Errors: KP_ERR_INVALID_ARG on null keys, pool_seq or pool_id (n_pools > 0) or bad dims.
 */
kp_status kpool_compress(const kp_dims* dims, const kp_cache* cache, int32_t n_pools, const void* keys,
                         const void* gates, const int32_t* src, const void* ape, const int32_t* pool_seq,
                         const int32_t* pool_id, void* stream);

/*
 * dsa_indexer_score -- scores of every complete pool each query can see.
 *   [llama.cpp PR, "What I implemented new": the indexer scores pools]; [GLM-5.3-Flash model card, "Raw
 *   config fields": 32 index heads of dim 128]; formula per the layer's specification:
 *     scores[q, p] = sum_{h < Hi} w[q, h] * max(0, sum_{c < D} q_idx[q, h, c] * pooled[seq(q), p, c])
 *   for p < n_c(pos(q)), accumulated in fp32 (products of storage values are exact in fp32).  One pooled key
 *   per pool serves every index head.  Columns p >= n_c(pos(q)) of a row are not written.
 *   q_idx: device [n_q, Hi, D] storage dtype; w: device [n_q, Hi] fp32 (any sign).
 *   scores: device fp32 [n_q, ld_scores], ld_scores >= (max_pos + 1) / P and a multiple of 4 (16-byte rows).
 *   MFMA: 32 index heads form the M side of a 32x32x16 bf16 (32x32x2 f32) tile; pools are N; D is K.
 *   Errors: KP_ERR_INVALID_ARG (null pointers, ld_scores too small), KP_ERR_UNSUPPORTED (D, dtype).
 */
kp_status dsa_indexer_score(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                            const void* q_idx, const float* w, float* scores, int64_t ld_scores, void* stream);

/*
 * dsa_compress_score -- kpool_compress followed by dsa_indexer_score, as one call.
 *   [llama.cpp PR, "What I implemented new": a decode step pools the keys of the tokens that complete a pool, then
 *   the indexer scores the pools]; [MAX glm5_next API page, per-request state: indexer tail rings, read here as
 *   each sequence's pending rows of its incomplete pool].  The arguments are kpool_compress's (dims, cache,
 *   n_pools .. pool_id) then dsa_indexer_score's (queries .. ld_scores), with the same meaning, layouts and checks.
 *   The results are exactly those of the two calls in that order: the pooled rows written, and scores computed
 *   over the cache with those rows in it.
 *   A decode batch (queries->group < 8) with 1 .. 64 pools to pool takes ONE launch: the scorer pools those
 *   entries itself (the rows are still written to the cache), saving the second launch and the wait between the
 *   two kernels.  Anything else runs the two kernels in order.  In either case the rows of the listed pools must
 *   not be read or written by other work in flight.
 *   Errors: those of kpool_compress and dsa_indexer_score; nothing is launched on an error.
 */
kp_status dsa_compress_score(const kp_dims* dims, const kp_cache* cache, int32_t n_pools, const void* keys,
                             const void* gates, const int32_t* src, const void* ape, const int32_t* pool_seq,
                             const int32_t* pool_id, const kp_queries* queries, const void* q_idx, const float* w,
                             float* scores, int64_t ld_scores, void* stream);

/*
 * dsa_topk_select -- causal top-k pools of each query, the incomplete tail forced.
 *   [MAX glm5_next API page, index_kpool_always_select_tail: the incomplete trailing pool is always visible];
 *   [llama.cpp PR, "What I implemented new": always keeps the incomplete tail]; [GLM-5.3-Flash model card,
 *   "Raw config fields": index_topk 2048, counted in pools]; ties toward the lower pool index per the layer's
 *   specification.  For a query at position i:
 *     budget = min(k - [r != 0], n_c); keep the `budget` complete pools first in the order (score desc,
 *     pool index asc), with -0.0 equal to +0.0; add tau when r != 0.
 *   sel: device int32 [n_q, k], the kept pool ids ascending, padded with -1; n_sel: device int32 [n_q].
 *   scores: as written by dsa_indexer_score (only columns < n_c are read); ld_scores as there.
 *   workspace: device, at least dsa_topk_workspace_size bytes (NULL when that is 0).  Rows of more than 32768
 *     pools, and the rows of a batch too small to fill the GPU, are selected in two steps through it
 *     (per-chunk candidates, then a final pass); its size depends on n_q and max_pos.
 *   Limit: (max_pos + 1) / P <= 16 * 32768 pools and 16 * topk <= 32768 when two steps are needed, else
 *     KP_ERR_UNSUPPORTED (covers 1M-token contexts at P = 4, topk = 2048).
 *   Errors: KP_ERR_INVALID_ARG, KP_ERR_WORKSPACE, KP_ERR_UNSUPPORTED.
 */
size_t dsa_topk_workspace_size(const kp_dims* dims, const kp_queries* queries);
kp_status dsa_topk_select(const kp_dims* dims, const kp_queries* queries, const float* scores,
                          int64_t ld_scores, int32_t* sel, int32_t* n_sel, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * sparse_mla_attn -- nope-only absorbed MLA over the selected tokens.
 *   [llama.cpp PR, "What I implemented new": attention layers are nope-only MLA]; [MAX glm5_next API page,
 *   mla_use_nope (no rotary embedding), build_layers() (576-wide latent, 64 rotary columns all zero)];
 *   [GLM-5.3-Flash model card, "Raw config fields": kv_lora_rank 512, 64 heads].  For query q and head h:
 *     S = tokens of the selected complete pools, plus tokens P*tau .. i of the tail pool when it is selected;
 *     l_t = scale * q[h] . latent[t]  (the key is the latent row; columns >= V are zero by contract and are
 *     not read);  a = softmax_t(l);  out[q, h, :] = sum_t a_t * latent[t, :V];  lse[q, h] = ln sum_t e^{l_t}.
 *   q: device [n_q, H, L] storage dtype; sel / n_sel: as written by dsa_topk_select.
 *   out: device [n_q, H, V] storage dtype (rounded once, nearest-even); lse: device fp32 [n_q, H] or NULL.
 *   Accumulation in fp32; softmax weights enter the value product in the storage dtype.
 *   workspace: device, at least sparse_mla_workspace_size bytes (split-KV partials; NULL when that is 0).
 *     When a query's selection is split over several blocks (batches too small to fill the GPU), each split's
 *     unnormalised partial output is stored in the storage dtype before the merge, so the output of such a
 *     query is rounded twice; the running max and sum stay fp32.
 *   Limit: a query's selection (plus the one pool sparse_mla_attn_shared may add) is split over at most 64
 *     blocks of at most min(8320 / P, 2064) pools, so topk + 1 <= 64 * min(8320 / P, 2064) (132096 pools at P = 4),
 *     else KP_ERR_UNSUPPORTED.  Only the first min(n_sel, topk) entries of a row are read.
 *   Errors: KP_ERR_INVALID_ARG, KP_ERR_UNSUPPORTED (V, H, dtype, topk), KP_ERR_WORKSPACE.
 */
size_t sparse_mla_workspace_size(const kp_dims* dims, const kp_queries* queries);
kp_status sparse_mla_attn(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries, const void* q,
                          const int32_t* sel, const int32_t* n_sel, void* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * sparse_mla_attn_shared -- sparse_mla_attn with selections shared between queries (MTP drafts).
 *   [MAX glm5_next API page, index_share_for_mtp_iteration: the MTP draft layer reuses the target's top-k
 *   selection; GLM-5.3-Flash model card, "Raw config fields": index_share_for_mtp_iteration true]; [MAX glm5_next
 *   API page, index_kpool_always_select_tail: the incomplete trailing pool is always visible].  Query i (at
 *   position pos[i]) attends
 *     - the tokens of the pools in selection row sel_row[i] of sel / n_sel (rows as written by dsa_topk_select
 *       for the target queries), each pool cut at pos[i]; and
 *     - its own incomplete trailing pool tau = pos[i] / P (tokens P*tau .. pos[i]) when (pos[i] + 1) mod P != 0
 *       and the row does not hold tau.  The shared item is the target's top-k pick; the forced tail is not a
 *       pick, so a draft always sees its own pending tokens, itself included (it may attend topk + 1 pools).
 *   A row's own query reads the same set as sparse_mla_attn (its row already holds its incomplete tail), so with
 *   sel_row[i] = i this is sparse_mla_attn.  sel_row: device int32 [n_q], each in [0, rows of sel).  Workspace,
 *   outputs, limits and errors as in sparse_mla_attn; KP_ERR_INVALID_ARG on a NULL sel_row (n_q > 0).
 */
kp_status sparse_mla_attn_shared(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                                 const void* q, const int32_t* sel, const int32_t* n_sel, const int32_t* sel_row,
                                 void* out, float* lse, void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_mla_attn_mtp -- MTP verification: a target and its draft over one gather of their shared selection.
 *   [MAX glm5_next API page, index_share_for_mtp_iteration: the draft reuses its target's top-k selection;
 *   index_kpool_always_select_tail]; [metrale glm5_next_load/loader.rs page: each sparse-attention layer's
 *   workspace is sized for verify_k rows, the tokens one verification step carries].  Queries come in runs of two
 *   consecutive entries -- query 2r
 *   (a target) and query 2r + 1 (its draft; absent for the last run when n_q is odd) -- and both attend
 *   selection row r of sel / n_sel (one row per run: ceil(n_q / 2) rows, as dsa_topk_select writes for the
 *   targets).  Each query attends exactly what sparse_mla_attn_shared with sel_row[i] = i / 2 gives it: the row's
 *   pools cut at its own position plus its own incomplete trailing pool when the row lacks it.
 *   The difference is the gather: when the two queries of a run are of one sequence (the verification layout),
 *   one block computes 32 heads of both queries over a single gathered copy of their rows, and the blocks of the
 *   two head halves run side by side on one XCD, so each latent row is read from HBM about once per run instead
 *   of once per query.  Runs of two sequences are still exact (each query's rows are listed separately).
 *   Results equal sparse_mla_attn_shared's within rounding (the split of the work differs).
 *   q, out, lse: [n_q, ...] as in sparse_mla_attn.  workspace: device, at least sparse_mla_mtp_workspace_size
 *   bytes (split-KV partials; NULL when that is 0).
 *   Limit: bf16 with v_dim 512 and heads <= 64 (else KP_ERR_UNSUPPORTED); 2 (topk + 1) <= 32 * min(8320 / P,
 *   2064).  Other errors as in sparse_mla_attn.
 */
size_t sparse_mla_mtp_workspace_size(const kp_dims* dims, const kp_queries* queries);
kp_status sparse_mla_attn_mtp(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries, const void* q,
                              const int32_t* sel, const int32_t* n_sel, void* out, float* lse, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * sparse_mla_attn_noalloc -- sparse_mla_attn with no workspace argument and no allocation.
 *   For callers that cannot allocate device memory or pass a workspace: code under HIP graph capture, tight
 *   serving loops, harnesses that forbid allocation.  Same formula, kernels, split count and results as
 *   sparse_mla_attn (bit for bit); the split-KV partials go to a static device array of KP_NOALLOC_SCRATCH_BYTES
 *   that the library holds on each GPU it runs on until the process ends (its address is looked up on the first
 *   call on each device).  The call allocates nothing.
 *   Every call on a GPU shares that GPU's array and it keeps the last call's contents (nothing in it needs to start
 *   at zero): calls that overlap on one GPU (different streams, or threads) race and must be ordered by the caller.
 *   Limit: sparse_mla_workspace_size(dims, queries) <= KP_NOALLOC_SCRATCH_BYTES (every query count at the model's
 *   dims, H = 64, V = 512, topk = 2048 in bf16, needs at most 33.7 MB), else KP_ERR_WORKSPACE and nothing runs.
 *   Errors: as sparse_mla_attn; KP_ERR_LAUNCH also when the array's address cannot be looked up.
 */
#define KP_NOALLOC_SCRATCH_BYTES (36u << 20)
kp_status sparse_mla_attn_noalloc(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries,
                                  const void* q, const int32_t* sel, const int32_t* n_sel, void* out, float* lse,
                                  void* stream);

/*
 * sparse_mla_attn_fp8 -- sparse_mla_attn over an fp8 latent cache.
 *   [MAX glm5_next API page, declared_state_dtype(): the KV cache format may put the MLA latent in fp8;
 *   DEFAULT_ENCODING: float8_e4m3fn]; [metrale glm5_next_load/loader.rs page: each sparse-attention layer carries
 *   a kv_scale].  cache->latent holds OCP E4M3 ("e4m3fn") codes, latent_dim bytes per token; the latent row of a
 *   token is the decoded codes times kv_scale (a host scalar, finite and > 0).  Everything else -- the formula,
 *   q (bf16), sel / n_sel, out (bf16), lse, workspace (sparse_mla_workspace_size), limits -- is as in
 *   sparse_mla_attn.  Built for dims->dtype bf16 with v_dim 512 only.
 *   Errors: KP_ERR_INVALID_ARG (kv_scale, buffers), KP_ERR_UNSUPPORTED (shape), KP_ERR_WORKSPACE.
 */
kp_status sparse_mla_attn_fp8(const kp_dims* dims, const kp_cache* cache, const kp_queries* queries, const void* q,
                              const int32_t* sel, const int32_t* n_sel, float kv_scale, void* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * kp_linear -- the dense projections beside the sparse path, as one strided-batched bf16 product
 *     C[b][m][n] = alpha * sum_k A[b][m][k] * W[b][n][k]     (0 <= b < batch, m < M, n < N, k < K)
 *   [llama.cpp PR, "What I implemented new": the indexer cache holds key | gate per token; the indexer and the
 *   MLA low-rank paths are kept unquantized]; [MAX glm5_next API page, compute_dtype: the indexer and kv_b_proj
 *   run in the compute dtype]; [GLM-5.3-Flash model card, "Raw config fields": hidden_size 4096, q_lora_rank
 *   1536, qk_nope_head_dim 256, v_head_dim 256].  Absorbed MLA (the layer's specification): head h's key and
 *   value of a latent row c are W_UK[h] c and W_UV[h] c, so the query enters latent space as W_UK[h]^T q and the
 *   latent output leaves it as W_UV[h] o.
 *   A: device bf16, row m of batch b at A + b*stride_a + m*lda (elements), k contiguous.
 *   W: device bf16, row n of batch b at W + b*stride_w + n*ldw, k contiguous (a weight stored output-major).
 *   C: device, c_dtype (KP_DTYPE_BF16: rounded once, nearest-even; KP_DTYPE_F32), row m at C + b*stride_c +
 *     m*ldc, n contiguous.  A stride of 0 reuses one matrix for every batch entry.
 *   Accumulation is fp32; the result is a deterministic function of the operands and the call shape.
 *   workspace (device, may be NULL, no initial contents): with at least kp_linear_workspace_size(batch, M, N, K)
 *     bytes, a shape whose few output tiles would each stream a long K (a decode step) splits K over several
 *     blocks that store fp32 partial tiles there; a second kernel on the same stream adds them in split order.  Calls that share a workspace must not overlap (same stream, or ordered).  NULL or smaller: no
 *     split, same formula (the sum may round differently).  A size of 0 means this shape never splits.
 *   The layer's projections (T tokens, hidden 4096, q_lora 1536, Hi = 32, D = 128, H = 64, dn = dv = 256):
 *     index query   A = cq [T, 1536], W = W_iq [Hi*D, 1536] (head-major rows)  -> C = q_idx [T, Hi*D] bf16
 *     head weights  A = x [T, 4096],  W = W_w [Hi, 4096]                       -> C = w [T, Hi] f32
 *     key, gate     A = x [T, 4096],  W = rows 0..D-1 / D..2D-1 of W_kg [2D, 4096] -> C = keys / gates [T, D]
 *     absorb        batch H: A = q_nope + h*dn (lda H*dn), W = W_UK[h]^T [V, dn] (stride V*dn)
 *                   -> C = q + h*L (ldc H*L): columns 0..V-1 of each query row; the rotary columns V..L-1 are
 *                   not written (keep them zero)
 *     un-absorb     batch H: A = out + h*V (lda H*V), W = W_UV[h] [dv, V] (stride dv*V) -> C = o + h*dv
 *   The absorb and un-absorb shapes, (N, K) = (512, 256) or (256, 512), with batch >= 8, M >= 512 and rows
 *     16-byte aligned (ldc, stride_c times the element size multiples of 16), run weight-stationary: one launch,
 *     each batch entry's weight held on chip while its rows stream past; no workspace, same formula.
 *   Limits: K a multiple of 64; lda, ldw, stride_a, stride_w multiples of 8; ldc, stride_c multiples of 4;
 *   lda, ldw >= K; ldc >= N; every operand 16-byte aligned.  batch, M or N = 0 is a valid empty call.
 *   Errors: KP_ERR_INVALID_ARG (pointers, strides, alignment, c_dtype, alpha not finite), KP_ERR_UNSUPPORTED (K).
 *   kp_linear_workspace_size: bytes of split-K workspace for a shape (0: never splits); host only.
 */
size_t kp_linear_workspace_size(int32_t batch, int32_t M, int32_t N, int32_t K);
kp_status kp_linear(int32_t batch, int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int64_t stride_a,
                    const void* W, int64_t ldw, int64_t stride_w, void* C, int64_t ldc, int64_t stride_c,
                    int32_t c_dtype, float alpha, void* workspace, size_t ws_bytes, void* stream);

/* One product of a kp_linear_group call: the arguments of kp_linear (host struct, read during the call only). */
typedef struct {
  int32_t batch, M, N, K;
  const void* A;
  int64_t lda, stride_a;
  const void* W;
  int64_t ldw, stride_w;
  void* C;
  int64_t ldc, stride_c;
  int32_t c_dtype;
  float alpha;
} kp_linear_problem;

/*
 * kp_linear_group -- up to 8 independent kp_linear products in one launch (plus one launch that adds split-K
 *   partials, when any product splits, and one launch of its own for each product that runs weight-stationary
 *   under kp_linear's rule, issued after them): the products of one layer step that do not depend on each other (the
 *   indexer's projections and the query absorb of a decode step) pay the launch cost once.  Each product follows
 *   kp_linear's formula and contract.  Its tile shape (chosen by the group's largest M) and its K split (chosen
 *   from the whole group's work) can differ from a kp_linear call of its own, and so can the rounding of its sums;
 *   for a given group the result is deterministic.
 *   problems: host array of n (0..8) products; their outputs must not overlap each other's inputs or outputs.
 *   workspace: as in kp_linear, at least kp_linear_group_workspace_size(n, problems) bytes for full splitting
 *   (products are given workspace in order; from the first that no longer fits on, they run unsplit).
 *   Errors: as kp_linear, per product; KP_ERR_INVALID_ARG for n outside 0..8 or a NULL list.
 */
size_t kp_linear_group_workspace_size(int32_t n, const kp_linear_problem* problems);
kp_status kp_linear_group(int32_t n, const kp_linear_problem* problems, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * kp_read_rows -- measurement reference: reads rows and discards them.
 *   Reads rows[i] (0 <= i < n_rows) of `base`, each row_bytes long at byte offset rows[i] * row_stride, the way the
 *   attention stage gathers its value rows (whole 1 KiB units straight into LDS, in list order, in contiguous runs
 *   per wave), and keeps nothing: no compute, no barrier, no output.  Timed over the attention's own row list (the
 *   attended tokens' physical latent rows), it gives the read bandwidth HBM delivers for that gather pattern -- the
 *   practical ceiling the attention kernel is measured against.  Not part of the layer.
 *   base: device, 16-byte aligned; rows: device int32 [n_rows], each row inside the caller's buffer (not checked).
 *   row_bytes: 1024 (a value row) or 4096 (a 64-token page of pooled keys); row_stride >= row_bytes, a multiple of
 *   16; blocks_per_cu 1..8.
 *   Errors: KP_ERR_INVALID_ARG, KP_ERR_LAUNCH.
 */
kp_status kp_read_rows(const void* base, int64_t row_stride, int32_t row_bytes, const int32_t* rows, int64_t n_rows,
                       int32_t blocks_per_cu, void* stream);

/* Message of the last failed call on this thread ("" if none).  Owned by the library. */
const char* kp_last_error(void);

/* ABI version of this header (bumped on any signature or struct change). */
int32_t kp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KPOOL_H */
