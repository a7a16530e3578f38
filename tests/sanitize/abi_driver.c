/*
 * Host-only exercise of the KPool-DSA C ABI (include/kpool.h) for a build of the library whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Every call below either fails validation (so no HIP call is
 * made and no device pointer is dereferenced) or is a pure host size query; the driver checks the documented
 * status codes and that kp_last_error() explains each failure.  Exit status 0 = every check held.
 */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "kpool.h"

static int failures = 0;
#define CHECK(cond, what)                                              \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "FAILED: %s (%s:%d)\n", what, __FILE__, __LINE__); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void* const FAKE = (void*)(uintptr_t)(1u << 20); /* aligned, non-null, never dereferenced */

static kp_dims dims(void) {
  kp_dims d = {4, 128, 32, 2048, 64, 576, 512, 64, KP_DTYPE_BF16, 1.0f / 16.0f};
  return d;
}
static kp_cache cache(void) {
  kp_cache c = {FAKE, FAKE, (const int32_t*)FAKE, 16};
  return c;
}
static kp_queries queries(int32_t n_q, int32_t max_pos) {
  kp_queries q = {n_q, (const int32_t*)FAKE, (const int32_t*)FAKE, max_pos, 1};
  return q;
}
static void explained(const char* what) {
  const char* e = kp_last_error();
  CHECK(e && strlen(e) > 0 && strlen(e) < 512, what);
}

int main(void) {
  CHECK(kp_abi_version() == 7, "abi version");
  kp_dims d = dims();
  kp_cache c = cache();
  kp_queries q = queries(4, 100);

  /* kpool_compress */
  CHECK(kpool_compress(NULL, &c, 1, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, NULL) == KP_ERR_INVALID_ARG, "compress dims");
  explained("compress dims message");
  { kp_dims b = d; b.pool = 3;
    CHECK(kpool_compress(&b, &c, 1, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, NULL) == KP_ERR_INVALID_ARG, "pool 3"); }
  CHECK(kpool_compress(&d, &c, -1, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, NULL) == KP_ERR_INVALID_ARG, "n_pools < 0");
  CHECK(kpool_compress(&d, &c, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == KP_OK, "empty compress");
  CHECK(kpool_compress(&d, &c, 2, NULL, FAKE, NULL, FAKE, FAKE, FAKE, NULL) == KP_ERR_INVALID_ARG, "null keys");
  CHECK(kpool_compress(&d, &c, 2, (char*)FAKE + 4, FAKE, NULL, FAKE, FAKE, FAKE, NULL) == KP_ERR_INVALID_ARG,
        "misaligned keys");
  { kp_cache b = c; b.block_table = NULL;
    CHECK(kpool_compress(&d, &b, 2, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, NULL) == KP_ERR_INVALID_ARG, "null bt"); }

  /* dsa_indexer_score */
  CHECK(dsa_indexer_score(&d, &c, &q, FAKE, FAKE, FAKE, 16, NULL) == KP_ERR_INVALID_ARG, "ld too small");
  explained("ld message");
  CHECK(dsa_indexer_score(&d, &c, &q, FAKE, FAKE, FAKE, 30, NULL) == KP_ERR_INVALID_ARG, "ld not multiple of 4");
  { kp_dims b = d; b.idx_dim = 64;
    CHECK(dsa_indexer_score(&b, &c, &q, FAKE, FAKE, FAKE, 64, NULL) == KP_ERR_UNSUPPORTED, "idx_dim 64"); }
  { kp_dims b = d; b.idx_heads = 33;
    CHECK(dsa_indexer_score(&b, &c, &q, FAKE, FAKE, FAKE, 64, NULL) == KP_ERR_UNSUPPORTED, "33 heads"); }
  { kp_queries e = queries(0, 0);
    CHECK(dsa_indexer_score(&d, &c, &e, NULL, NULL, NULL, 4, NULL) == KP_OK, "empty score"); }
  { kp_queries b = queries(4, 100); b.seq = NULL;
    CHECK(dsa_indexer_score(&d, &c, &b, FAKE, FAKE, FAKE, 64, NULL) == KP_ERR_INVALID_ARG, "null seq"); }
  CHECK(dsa_indexer_score(&d, &c, NULL, FAKE, FAKE, FAKE, 64, NULL) == KP_ERR_INVALID_ARG, "null queries");

  /* dsa_compress_score: both calls' checks, before anything is launched */
  CHECK(dsa_compress_score(&d, &c, 2, NULL, FAKE, NULL, FAKE, FAKE, FAKE, &q, FAKE, FAKE, FAKE, 64, NULL) ==
            KP_ERR_INVALID_ARG, "fused: null keys");
  explained("fused: null keys message");
  CHECK(dsa_compress_score(&d, &c, -1, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, &q, FAKE, FAKE, FAKE, 64, NULL) ==
            KP_ERR_INVALID_ARG, "fused: n_pools < 0");
  CHECK(dsa_compress_score(&d, &c, 2, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, &q, FAKE, FAKE, FAKE, 16, NULL) ==
            KP_ERR_INVALID_ARG, "fused: ld too small");
  { kp_dims b = d; b.idx_dim = 64;
    CHECK(dsa_compress_score(&b, &c, 2, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, &q, FAKE, FAKE, FAKE, 64, NULL) ==
              KP_ERR_UNSUPPORTED, "fused: idx_dim 64"); }
  CHECK(dsa_compress_score(&d, &c, 2, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, 64, NULL) ==
            KP_ERR_INVALID_ARG, "fused: null queries");
  { kp_queries e = queries(0, 0);
    CHECK(dsa_compress_score(&d, &c, 0, NULL, NULL, NULL, NULL, NULL, NULL, &e, NULL, NULL, NULL, 4, NULL) == KP_OK,
          "fused: empty"); }

  /* dsa_topk_select */
  {
    kp_queries big = queries(64, 131071);
    size_t ws = dsa_topk_workspace_size(&d, &big);
    CHECK(dsa_topk_workspace_size(NULL, &big) == 0, "topk ws null dims");
    if (ws > 0)
      CHECK(dsa_topk_select(&d, &big, FAKE, 32768, FAKE, FAKE, FAKE, ws - 1, NULL) == KP_ERR_WORKSPACE,
            "topk workspace short");
    CHECK(dsa_topk_select(&d, &q, FAKE, 10, FAKE, FAKE, NULL, 0, NULL) == KP_ERR_INVALID_ARG, "topk ld");
    CHECK(dsa_topk_select(&d, &q, NULL, 64, FAKE, FAKE, NULL, 0, NULL) == KP_ERR_INVALID_ARG, "topk null scores");
    kp_queries huge = queries(8, (1 << 23) - 1);  /* 2M pools: beyond the two-step limit */
    CHECK(dsa_topk_select(&d, &huge, FAKE, 1 << 21, FAKE, FAKE, FAKE, (size_t)1 << 40, NULL) == KP_ERR_UNSUPPORTED,
          "topk beyond two-step limit");
    explained("topk limit message");
  }

  /* sparse_mla_attn and its variants */
  {
    size_t need = sparse_mla_workspace_size(&d, &q);
    CHECK(need > 0, "4 queries split");
    CHECK(sparse_mla_attn(&d, &c, &q, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, need - 16, NULL) == KP_ERR_WORKSPACE,
          "attn workspace short");
    { kp_dims b = d; b.v_dim = 128;
      CHECK(sparse_mla_attn(&b, &c, &q, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, need, NULL) == KP_ERR_UNSUPPORTED, "v 128"); }
    { kp_dims b = d; b.heads = 65;
      CHECK(sparse_mla_attn(&b, &c, &q, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, need, NULL) == KP_ERR_UNSUPPORTED, "65 heads"); }
    { kp_dims b = d; b.latent_dim = 577;
      CHECK(sparse_mla_attn(&b, &c, &q, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, need, NULL) == KP_ERR_INVALID_ARG, "L 577"); }
    CHECK(sparse_mla_attn_shared(&d, &c, &q, FAKE, FAKE, FAKE, NULL, FAKE, NULL, FAKE, need, NULL) == KP_ERR_INVALID_ARG,
          "shared null sel_row");
    CHECK(sparse_mla_attn_fp8(&d, &c, &q, FAKE, FAKE, FAKE, 0.0f, FAKE, NULL, FAKE, need, NULL) == KP_ERR_INVALID_ARG,
          "fp8 scale 0");
    { size_t mneed = sparse_mla_mtp_workspace_size(&d, &q);
      CHECK(mneed > 0, "mtp workspace size");
      CHECK(sparse_mla_attn_mtp(&d, &c, &q, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, mneed - 16, NULL) == KP_ERR_WORKSPACE,
            "mtp workspace short");
      explained("mtp workspace message");
      kp_dims b = d; b.v_dim = 64;
      CHECK(sparse_mla_attn_mtp(&b, &c, &q, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, mneed, NULL) == KP_ERR_UNSUPPORTED,
            "mtp v 64"); }
    { kp_dims b = d; b.topk = 65536; kp_queries q64 = queries(64, 100);
      CHECK(sparse_mla_attn_noalloc(&b, &c, &q64, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == KP_ERR_WORKSPACE,
            "noalloc beyond its scratch"); }
    { kp_queries q4096 = queries(4096, 100);
      CHECK(sparse_mla_attn_noalloc(&d, &c, &q4096, FAKE, NULL, FAKE, FAKE, NULL, NULL) == KP_ERR_INVALID_ARG,
            "noalloc null sel"); }
    size_t worst = 0;
    for (int n = 1; n < 600; ++n) {
      kp_queries qn = queries(n, 100);
      size_t w = sparse_mla_workspace_size(&d, &qn);
      if (w > worst) worst = w;
    }
    CHECK(worst > 0 && worst <= KP_NOALLOC_SCRATCH_BYTES, "every query count fits the no-alloc scratch");
  }

  /* kp_linear / kp_linear_group */
  CHECK(kp_linear(1, 4, 4, 60, FAKE, 64, 0, FAKE, 64, 0, FAKE, 4, 0, KP_DTYPE_F32, 1.f, NULL, 0, NULL) ==
            KP_ERR_UNSUPPORTED, "linear K 60");
  CHECK(kp_linear(1, 4, 4, 64, FAKE, 63, 0, FAKE, 64, 0, FAKE, 4, 0, KP_DTYPE_F32, 1.f, NULL, 0, NULL) ==
            KP_ERR_INVALID_ARG, "linear lda");
  CHECK(kp_linear(1, 4, 4, 64, FAKE, 64, 0, FAKE, 64, 0, FAKE, 4, 0, 7, 1.f, NULL, 0, NULL) == KP_ERR_INVALID_ARG,
        "linear c_dtype");
  CHECK(kp_linear(0, 4, 4, 64, NULL, 64, 0, NULL, 64, 0, NULL, 4, 0, KP_DTYPE_F32, 1.f, NULL, 0, NULL) == KP_OK,
        "linear empty");
  CHECK(kp_linear_workspace_size(1, 64, 128, 4096) > 0, "decode product splits K");
  CHECK(kp_linear_group(9, NULL, NULL, 0, NULL) == KP_ERR_INVALID_ARG, "group of 9");
  {
    kp_linear_problem p[2];
    memset(p, 0, sizeof(p));
    p[0].batch = 1; p[0].M = 4; p[0].N = 4; p[0].K = 64; p[0].A = FAKE; p[0].lda = 64; p[0].W = FAKE; p[0].ldw = 64;
    p[0].C = FAKE; p[0].ldc = 4; p[0].c_dtype = KP_DTYPE_F32; p[0].alpha = 1.f;
    p[1] = p[0];
    p[1].ldc = 3;
    CHECK(kp_linear_group(2, p, NULL, 0, NULL) == KP_ERR_INVALID_ARG, "group bad ldc");
    CHECK(kp_linear_group_workspace_size(2, p) == 0, "group ws of an invalid group");
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi driver: all checks passed\n");
  return 0;
}
