"""The C-ABI library: it loads, exports every function include/kpool.h declares, and its host-side validation
returns the documented status codes.  Every call here fails validation before any HIP call, so no GPU is
needed."""
import ctypes
import os
import re

import pytest

import sparse_attention_kpool_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kpool.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", src, flags=re.M)))


def test_header_declares_the_four_calls():
    names = _declared()
    for f in ("kpool_compress", "dsa_indexer_score", "dsa_compress_score", "dsa_topk_select", "sparse_mla_attn",
              "sparse_mla_attn_fp8",
              "sparse_mla_attn_shared", "sparse_mla_attn_noalloc", "sparse_mla_attn_mtp",
              "sparse_mla_mtp_workspace_size", "kp_read_rows", "kp_linear", "kp_linear_workspace_size", "kp_linear_group",
              "kp_linear_group_workspace_size",
              "dsa_topk_workspace_size", "sparse_mla_workspace_size", "kp_last_error", "kp_abi_version"):
        assert f in names
    assert set(names) == set(K.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = K.load()
    for f in _declared():
        assert hasattr(lib, f), f
    assert lib.kp_abi_version() == K.ABI_VERSION


def _dims(**kw):
    d = dict(pool=4, idx_dim=128, idx_heads=32, topk=2048, heads=64, latent_dim=576, v_dim=512, page_tokens=64,
             dtype=K.KP_DTYPE_BF16, scale=1 / 16)
    d.update(kw)
    return K._Dims(**d)


FAKE = 1 << 20          # an aligned, non-null address; validation must fail before anything dereferences it


def _cache():
    return K._Cache(FAKE, FAKE, FAKE, 16)


def _queries(n_q=4, max_pos=100, group=1):
    return K._Queries(n_q, FAKE, FAKE, max_pos, group)


def _score(d, c=None, q=None, ld=64, qidx=FAKE):
    lib = K.load()
    return lib.dsa_indexer_score(ctypes.byref(d), None if c is False else ctypes.byref(c or _cache()),
                                 ctypes.byref(q or _queries()), qidx, FAKE, FAKE, ld, None)


@pytest.mark.parametrize("kw,code", [
    (dict(pool=3), K.KP_ERR_INVALID_ARG),               # not a power of two
    (dict(pool=64), K.KP_ERR_INVALID_ARG),
    (dict(topk=0), K.KP_ERR_INVALID_ARG),
    (dict(v_dim=600), K.KP_ERR_INVALID_ARG),            # V > L
    (dict(page_tokens=2), K.KP_ERR_INVALID_ARG),        # not a multiple of the pool
    (dict(page_tokens=96), K.KP_ERR_INVALID_ARG),       # not a power of two
    (dict(dtype=7), K.KP_ERR_UNSUPPORTED),
    (dict(idx_dim=64), K.KP_ERR_UNSUPPORTED),           # D not built
    (dict(idx_heads=33), K.KP_ERR_UNSUPPORTED),
    (dict(dtype=K.KP_DTYPE_F32), K.KP_ERR_UNSUPPORTED), # f32 is built for D = 32 only
])
def test_score_rejects_bad_dims(kw, code):
    assert _score(_dims(**kw)) == code
    assert K.last_error().startswith("dsa_indexer_score")


def test_score_rejects_small_ld_and_nulls_and_misalignment():
    assert _score(_dims(), ld=10) == K.KP_ERR_INVALID_ARG            # 25 visible pools
    assert "ld_scores" in K.last_error()
    assert _score(_dims(), c=False) == K.KP_ERR_INVALID_ARG
    assert _score(_dims(), qidx=None) == K.KP_ERR_INVALID_ARG
    assert _score(_dims(), qidx=FAKE + 8) == K.KP_ERR_INVALID_ARG
    assert "misaligned" in K.last_error()
    assert _score(_dims(), q=K._Queries(4, None, FAKE, 100, 1)) == K.KP_ERR_INVALID_ARG


def test_compress_score_checks_both_calls_before_launching():
    """dsa_compress_score applies kpool_compress's and dsa_indexer_score's checks (each failure is one of theirs,
    found before anything is launched); with no pools and no queries it is a valid no-op."""
    lib = K.load()
    d, c, q = _dims(), _cache(), _queries()

    def call(d=d, n_pools=2, keys=FAKE, q=q, ld=64):
        return lib.dsa_compress_score(ctypes.byref(d), ctypes.byref(c), n_pools, keys, FAKE, None, FAKE, FAKE, FAKE,
                                      None if q is None else ctypes.byref(q), FAKE, FAKE, FAKE, ld, None)
    assert call(keys=None) == K.KP_ERR_INVALID_ARG and b"dsa_compress_score" in lib.kp_last_error()
    assert call(n_pools=-1) == K.KP_ERR_INVALID_ARG
    assert call(ld=16) == K.KP_ERR_INVALID_ARG and b"ld_scores" in lib.kp_last_error()
    assert call(d=_dims(idx_dim=64)) == K.KP_ERR_UNSUPPORTED
    assert call(q=None) == K.KP_ERR_INVALID_ARG
    assert call(n_pools=0, keys=None, q=_queries(0, 0), ld=4) == K.KP_OK


def test_empty_query_batches_are_valid_noops():
    assert _score(_dims(), q=K._Queries(0, None, None, 0, 1), ld=0) == K.KP_OK
    lib = K.load()
    assert lib.kpool_compress(ctypes.byref(_dims()), ctypes.byref(_cache()), 0, None, None, None, None, None,
                              None, None) == K.KP_OK


def test_topk_and_attn_validation():
    lib = K.load()
    d, q = _dims(), _queries()
    assert lib.dsa_topk_select(ctypes.byref(d), ctypes.byref(q), FAKE, 10, FAKE, FAKE, None, 0, None) \
        == K.KP_ERR_INVALID_ARG
    assert lib.dsa_topk_select(ctypes.byref(d), ctypes.byref(q), None, 64, FAKE, FAKE, None, 0, None) \
        == K.KP_ERR_INVALID_ARG
    need = lib.sparse_mla_workspace_size(ctypes.byref(d), ctypes.byref(q))
    assert need > 0      # 4 queries split their selections across blocks
    st = lib.sparse_mla_attn(ctypes.byref(d), ctypes.byref(_cache()), ctypes.byref(q), FAKE, FAKE, FAKE, FAKE,
                             None, FAKE, need - 16, None)
    assert st == K.KP_ERR_WORKSPACE and "workspace" in K.last_error()
    st = lib.sparse_mla_attn(ctypes.byref(_dims(v_dim=128)), ctypes.byref(_cache()), ctypes.byref(q), FAKE, FAKE,
                             FAKE, FAKE, None, FAKE, need, None)
    assert st == K.KP_ERR_UNSUPPORTED
    st = lib.sparse_mla_attn(ctypes.byref(_dims(heads=65)), ctypes.byref(_cache()), ctypes.byref(q), FAKE, FAKE,
                             FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == K.KP_ERR_UNSUPPORTED
    st = lib.sparse_mla_attn(ctypes.byref(_dims(latent_dim=577)), ctypes.byref(_cache()), ctypes.byref(q), FAKE,
                             FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == K.KP_ERR_INVALID_ARG


def test_noalloc_limits():
    """sparse_mla_attn_noalloc: every query count at the model's dims fits its static scratch; a call that needs more
    (a huge top-k forces many splits) is rejected with KP_ERR_WORKSPACE before anything runs, and argument
    errors come back as they do from sparse_mla_attn."""
    lib = K.load()
    d = _dims()
    worst = max(lib.sparse_mla_workspace_size(ctypes.byref(d), ctypes.byref(_queries(n_q=n))) for n in range(1, 600))
    assert 0 < worst <= K.NOALLOC_SCRATCH_BYTES and worst == 510 * 64 * (512 * 2 + 8)
    st = lib.sparse_mla_attn_noalloc(ctypes.byref(_dims(topk=65536)), ctypes.byref(_cache()),
                                     ctypes.byref(_queries(n_q=64)), FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == K.KP_ERR_WORKSPACE and "scratch" in K.last_error()
    st = lib.sparse_mla_attn_noalloc(ctypes.byref(_dims(pool=3)), ctypes.byref(_cache()), ctypes.byref(_queries()),
                                     FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == K.KP_ERR_INVALID_ARG
    st = lib.sparse_mla_attn_noalloc(ctypes.byref(_dims(v_dim=128)), ctypes.byref(_cache()),
                                     ctypes.byref(_queries(n_q=4096)), FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == K.KP_ERR_UNSUPPORTED
    st = lib.sparse_mla_attn_noalloc(ctypes.byref(d), ctypes.byref(_cache()), ctypes.byref(_queries(n_q=4096)),
                                     FAKE, None, FAKE, FAKE, None, None)
    assert st == K.KP_ERR_INVALID_ARG


def test_mtp_validation_and_workspace():
    """sparse_mla_attn_mtp: built for bf16 with v_dim 512; its workspace follows its own split rule (about 256 blocks
    over the runs' head halves, and at least two splits for a run that lists two queries' pools)."""
    lib = K.load()
    d = _dims()
    ws = lambda n, dd=d: lib.sparse_mla_mtp_workspace_size(ctypes.byref(dd), ctypes.byref(_queries(n_q=n)))
    per = 64 * (512 * 2 + 8)              # one query's partial per split: H x (V bf16 + (m, l) fp32)
    assert ws(64) == 64 * 4 * per         # 32 runs x 2 head halves = 64 units: 4 splits
    assert ws(8) == 8 * 32 * per          # 4 runs: 32 splits (the cap)
    assert ws(4096) == 4096 * 2 * per     # many runs: still 2 splits, the two-sequence list needs them
    assert ws(7) == 7 * 32 * per          # an odd count: 4 runs, the last a target alone
    q = _queries(n_q=64)
    st = lib.sparse_mla_attn_mtp(ctypes.byref(d), ctypes.byref(_cache()), ctypes.byref(q), FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, ws(64) - 16, None)
    assert st == K.KP_ERR_WORKSPACE and "sparse_mla_attn_mtp" in K.last_error()
    for bad in (_dims(v_dim=64), _dims(dtype=K.KP_DTYPE_F32, v_dim=64)):
        st = lib.sparse_mla_attn_mtp(ctypes.byref(bad), ctypes.byref(_cache()), ctypes.byref(q), FAKE, FAKE, FAKE,
                                     FAKE, None, FAKE, 1 << 40, None)
        assert st == K.KP_ERR_UNSUPPORTED
    st = lib.sparse_mla_attn_mtp(ctypes.byref(d), ctypes.byref(_cache()), ctypes.byref(q), FAKE, None, FAKE, FAKE,
                                 None, FAKE, 1 << 40, None)
    assert st == K.KP_ERR_INVALID_ARG
    assert lib.sparse_mla_attn_mtp(ctypes.byref(d), ctypes.byref(_cache()), ctypes.byref(_queries(n_q=0)), None,
                                   None, None, None, None, None, 0, None) == K.KP_OK


def test_workspace_sizes_follow_the_split_rule():
    lib = K.load()
    d = _dims()
    big = lib.sparse_mla_workspace_size(ctypes.byref(d), ctypes.byref(_queries(n_q=4096)))
    assert big == 0                      # enough queries to fill the chip: no split, no workspace
    assert lib.dsa_topk_workspace_size(ctypes.byref(d), ctypes.byref(_queries())) >= 0


def test_binding_raises_without_library(tmp_path, monkeypatch):
    import importlib
    monkeypatch.setattr(K, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU or PyTorch fallback"):
        K.load(str(tmp_path / "missing.so"))
    monkeypatch.undo()
    importlib.reload(K)  # a fresh module: the next load() binds the library to this module's ctypes classes


def _linear(batch=1, M=64, N=64, k=128, A=FAKE, lda=128, sa=0, W=FAKE, ldw=128, sw=0, C=FAKE, ldc=64, sc=0,
            c_dtype=K.KP_DTYPE_BF16, alpha=1.0, ws=None, ws_bytes=0):
    return K.load().kp_linear(batch, M, N, k, A, lda, sa, W, ldw, sw, C, ldc, sc, c_dtype, alpha, ws, ws_bytes, None)


def test_linear_validation():
    """kp_linear rejects every bad argument before launching anything (no GPU is touched here)."""
    ok_empty = [dict(batch=0), dict(M=0), dict(N=0), dict(M=0, A=None)]
    for kw in ok_empty:
        assert _linear(**kw) == K.KP_OK, kw
    bad = [
        (dict(batch=-1), K.KP_ERR_INVALID_ARG),
        (dict(k=96, lda=96, ldw=96), K.KP_ERR_UNSUPPORTED),     # not a multiple of 64
        (dict(k=0), K.KP_ERR_UNSUPPORTED),
        (dict(c_dtype=7), K.KP_ERR_INVALID_ARG),
        (dict(A=None), K.KP_ERR_INVALID_ARG),
        (dict(W=FAKE + 8), K.KP_ERR_INVALID_ARG),               # misaligned
        (dict(lda=64), K.KP_ERR_INVALID_ARG),                   # below K
        (dict(ldc=60), K.KP_ERR_INVALID_ARG),                   # below N
        (dict(lda=132), K.KP_ERR_INVALID_ARG),                  # not a multiple of 8
        (dict(sw=4), K.KP_ERR_INVALID_ARG),
        (dict(ldc=66), K.KP_ERR_INVALID_ARG),                   # not a multiple of 4
        (dict(sc=-4), K.KP_ERR_INVALID_ARG),
        (dict(alpha=float("inf")), K.KP_ERR_INVALID_ARG),
        (dict(ws=FAKE + 4, ws_bytes=1 << 20), K.KP_ERR_INVALID_ARG),  # misaligned workspace
    ]
    for kw, code in bad:
        assert _linear(**kw) == code, kw
        assert "kp_linear" in K.last_error()


def test_linear_workspace_sizes():
    """Decode-shaped products (few output tiles) ask for split-K workspace; shapes with enough tiles, or too short a
    K, need none."""
    ws = K.linear_workspace_size
    assert ws(1, 64, 4096, 1536) > 0          # index query at a 64-token step: 64 tiles
    assert ws(1, 64, 32, 4096) > 0            # head weights: one tile, long K
    assert ws(1, 4096, 4096, 1536) == 0       # prefill: 1024 tiles
    assert ws(64, 64, 512, 256) == 0          # absorb at a decode step: 512 tiles, 4 stages
    assert ws(1, 64, 64, 64) == 0             # one stage: nothing to split
    assert ws(0, 64, 64, 4096) == 0 and ws(1, 0, 64, 4096) == 0
    # fp32 partial tiles: 64 x 64 per split of each tile
    n = ws(1, 64, 32, 4096)
    assert n > 0 and n % (64 * 64 * 4) == 0


def test_linear_prefill_split_rule_and_weight_stationary_products():
    """At prefill sizes a product of 128 x 128 tiles splits K once its blocks would run more stages than the group's
    average per block slot (the head-weight product beside the index query: 64 stages against an average of 52),
    and the absorb / un-absorb shapes run weight-stationary: they take no workspace and do not count towards the
    other products' split (a group with the absorb asks for exactly what the group without it asks for)."""
    lib = K.load()
    T = 4096

    def prob(batch, M, N, K_, lda, sa, ldw, sw, ldc, sc, dt=K.KP_DTYPE_BF16):
        return K._LinearProblem(batch, M, N, K_, FAKE, lda, sa, FAKE, ldw, sw, FAKE, ldc, sc, dt, 1.0)
    index_query = prob(1, T, 4096, 1536, 1536, 0, 1536, 0, 4096, 0)
    head_weights = prob(1, T, 32, 4096, 4096, 0, 4096, 0, 32, 0, K.KP_DTYPE_F32)
    absorb = prob(64, T, 512, 256, 64 * 256, 256, 256, 512 * 256, 64 * 576, 576)
    unabsorb = prob(64, T, 256, 512, 64 * 512, 512, 512, 256 * 512, 64 * 256, 256)
    two = (K._LinearProblem * 2)(index_query, head_weights)
    three = (K._LinearProblem * 3)(index_query, head_weights, absorb)
    assert lib.kp_linear_group_workspace_size(2, two) > 0
    assert lib.kp_linear_group_workspace_size(3, three) == lib.kp_linear_group_workspace_size(2, two)
    assert K.linear_workspace_size(64, T, 512, 256) == 0 and K.linear_workspace_size(64, T, 256, 512) == 0
    assert lib.kp_linear_group_workspace_size(1, (K._LinearProblem * 1)(unabsorb)) == 0


def test_linear_group_validation():
    """kp_linear_group checks the product count, the list and every product before launching anything."""
    lib = K.load()
    good = K._LinearProblem(1, 64, 64, 128, FAKE, 128, 0, FAKE, 128, 0, FAKE, 64, 0, K.KP_DTYPE_BF16, 1.0)
    bad_k = K._LinearProblem(1, 64, 64, 96, FAKE, 128, 0, FAKE, 128, 0, FAKE, 64, 0, K.KP_DTYPE_BF16, 1.0)
    empty = K._LinearProblem(0, 64, 64, 96, None, 0, 0, None, 0, 0, None, 0, 0, 9, 1.0)  # never read
    arr = (K._LinearProblem * 9)(*([good] * 9))
    assert lib.kp_linear_group(0, arr, None, 0, None) == K.KP_OK
    assert lib.kp_linear_group(9, arr, None, 0, None) == K.KP_ERR_INVALID_ARG
    assert lib.kp_linear_group(-1, arr, None, 0, None) == K.KP_ERR_INVALID_ARG
    assert lib.kp_linear_group(2, None, None, 0, None) == K.KP_ERR_INVALID_ARG
    two = (K._LinearProblem * 2)(empty, bad_k)
    assert lib.kp_linear_group(2, two, None, 0, None) == K.KP_ERR_UNSUPPORTED
    assert "kp_linear_group" in K.last_error()
    one_empty = (K._LinearProblem * 1)(empty)
    assert lib.kp_linear_group(1, one_empty, None, 0, None) == K.KP_OK
    # the group's workspace is the sum of its products' (same tile shape here)
    pair = (K._LinearProblem * 2)(
        K._LinearProblem(1, 64, 32, 4096, FAKE, 4096, 0, FAKE, 4096, 0, FAKE, 32, 0, K.KP_DTYPE_F32, 1.0),
        K._LinearProblem(1, 64, 4096, 1536, FAKE, 1536, 0, FAKE, 1536, 0, FAKE, 4096, 0, K.KP_DTYPE_BF16, 1.0))
    assert lib.kp_linear_group_workspace_size(2, pair) == \
        K.linear_workspace_size(1, 64, 32, 4096) + K.linear_workspace_size(1, 64, 4096, 1536)
