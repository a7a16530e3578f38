"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, stage by stage and end to end.

Each stage is compared on the inputs the previous GPU stage produced, so a mismatch names its stage:
  compress  pooled-cache rows written in-step  vs  oracle pooling of the same key/gate rows (bit-exact on the
            constant-key parity instance; <= 1 bf16 ulp / 1e-6 relative in fp32 otherwise)
  score     GPU score row  vs  oracle scores from the GPU's pooled cache (bit-exact on integer data)
  select    GPU selection  vs  oracle top-k of the GPU's own score row (always bit-exact)
  attend    GPU output     vs  oracle attention over the GPU's selection (bf16: max-abs 3e-2, rel-RMS 1e-2;
            fp32: max-abs 1e-4, rel-RMS 1e-5)
On the parity instance the oracle's own end-to-end selection must equal the GPU's as well.
Full-size workloads check sampled queries (every score of a sampled row, its selection and output).
"""
import sys

import numpy as np
import pytest
import torch

import kpool_synth as ks
import oracle as O
from harness import DeviceRun, attn_tolerance, oracle_pooled, oracle_query, rel_rms

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_run(run: DeviceRun, samples, n_compress_check=64, parity=True):
    wl = run.wl
    P = wl.P
    errs, refs, max_abs = [], [], 0.0
    # -------- compress: rows written this step
    if run.cpools:
        rng = np.random.default_rng(0)
        pick = run.cpools if len(run.cpools) <= n_compress_check else [
            run.cpools[t] for t in sorted(rng.choice(len(run.cpools), n_compress_check, replace=False))]
        for s, p in pick:
            got = run.pooled_rows(s, [p])[0]
            toks = np.arange(p * P, p * P + P)
            ref = O.store_round(O.pool_compress(ks.host_token_keys(wl, s, toks)[None],
                                                ks.host_gates(wl, s, toks)[None], ks.host_ape(wl)), wl.dtype)[0]
            if parity:
                np.testing.assert_array_equal(got, ref, err_msg=f"compress seq {s} pool {p}")
            elif wl.dtype == "bf16":
                ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
                assert (np.abs(got - ref) <= ulp).all(), f"compress seq {s} pool {p}"
            else:
                np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6, err_msg=f"compress seq {s} pool {p}")
    # -------- per sampled query
    for j in samples:
        s, i = int(wl.q_seq[j]), int(wl.q_pos[j])
        n_c, r, tau = O.pool_geometry(i, P)
        gpu_pooled = run.pooled_rows(s, np.arange(n_c)) if n_c else np.zeros((0, wl.D))
        if parity:
            np.testing.assert_array_equal(gpu_pooled, oracle_pooled(wl, s, n_c), err_msg=f"pooled cache q{j}")
        qidx, w = ks.host_qidx(wl, s, i)[0], ks.host_w(wl, s, i)[0]
        ref_scores = O.indexer_scores(qidx, w, gpu_pooled, n_c)
        got_scores = run.scores_row(j, n_c)
        if parity:
            np.testing.assert_array_equal(got_scores, ref_scores, err_msg=f"scores q{j} (seq {s}, pos {i})")
        else:
            bound = 1e-5 * (np.abs(w)[None, :] * np.abs(gpu_pooled @ np.abs(qidx).T)).sum(1) + 1e-30
            assert (np.abs(got_scores - ref_scores) <= bound).all(), f"scores q{j}"
        sel_row, ns = run.sel_row(j)
        ref_sel = O.select_pools(got_scores, i, P, wl.k)
        assert ns == len(ref_sel), f"n_sel q{j}: {ns} != {len(ref_sel)}"
        np.testing.assert_array_equal(sel_row[:ns], ref_sel, err_msg=f"selection q{j} (seq {s}, pos {i})")
        assert (sel_row[ns:] == -1).all(), f"padding q{j}"
        if parity:
            own = oracle_query(wl, j)
            np.testing.assert_array_equal(own["sel"], ref_sel, err_msg=f"end-to-end selection q{j}")
        ref = oracle_query(wl, j, pooled=gpu_pooled, sel=ref_sel)
        got = run.out[j].float().cpu().numpy().astype(np.float64)
        got_lse = run.lse[j].cpu().numpy().astype(np.float64)
        errs.append(got - ref["out"])
        refs.append(ref["out"])
        max_abs = max(max_abs, float(np.abs(got - ref["out"]).max()))
        np.testing.assert_allclose(got_lse, ref["lse"], rtol=1e-4, atol=1e-3, err_msg=f"lse q{j}")
    tol_abs, tol_rel = attn_tolerance(wl.dtype)
    rr = rel_rms(np.concatenate([e.ravel() for e in errs]) + np.concatenate([x.ravel() for x in refs]),
                 np.concatenate([x.ravel() for x in refs]))
    _say(f"  {wl.name}: {len(samples)} queries, attention max-abs {max_abs:.3g} (<= {tol_abs}), rel-RMS {rr:.3g} "
         f"(<= {tol_rel})")
    assert max_abs <= tol_abs, f"attention max-abs {max_abs}"
    assert rr <= tol_rel, f"attention rel-RMS {rr}"


# ----------------------------------------------------------------------------------------------------------
# small cases: every query checked
# ----------------------------------------------------------------------------------------------------------
def _small_decode(name="small_decode", ctx=(37, 1000, 4099, 8192, 20001), **kw):
    wl = ks.workloads()["batch64"]
    ctx = list(ctx)
    base = dict(name=name, ctx=ctx, new_from=[t - 1 for t in ctx], q_seq=np.arange(len(ctx), dtype=np.int32),
                q_pos=np.array([t - 1 for t in ctx], np.int32), page_perm_seed=7)
    base.update(kw)
    return ks.scaled(wl, **base)


SMALL = {
    "tiny": lambda: ks.workloads()["tiny"],
    "tiny_general": lambda: ks.scaled(ks.workloads()["tiny"], name="tiny_general", key_per_token=True),
    "tiny_dense_k": lambda: ks.scaled(ks.workloads()["tiny"], name="tiny_dense_k", k=64),
    "tiny_k1": lambda: ks.scaled(ks.workloads()["tiny"], name="tiny_k1", k=1),
    "small_decode": lambda: _small_decode(),
    "small_decode_pool16": lambda: _small_decode("small_decode_pool16", P=16, k=128),
    "small_decode_pool1": lambda: _small_decode("small_decode_pool1", ctx=(5, 300, 2500), P=1, k=512),
    "small_decode_contig": lambda: _small_decode("small_decode_contig", page_perm_seed=None, page_tokens=1 << 15),
    # fp8 (E4M3) latent cache with a scale: attention through sparse_mla_attn_fp8
    "small_decode_fp8": lambda: _small_decode("small_decode_fp8", latent_fp8=True, kv_scale=0.5),
    "two_step_fp8": lambda: _small_decode("two_step_fp8", ctx=(140001, 3001, 131076), latent_fp8=True,
                                          kv_scale=0.25),
    # pages of 2 pooled rows: a 4-row wave load of the decode scorer crosses pages (per-lane page lookup)
    "small_decode_page8": lambda: _small_decode("small_decode_page8", ctx=(37, 1000, 4099, 9001), page_tokens=8),
    # a small batch with k far below its rows: the rows are split over many top-k blocks (chunks of 256 pools)
    "small_decode_k64": lambda: _small_decode("small_decode_k64", ctx=(10001, 17, 9999, 4099), k=64),
    "small_bf16_narrow": lambda: ks.scaled(_small_decode("small_bf16_narrow", ctx=(3, 64, 777, 5000)), D=32, Hi=1,
                                           H=4, L=80, V=64, k=16),
    "small_prefill": lambda: ks.scaled(ks.workloads()["prefill64k"], name="small_prefill", ctx=[3000],
                                       new_from=[2500], q_seq=np.zeros(500, np.int32),
                                       q_pos=np.arange(2500, 3000, dtype=np.int32), k=256),
    # rows longer than one LDS-resident top-k block (32768 pools) next to a short row: the two-step selection
    "two_step_mixed": lambda: _small_decode("two_step_mixed", ctx=(140001, 3001, 131076)),
    # every score 0: selection is decided by the lower-index tie-break alone, at full top-k
    "all_ties": lambda: ks.scaled(_small_decode("all_ties", ctx=(20000, 9001, 70003)), w_scale=0.0),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_small_all_queries(case):
    wl = SMALL[case]()
    _say(f"[case {case}] B={wl.B} n_q={wl.n_q} dtype={wl.dtype} P={wl.P} k={wl.k}")
    run = DeviceRun(wl).run()
    check_run(run, range(wl.n_q), parity=not wl.key_per_token)
    del run
    _free()


def test_group_hint_violated_is_still_exact():
    """Queries of different sequences under a group hint that promises otherwise: results unchanged."""
    wl = _small_decode("mixed_groups", ctx=(100, 2000, 2001, 333, 4096, 70, 9000, 12))
    _say(f"[case mixed_groups] n_q={wl.n_q}")
    a = DeviceRun(wl, group=1).run()
    b = DeviceRun(wl, group=8).run()   # promises one sequence per 8 queries: the prefill shape
    for j in range(wl.n_q):
        n_c = (int(wl.q_pos[j]) + 1) // wl.P
        np.testing.assert_array_equal(a.scores_row(j, n_c), b.scores_row(j, n_c))
    assert torch.equal(a.layer.sel, b.layer.sel) and torch.equal(a.out, b.out)
    check_run(b, range(wl.n_q))
    del a, b
    _free()


def test_paged_equals_contiguous_and_deterministic():
    wl1 = _small_decode("paged", ctx=(5000, 17, 9999))
    wl2 = ks.scaled(wl1, name="contig", page_perm_seed=None, page_tokens=1 << 14)
    _say("[case paged_vs_contig]")
    a = DeviceRun(wl1).run()
    out1, sel1 = a.out.clone(), a.layer.sel.clone()
    a.run()
    assert torch.equal(out1, a.out) and torch.equal(sel1, a.layer.sel), "two runs differ"
    b = DeviceRun(wl2).run()
    assert torch.equal(sel1, b.layer.sel)
    assert torch.equal(out1, b.out)
    del a, b
    _free()


def test_workspace_reuse_across_query_counts():
    """One attention workspace serves calls with different query counts (so different split counts) in any
    order: results repeat bit for bit, and match a repeated batch within the attention tolerance."""
    import sparse_attention_kpool_amd as K
    wl = _small_decode("ws_reuse")
    _say("[case ws_reuse]")
    run = DeviceRun(wl).run()
    n5 = wl.n_q
    rep = 20
    idx = torch.arange(n5, device="cuda").repeat(rep)
    seq, pos = run.queries.seq[idx].contiguous(), run.queries.pos[idx].contiguous()
    q100 = K.Queries(seq=seq, pos=pos, max_pos=run.queries.max_pos, group=1)
    q5 = K.Queries(seq=run.queries.seq, pos=run.queries.pos, max_pos=run.queries.max_pos, group=1)
    sel5, nsel5 = run.layer.sel[:n5], run.layer.n_sel[:n5]
    sel100, nsel100 = sel5[idx].contiguous(), nsel5[idx].contiguous()
    qq100 = run.q[idx].contiguous()
    need = max(K.sparse_mla_workspace_size(run.dims, q5), K.sparse_mla_workspace_size(run.dims, q100))
    ws = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device="cuda")
    out100 = torch.empty((n5 * rep, wl.H, wl.V), dtype=run.out.dtype, device="cuda")
    out5 = torch.empty_like(run.out)

    def call(queries, q, sel, nsel, out):
        K.sparse_mla_attn(run.dims, run.cache, queries, q, sel, nsel, out, workspace=ws)
        torch.cuda.synchronize()
        return out.clone()

    a1 = call(q100, qq100, sel100, nsel100, out100)
    b1 = call(q5, run.q, sel5, nsel5, out5)
    a2 = call(q100, qq100, sel100, nsel100, out100)
    b2 = call(q5, run.q, sel5, nsel5, out5)
    assert torch.equal(a1, a2) and torch.equal(b1, b2), "repeated calls differ"
    assert torch.equal(b1, run.out), "the layer step with the same queries gave another result"
    ref = b1.float().repeat(rep, 1, 1)
    assert (a1.float() - ref).abs().max().item() <= attn_tolerance(wl.dtype)[0]
    del run
    _free()


def test_mtp_shared_selection():
    """MTP drafts reusing their targets' selections (sparse_mla_attn_shared): targets at T-2, drafts at T-1 of the
    same sequences.  A target reading its own row reproduces sparse_mla_attn bit for bit; a draft matches the oracle
    over the target's selected pools cut at the draft's own position (so with T-1 = 9000 the draft's new pool,
    which the target could not select, is not attended)."""
    import sparse_attention_kpool_amd as K
    ctx = [37, 1000, 4099, 9001]
    n = len(ctx)
    base = ks.workloads()["batch64"]
    wl = ks.scaled(base, name="mtp_shared", ctx=ctx, new_from=[t - 2 for t in ctx],
                   q_seq=np.array(list(range(n)) * 2, np.int32),
                   q_pos=np.array([t - 2 for t in ctx] + [t - 1 for t in ctx], np.int32), page_perm_seed=7)
    _say("[case mtp_shared] targets at T-2, drafts at T-1")
    run = DeviceRun(wl).run()
    check_run(run, list(range(2 * n)))
    n_q = wl.n_q
    sel_row = torch.tensor(list(range(n)) * 2, dtype=torch.int32, device="cuda")
    out = torch.empty_like(run.out)
    lse = torch.empty_like(run.lse)
    K.sparse_mla_attn_shared(run.dims, run.cache, run.queries, run.q, run.layer.sel[:n_q], run.layer.n_sel[:n_q],
                             sel_row, out, lse=lse, workspace=run.layer.ws_attn)
    torch.cuda.synchronize()
    assert torch.equal(out[:n], run.out[:n]) and torch.equal(lse[:n], run.lse[:n]), "target rows differ"
    tol_abs, tol_rel = attn_tolerance(wl.dtype)
    for d in range(n, 2 * n):
        t = d - n
        s, i = int(wl.q_seq[d]), int(wl.q_pos[d])
        sel_t, ns = run.sel_row(t)
        toks = O.attended_tokens(sel_t[:ns], i, wl.P)
        ref_out, ref_lse = O.sparse_mla(ks.host_q(wl, s, i)[0], ks.host_latent(wl, s, toks), wl.scale, wl.V)
        got = out[d].float().cpu().numpy()
        assert np.abs(got - ref_out).max() <= tol_abs, f"draft {d}: max-abs"
        assert rel_rms(got, ref_out) <= tol_rel, f"draft {d}: rel-RMS"
        np.testing.assert_allclose(lse[d].cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-3, err_msg=f"draft {d} lse")
        if i == 9000:
            assert 9000 not in set(toks.tolist()), "the draft's new pool must not be attended"
    del run
    _free()


def test_compress_plain_mean():
    """Pooling without the learned weights (gates and ape NULL) against the oracle's plain mean: bit-exact on
    dyadic keys (every step exact in fp32), within one bf16 ulp on random bf16 keys; and NULL gates / ape write
    the same rows as explicit zeros."""
    import sparse_attention_kpool_amd as K
    wl = _small_decode("plain_mean", ctx=(64, 1000))
    run = DeviceRun(wl)
    P, D = wl.P, wl.D
    rng = np.random.default_rng(21)
    seqs = np.array([0] * 16 + [1] * 8, np.int32)
    pids = np.array(list(range(16)) + list(range(100, 108)), np.int32)
    n = len(seqs)
    dev = lambda a: torch.from_numpy(a).to("cuda")
    for kind in ("dyadic", "random"):
        if kind == "dyadic":
            keys = rng.integers(-64, 65, size=(n, P, D)).astype(np.float64) / 8.0
        else:
            keys = O.bf16_round(rng.standard_normal((n, P, D)) * 3.0)
        kt = dev(keys.astype(np.float32)).to(torch.bfloat16).contiguous()
        K.kpool_compress(run.dims, run.cache, kt, None, None, dev(seqs), dev(pids))
        torch.cuda.synchronize()
        ref = O.store_round(O.pool_mean(keys), "bf16")
        for t in range(n):
            got = run.pooled_rows(int(seqs[t]), [int(pids[t])])[0]
            if kind == "dyadic":
                np.testing.assert_array_equal(got, ref[t], err_msg=f"plain mean, pool {t}")
            else:
                ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref[t]), 1e-30))[1] - 8)
                assert (np.abs(got - ref[t]) <= ulp).all(), f"plain mean, pool {t}"
        first = run.pooled.clone()
        zeros = torch.zeros_like(kt)
        K.kpool_compress(run.dims, run.cache, kt, zeros, zeros[0], dev(seqs), dev(pids))
        torch.cuda.synchronize()
        assert torch.equal(first, run.pooled), "NULL gates/ape differ from explicit zeros"
    del run
    _free()


def test_empty_calls():
    """n_q = 0 and n_pools = 0 are valid and write nothing."""
    import sparse_attention_kpool_amd as K
    wl = _small_decode("empty", ctx=(64,))
    run = DeviceRun(wl)
    before = run.pooled.clone()
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    qe = K.Queries(seq=e, pos=e, max_pos=0)
    K.dsa_indexer_score(run.dims, run.cache, qe, run.q_idx, run.w, run.layer.scores[:0])
    K.dsa_topk_select(run.dims, qe, run.layer.scores[:0], run.layer.sel[:0], run.layer.n_sel[:0])
    K.sparse_mla_attn(run.dims, run.cache, qe, run.q, run.layer.sel[:0], run.layer.n_sel[:0], run.out[:0])
    K.kpool_compress(run.dims, run.cache, run.q_idx, run.q_idx, run.q_idx, e, e)
    torch.cuda.synchronize()
    assert torch.equal(before, run.pooled)
    del run
    _free()


# ----------------------------------------------------------------------------------------------------------
# published workload shapes at full size: sampled queries
# ----------------------------------------------------------------------------------------------------------
def test_full_decode32k():
    wl = ks.workloads()["decode32k"]
    _say("[case decode32k] B=1 T=32768")
    run = DeviceRun(wl).run()
    check_run(run, [0])
    del run
    _free()


def test_full_decode128k():
    wl = ks.workloads()["decode128k"]
    _say("[case decode128k] B=1 T=131072")
    run = DeviceRun(wl).run()
    check_run(run, [0])
    del run
    _free()


@pytest.mark.slow
def test_full_batch64():
    wl = ks.workloads()["batch64"]
    _say(f"[case batch64] B=64 sumT={sum(wl.ctx)}")
    run = DeviceRun(wl).run()
    ctx = np.array(wl.ctx)
    picks = sorted({int(ctx.argmax()), int(ctx.argmin()), 0, 31, 63,
                    int(np.flatnonzero(ctx % 4 == 0)[0]), int(np.flatnonzero(ctx % 4 == 1)[0])})
    check_run(run, picks)
    del run
    _free()


@pytest.mark.slow
def test_full_prefill64k():
    wl = ks.workloads()["prefill64k"]
    _say("[case prefill64k] 4096 queries on 65536 tokens")
    run = DeviceRun(wl).run()
    check_run(run, [0, 1, 2, 3, 1234, 2047, 4094, 4095], n_compress_check=1024)
    del run
    _free()


@pytest.mark.slow
def test_full_long1m():
    wl = ks.workloads()["long1m"]
    _say("[case long1m] B=8 T=1048576")
    run = DeviceRun(wl).run()
    check_run(run, [0, 5])
    del run
    _free()
