"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, stage by stage and end to end.

Each stage is compared on the inputs the previous GPU stage produced, so a mismatch names its stage:
  compress  pooled-cache rows written in-step  vs  oracle pooling of the same key/gate rows (bit-exact on the
            constant-key parity instance; <= 1 bf16 ulp / 1e-6 relative in fp32 otherwise)
  score     GPU score row  vs  oracle scores from the GPU's pooled cache (bit-exact on integer data)
  select    GPU selection  vs  oracle top-k of the GPU's own score row (always bit-exact)
  attend    GPU output     vs  oracle attention over the GPU's selection (bf16: max-abs 3e-2, rel-RMS 1e-2;
            fp32: max-abs 1e-4, rel-RMS 1e-5)
On the parity instance the oracle's own end-to-end selection must equal the GPU's as well.
Full-size workloads check every query's score row and selection, and the attention output of every decode query
(of 32 sampled queries in the 4096-query prefill).  Every output buffer sits between guard bands that must stay
untouched, and no score may be written past a query's visible pools.
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


def check_run(run: DeviceRun, samples, n_compress_check=64, parity=True, attn_samples=None):
    """Stage-by-stage parity of `samples` (query indices); attention only for `attn_samples` (default: all)."""
    wl = run.wl
    P = wl.P
    run.check_guards()
    attn_samples = set(samples if attn_samples is None else attn_samples)
    errs, refs, max_abs = [], [], 0.0
    near_ties = 0
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
            bound = None
        else:
            # fp32 accumulation of D products per head and Hi weighted heads: |error| <= ~(D + Hi) 2^-24 sum|terms|
            bound = 1e-5 * (np.abs(w)[None, :] * (np.abs(gpu_pooled) @ np.abs(qidx).T)).sum(1) + 1e-30
            assert (np.abs(got_scores - ref_scores) <= bound).all(), f"scores q{j}"
        sel_row, ns = run.sel_row(j)
        ref_sel = O.select_pools(got_scores, i, P, wl.k)
        assert ns == len(ref_sel), f"n_sel q{j}: {ns} != {len(ref_sel)}"
        np.testing.assert_array_equal(sel_row[:ns], ref_sel, err_msg=f"selection q{j} (seq {s}, pos {i})")
        assert (sel_row[ns:] == -1).all(), f"padding q{j}"
        if parity:
            # end to end: the oracle's own pooled cache (asserted equal above) and its own scores select the same
            np.testing.assert_array_equal(O.select_pools(ref_scores, i, P, wl.k), ref_sel,
                                          err_msg=f"end-to-end selection q{j}")
        else:
            # general instance: the oracle's selection from exact scores may differ from the GPU's only where the
            # budget's boundary scores lie within the fp32 error bound of each other
            near_ties += tie_aware_selection(ref_scores, got_scores, bound, sel_row[:ns], i, P, wl.k, f"q{j}")
        if j not in attn_samples:
            continue
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
    _say(f"  {wl.name}: {len(samples)} queries ({len(attn_samples)} attended), attention max-abs {max_abs:.3g} "
         f"(<= {tol_abs}), rel-RMS {rr:.3g} (<= {tol_rel})" + ("" if parity else f", near-tie selections {near_ties}"))
    assert max_abs <= tol_abs, f"attention max-abs {max_abs}"
    assert rr <= tol_rel, f"attention rel-RMS {rr}"


def tie_aware_selection(exact, got_scores, bound, gpu_sel, i, P, k, what) -> int:
    """The oracle's selection from exact scores against the GPU's: equal, or differing only in pools whose exact
    scores lie within the fp32 error bound of the budget's boundary score.  Returns 1 if such a near tie decided a
    pool, else 0."""
    own = O.select_pools(exact, i, P, k)
    if np.array_equal(own, gpu_sel):
        return 0
    n_c, r, tau = O.pool_geometry(i, P)
    budget = min(k - (1 if r else 0), n_c)
    thr = np.sort(exact)[::-1][budget - 1]
    diff = set(own.tolist()) ^ set(np.asarray(gpu_sel).tolist())
    for p in diff:
        assert p < n_c and abs(exact[p] - thr) <= 2 * bound[p] + 2 * bound.max(), \
            f"selection {what}: pool {p} differs from the oracle's without a near tie"
    return 1


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
    # general instance at full dims, bf16: keys drawn per token, so the learned pooling weights (gate + position
    # term) decide the pooled keys; 16 pools per sequence compressed in-step (a decode batch after a short chunk)
    "small_decode_general": lambda: _small_decode("small_decode_general", key_per_token=True,
                                                  new_from=[max(0, t - 64) for t in (37, 1000, 4099, 8192, 20001)]),
    # general instance, prefill chunk: 125 pools compressed in-step from per-token keys, 500 queries
    "small_prefill_general": lambda: ks.scaled(ks.workloads()["prefill64k"], name="small_prefill_general",
                                               ctx=[3000], new_from=[2500], q_seq=np.zeros(500, np.int32),
                                               q_pos=np.arange(2500, 3000, dtype=np.int32), k=256,
                                               key_per_token=True),
    # 200 decode queries over 8 sequences (25 consecutive positions each): the decode scorer's cursor search past
    # the first 64 queries, one-block top-k rows, two attention splits
    "many_queries": lambda: ks.scaled(ks.workloads()["batch64"], name="many_queries",
                                      ctx=[1000 + 977 * s for s in range(8)],
                                      new_from=[1000 + 977 * s - 25 for s in range(8)],
                                      q_seq=np.repeat(np.arange(8, dtype=np.int32), 25),
                                      q_pos=np.concatenate([np.arange(1000 + 977 * s - 25, 1000 + 977 * s)
                                                            for s in range(8)]).astype(np.int32),
                                      k=256, page_perm_seed=9),
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


@pytest.mark.parametrize("case", ["small_decode_general", "two_step_mixed"])
def test_decode_step_graph_replay(case):
    """The layer step captured in a HIP graph (as a serving loop replays its decode step): every replay writes what
    the eager step wrote, bit for bit -- pooled keys of the pools completing in-step, scores, selection, output and
    lse -- with every output cleared by eager work and a synchronisation between the replays."""
    from harness import SENTINEL
    wl = SMALL[case]()
    _say(f"[case graph_replay {case}] n_q={wl.n_q}")
    run = DeviceRun(wl).run()
    L, d = run.layer, run.inputs
    ppp = wl.page_tokens // wl.P
    done = None
    if d.c_seq is not None:   # cache rows of the pools compressed in-step
        pages = d.block_table[d.c_seq.long(), (d.c_pool // ppp).long()].long()
        done = (pages, (d.c_pool % ppp).long())

    def bits(t):
        return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)

    def outputs():
        o = {"scores": L.scores, "sel": L.sel, "n_sel": L.n_sel, "out": run.out, "lse": run.lse}
        if done is not None:
            o["pooled"] = run.pooled[done[0], done[1]]
        return {k: bits(v).clone() for k, v in o.items()}

    ref = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.step(run.cache, run.queries, run.q_idx, run.w, run.q, run.out, lse=run.lse, compress=run.compress)
    for r in range(3):
        bits(L.scores).fill_(SENTINEL[torch.float32])
        L.sel.fill_(-7)
        L.n_sel.fill_(-7)
        bits(run.out).fill_(0x7FC1)
        bits(run.lse).fill_(0x7FC0DEAD)
        if done is not None:
            run.pooled[done[0], done[1]] = 0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {r}: {k} differs from the eager step"
        run.check_guards()
    del g, run
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


def test_split_merge_lane_groups():
    """The split merge at every lane grouping: batches of 10, 15, 20 and 25 queries (5 queries repeated) take
    26, 18, 13 and 11 splits, merged by groups of 4, 4, 2 and 2 lanes; every output row is within the attention
    tolerance of the 5-query call (52 splits, groups of 8), which the oracle checks, and its lse likewise."""
    import sparse_attention_kpool_amd as K
    wl = _small_decode("merge_lanes")
    _say("[case merge_lanes]")
    run = DeviceRun(wl).run()
    check_run(run, list(range(wl.n_q)))
    n5 = wl.n_q
    tol = attn_tolerance(wl.dtype)[0]
    for rep in (2, 3, 4, 5):
        idx = torch.arange(n5, device="cuda").repeat(rep)
        qs = K.Queries(seq=run.queries.seq[idx].contiguous(), pos=run.queries.pos[idx].contiguous(),
                       max_pos=run.queries.max_pos, group=1)
        sel, nsel = run.layer.sel[:n5][idx].contiguous(), run.layer.n_sel[:n5][idx].contiguous()
        out = torch.empty((n5 * rep, wl.H, wl.V), dtype=run.out.dtype, device="cuda")
        lse = torch.empty((n5 * rep, wl.H), dtype=torch.float32, device="cuda")
        ws = torch.empty((K.sparse_mla_workspace_size(run.dims, qs) + 15) // 16 * 4, dtype=torch.float32,
                         device="cuda")
        K.sparse_mla_attn(run.dims, run.cache, qs, run.q[idx].contiguous(), sel, nsel, out, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        err = (out.float() - run.out.float().repeat(rep, 1, 1)).abs().max().item()
        assert err <= tol, f"{n5 * rep} queries: max abs {err} against the 5-query call"
        lerr = (lse - run.lse.repeat(rep, 1)).abs().max().item()
        assert lerr <= 1e-3, f"{n5 * rep} queries: lse differs by {lerr}"
    del run
    _free()


def test_mtp_shared_selection():
    """MTP drafts reusing their targets' selections (sparse_mla_attn_shared): targets at T-2, drafts at T-1 of the
    same sequences.  A target reading its own row reproduces sparse_mla_attn bit for bit; a draft matches the oracle
    over the target's selected pools cut at the draft's own position plus the draft's own incomplete tail (so with
    T-1 = 9000 the draft attends token 9000, the first of a pool the target could not select)."""
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
        toks = O.shared_attended_tokens(sel_t[:ns], i, wl.P)
        ref_out, ref_lse = O.sparse_mla(ks.host_q(wl, s, i)[0], ks.host_latent(wl, s, toks), wl.scale, wl.V)
        got = out[d].float().cpu().numpy()
        assert np.abs(got - ref_out).max() <= tol_abs, f"draft {d}: max-abs"
        assert rel_rms(got, ref_out) <= tol_rel, f"draft {d}: rel-RMS"
        np.testing.assert_allclose(lse[d].cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-3, err_msg=f"draft {d} lse")
        assert i in set(toks.tolist()), f"draft {d} must attend itself"
        if i == 9000:
            assert 9000 // wl.P not in set(sel_t[:ns].tolist()), "the target could not have selected pool 2250"
    del run
    _free()


def test_mtp_runs_one_gather():
    """sparse_mla_attn_mtp: queries 2r (target) and 2r + 1 (draft) attend selection row r.  Runs of one sequence
    (targets at T-2, drafts at T-1; the draft at 9000 starts a pool the target could not select), a run whose two
    queries are of different sequences (each query's rows listed on their own), and an odd last run (a target
    alone).  Every query matches the oracle over the tokens sparse_mla_attn_shared with sel_row[i] = i // 2 would
    give it, and that call within the attention tolerance; nothing is written outside out / lse."""
    import sparse_attention_kpool_amd as K
    from harness import Guarded
    ctx = [37, 1000, 4099, 9001, 20000, 3000, 512]
    q_seq = [0, 0, 1, 1, 2, 2, 3, 3, 4, 5, 6]
    q_pos = [35, 36, 998, 999, 4097, 4098, 8999, 9000, 19998, 2999, 511]
    base = ks.workloads()["batch64"]
    wl = ks.scaled(base, name="mtp_runs", ctx=ctx, new_from=[t - 2 for t in ctx],
                   q_seq=np.array(q_seq, np.int32), q_pos=np.array(q_pos, np.int32), page_perm_seed=11)
    n_q, n_runs = wl.n_q, (wl.n_q + 1) // 2
    _say(f"[case mtp_runs] n_q={n_q} runs={n_runs}")
    run = DeviceRun(wl).run()
    targets = torch.arange(0, n_q, 2, device="cuda")
    sel = run.layer.sel[:n_q][targets].contiguous()
    n_sel = run.layer.n_sel[:n_q][targets].contiguous()
    ws_n = K.sparse_mla_mtp_workspace_size(run.dims, run.queries)
    ws = torch.empty(max(ws_n // 4, 4), dtype=torch.float32, device="cuda")
    g_out = Guarded((n_q, wl.H, wl.V), torch.bfloat16, "cuda")
    g_lse = Guarded((n_q, wl.H), torch.float32, "cuda")
    K.sparse_mla_attn_mtp(run.dims, run.cache, run.queries, run.q, sel, n_sel, g_out.t, lse=g_lse.t, workspace=ws)
    torch.cuda.synchronize()
    assert g_out.intact() and g_lse.intact(), "sparse_mla_attn_mtp wrote outside out / lse"
    out, lse = g_out.t, g_lse.t
    # the same sets through sparse_mla_attn_shared
    sel_row = torch.arange(n_q, device="cuda", dtype=torch.int32) // 2
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    K.sparse_mla_attn_shared(run.dims, run.cache, run.queries, run.q, sel, n_sel, sel_row, out2, lse=lse2,
                             workspace=run.layer.ws_attn)
    torch.cuda.synchronize()
    tol_abs, tol_rel = attn_tolerance(wl.dtype)
    for i in range(n_q):
        s, p = q_seq[i], q_pos[i]
        sel_t, ns = run.sel_row(2 * (i // 2))
        toks = O.shared_attended_tokens(sel_t[:ns], p, wl.P)
        ref_out, ref_lse = O.sparse_mla(ks.host_q(wl, s, p)[0], ks.host_latent(wl, s, toks), wl.scale, wl.V)
        for name, o, l in (("mtp", out, lse), ("shared", out2, lse2)):
            got = o[i].float().cpu().numpy()
            assert np.abs(got - ref_out).max() <= tol_abs, f"{name} query {i}: max-abs"
            assert rel_rms(got, ref_out) <= tol_rel, f"{name} query {i}: rel-RMS"
            np.testing.assert_allclose(l[i].cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-3, err_msg=f"{name} q {i}")
        assert p in set(toks.tolist()), f"query {i} must attend itself"
    assert 9000 // wl.P not in set(run.sel_row(6)[0][:run.sel_row(6)[1]].tolist())
    # the layer's verification step (score and select the targets alone, then one gather per run) writes the same
    # bits as the calls above
    from sparse_attention_kpool_amd.layer import KPoolDSALayer
    d = run.inputs
    tq = K.Queries(seq=d.q_seq[0::2].contiguous(), pos=d.q_pos[0::2].contiguous(), max_pos=wl.max_pos(), group=1)
    layer = KPoolDSALayer(run.dims, "cuda", max_q=n_q, max_pos=wl.max_pos(), mtp=True)
    out3, lse3 = torch.empty_like(out), torch.empty_like(lse)
    layer.verify_step(run.cache, run.queries, tq, run.q_idx[0::2].contiguous(), run.w[0::2].contiguous(), run.q,
                      out3, lse=lse3)
    torch.cuda.synchronize()
    assert torch.equal(layer.sel[:n_runs], sel) and torch.equal(layer.n_sel[:n_runs], n_sel)
    assert torch.equal(out3, out) and torch.equal(lse3, lse), "verify_step differs from the direct calls"
    del run, layer
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


def test_compress_through_ring():
    """kpool_compress reading each pool's key / gate rows from a per-sequence ring through `src` (the decode step's
    form: the ring holds every sequence's pending P rows, src names the sequences whose pool completes) writes the
    same pooled rows as compressing the same rows laid out in order, and both match the oracle (general instance:
    per-token keys, within one bf16 ulp)."""
    import sparse_attention_kpool_amd as K
    ctx = (1000, 4100, 8192, 20000, 64, 12)
    wl = _small_decode("ring", ctx=ctx, key_per_token=True)
    _say("[case compress_ring]")
    run = DeviceRun(wl)
    P, D = wl.P, wl.D
    seqs = [s for s, t in enumerate(ctx) if t % P == 0]       # the sequences whose last pool completes now
    pools = [ctx[s] // P - 1 for s in seqs]
    # the ring: one [P, D] slot per sequence, in a shuffled slot order
    slot = np.random.default_rng(4).permutation(len(ctx))
    keys = torch.zeros((len(ctx), P, D), dtype=torch.bfloat16, device="cuda")
    gates = torch.zeros_like(keys)
    for s, p in zip(seqs, pools):
        kk, gg = ks.device_tokens(wl, s, np.arange(p * P, p * P + P), "cuda")
        keys[slot[s]], gates[slot[s]] = kk, gg
    ape = ks.device_ape(wl, "cuda")
    dev = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to("cuda")
    K.kpool_compress(run.dims, run.cache, keys, gates, ape, dev(seqs), dev(pools), src=dev([slot[s] for s in seqs]))
    torch.cuda.synchronize()
    via_ring = [run.pooled_rows(s, [p])[0] for s, p in zip(seqs, pools)]
    run.pooled.zero_()
    ordered = torch.stack([keys[slot[s]] for s in seqs]).contiguous()
    ordered_g = torch.stack([gates[slot[s]] for s in seqs]).contiguous()
    K.kpool_compress(run.dims, run.cache, ordered, ordered_g, ape, dev(seqs), dev(pools))
    torch.cuda.synchronize()
    for t, (s, p) in enumerate(zip(seqs, pools)):
        bulk = run.pooled_rows(s, [p])[0]
        np.testing.assert_array_equal(via_ring[t], bulk, err_msg=f"ring vs bulk, seq {s}")
        toks = np.arange(p * P, p * P + P)
        ref = O.store_round(O.pool_compress(ks.host_token_keys(wl, s, toks)[None], ks.host_gates(wl, s, toks)[None],
                                            ks.host_ape(wl)), "bf16")[0]
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
        assert (np.abs(bulk - ref) <= ulp).all(), f"ring compress vs oracle, seq {s}"
    del run
    _free()


def _ints(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


FUSED = {
    # 4 sequences x 16 pools pooled in the call (64 entries, one launch): every segment holds many of them
    "general_16_per_seq": lambda: (_small_decode("fused_general", ctx=(1000, 4099, 8192, 20001), key_per_token=True,
                                                 new_from=[t - 64 for t in (1000, 4099, 8192, 20001)]), {}),
    # 5 x 16 = 80 entries: more than one launch pools, so the two kernels run in order
    "over_64": lambda: (_small_decode("fused_over64", ctx=(1000, 4099, 8192, 20001, 3000), key_per_token=True,
                                      new_from=[t - 64 for t in (1000, 4099, 8192, 20001, 3000)]), {}),
    # 25 queries per sequence at consecutive positions: an entry is visible to the later queries only; sequence 0
    # has entries but no query; the first entry is listed twice
    "partly_visible": lambda: (SMALL["many_queries"](), {"drop_seq0": True, "duplicate": True}),
    # D = 32, one index head
    "narrow": lambda: (SMALL["small_bf16_narrow"](), {}),
    # fp32 storage, 64 tokens of one sequence scored as a decode batch (16 entries)
    "f32_decode_shape": lambda: (SMALL["tiny_general"](), {}),
}


@pytest.mark.parametrize("plain", [False, True], ids=["learned", "plain_mean"])
@pytest.mark.parametrize("case", list(FUSED))
def test_compress_score_fused(case, plain):
    """dsa_compress_score equals kpool_compress followed by dsa_indexer_score bit for bit: the whole pooled cache
    and every visible score column, whether the decode scorer pools the entries itself (up to 64) or the two kernels
    run (more).  Learned pooling and the plain mean (gates and ape NULL)."""
    import sparse_attention_kpool_amd as K
    wl, opt = FUSED[case]()
    _say(f"[case fused {case} plain={plain}] n_q={wl.n_q} dtype={wl.dtype}")
    runs = [DeviceRun(wl, group=1), DeviceRun(wl, group=1)]
    c = runs[0].compress
    n = int(c.pool_seq.numel())
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    seq, pid = c.pool_seq, c.pool_id
    if opt.get("duplicate"):
        src, seq, pid = (torch.cat([x, x[:1]]) for x in (src, seq, pid))
    keep = torch.ones(wl.n_q, dtype=torch.bool, device="cuda")
    if opt.get("drop_seq0"):
        keep = runs[0].queries.seq != 0
    qs = K.Queries(seq=runs[0].queries.seq[keep].contiguous(), pos=runs[0].queries.pos[keep].contiguous(),
                   max_pos=wl.max_pos(), group=1)
    m = int(keep.sum().item())
    gates, ape = (None, None) if plain else (c.gates, c.ape)
    a, b = runs
    K.kpool_compress(a.dims, a.cache, c.keys, gates, ape, seq, pid, src=src)
    K.dsa_indexer_score(a.dims, a.cache, qs, a.q_idx[keep], a.w[keep], a.layer.scores[:m])
    K.dsa_compress_score(b.dims, b.cache, c.keys, gates, ape, seq, pid, qs, b.q_idx[keep], b.w[keep],
                         b.layer.scores[:m], src=src)
    torch.cuda.synchronize()
    assert torch.equal(_ints(a.pooled), _ints(b.pooled)), "pooled cache differs"
    n_c = ((qs.pos.long() + 1) // wl.P).cpu().numpy()
    for j in range(m):
        assert torch.equal(_ints(a.layer.scores[j, :n_c[j]]), _ints(b.layer.scores[j, :n_c[j]])), f"scores of query {j}"
    if m == wl.n_q:
        for r in runs:
            r.check_guards()
    del runs, a, b
    _free()


def test_chunked_prefill_equals_one_shot():
    """A prefill of 500 queries run as chunks of 77, 128 and 200 queries (each chunk compressing the pools its
    tokens complete before it scores, as a chunked prefill does) gives the same scores and selections as one call
    with all 500, bit for bit, and the same attention output where the split count is the same (within the
    attention tolerance otherwise).  The last row also equals a decode step at context 3000 (the analogue of the
    prefill / ubatch / decode agreement test on the llama.cpp PR page)."""
    import sparse_attention_kpool_amd as K
    from sparse_attention_kpool_amd.layer import KPoolDSALayer
    wl = ks.scaled(ks.workloads()["prefill64k"], name="chunked", ctx=[3000], new_from=[2500],
                   q_seq=np.zeros(500, np.int32), q_pos=np.arange(2500, 3000, dtype=np.int32), k=256)
    _say("[case chunked_prefill]")
    one = DeviceRun(wl).run()
    check_run(one, [0, 1, 2, 3, 250, 498, 499])
    P = wl.P
    for chunk in (77, 128, 200):
        run = DeviceRun(wl)                                       # fresh caches: in-step pools start empty
        layer = KPoolDSALayer(run.dims, "cuda", max_q=chunk, max_pos=wl.max_pos())
        out = torch.empty_like(run.out)
        for a in range(0, wl.n_q, chunk):
            b = min(a + chunk, wl.n_q)
            qs = K.Queries(seq=run.queries.seq[a:b], pos=run.queries.pos[a:b], max_pos=int(wl.q_pos[b - 1]),
                           group=b - a)
            # pools completed by tokens a .. b-1 of the chunk (token 2500 + t is query t)
            p0, p1 = (2500 + a) // P, (2500 + b) // P
            comp = None
            if p1 > p0:
                c = run.compress
                sl = slice(p0 - 2500 // P, p1 - 2500 // P)
                from sparse_attention_kpool_amd.layer import CompressInput
                comp = CompressInput(keys=c.keys[sl].contiguous(), gates=c.gates[sl].contiguous(), ape=c.ape,
                                     pool_seq=c.pool_seq[sl].contiguous(), pool_id=c.pool_id[sl].contiguous())
            layer.step(run.cache, qs, run.q_idx[a:b], run.w[a:b], run.q[a:b], out[a:b], compress=comp)
            torch.cuda.synchronize()
            for j in range(a, b):
                n_c = (int(wl.q_pos[j]) + 1) // P
                assert torch.equal(layer.scores[j - a, :n_c], one.layer.scores[j, :n_c]), f"chunk {chunk}: scores {j}"
            assert torch.equal(layer.sel[:b - a], one.layer.sel[a:b]), f"chunk {chunk}: selection {a}..{b}"
            assert torch.equal(layer.n_sel[:b - a], one.layer.n_sel[a:b])
        same_split = K.sparse_mla_workspace_size(run.dims, K.Queries(seq=run.queries.seq[:chunk],
                                                                     pos=run.queries.pos[:chunk], max_pos=0)) == \
            K.sparse_mla_workspace_size(run.dims, run.queries)
        if same_split:
            assert torch.equal(out, one.out), f"chunk {chunk}: attention output"
        else:
            assert (out.float() - one.out.float()).abs().max().item() <= attn_tolerance(wl.dtype)[0]
        del run, layer
    # the last prefill row against a decode step at context 3000 on the prefilled caches
    dq = K.Queries(seq=one.queries.seq[-1:], pos=one.queries.pos[-1:], max_pos=2999, group=1)
    dec = KPoolDSALayer(one.dims, "cuda", max_q=1, max_pos=2999)
    dout = torch.empty_like(one.out[-1:])
    dec.step(one.cache, dq, one.q_idx[-1:], one.w[-1:], one.q[-1:], dout)
    torch.cuda.synchronize()
    assert torch.equal(dec.scores[0, :750], one.layer.scores[499, :750]) and torch.equal(dec.sel[0], one.layer.sel[499])
    assert (dout.float() - one.out[-1:].float()).abs().max().item() <= attn_tolerance(wl.dtype)[0]
    del one, dec
    _free()


def test_binding_rejects_bad_tensors():
    """The binding checks dtype, device, shape and contiguity before calling the library: a strided view of q (its
    first V columns), a wrong dtype and a short output raise ValueError and launch nothing."""
    import sparse_attention_kpool_amd as K
    wl = _small_decode("binding", ctx=(100, 2000))
    run = DeviceRun(wl).run()
    L, n = run.layer, wl.n_q
    with pytest.raises(ValueError):
        K.sparse_mla_attn(run.dims, run.cache, run.queries, run.q[:, :, :wl.V], L.sel[:n], L.n_sel[:n], run.out)
    with pytest.raises(ValueError):
        K.sparse_mla_attn(run.dims, run.cache, run.queries, run.q.float(), L.sel[:n], L.n_sel[:n], run.out)
    with pytest.raises(ValueError):
        K.sparse_mla_attn(run.dims, run.cache, run.queries, run.q, L.sel[:n], L.n_sel[:n], run.out[:1])
    with pytest.raises(ValueError):
        K.dsa_indexer_score(run.dims, run.cache, run.queries, run.q_idx, run.w.to(torch.bfloat16), L.scores[:n])
    with pytest.raises(ValueError):
        K.dsa_topk_select(run.dims, run.queries, L.scores[:n], L.sel[:n, :10], L.n_sel[:n])
    with pytest.raises(ValueError):
        K.kpool_compress(run.dims, run.cache, run.q_idx, None, None, L.n_sel[:1], L.n_sel[:1])
    run.check_guards()
    del run
    _free()


# ----------------------------------------------------------------------------------------------------------
# published workload shapes at full size
# ----------------------------------------------------------------------------------------------------------
def check_all_rows(run: DeviceRun, chunk=64):
    """Every query's score row (bit-exact against exact scores from the GPU's pooled cache, which must itself equal
    the oracle's) and selection (against the oracle's top-k of that row), vectorised per sequence."""
    wl = run.wl
    P = wl.P
    for s in sorted(set(wl.q_seq.tolist())):
        js = np.flatnonzero(wl.q_seq == s)
        n_cmax = (int(wl.q_pos[js].max()) + 1) // P
        pooled = run.pooled_rows(s, np.arange(n_cmax))
        np.testing.assert_array_equal(pooled, oracle_pooled(wl, s, n_cmax), err_msg=f"pooled cache seq {s}")
        for c0 in range(0, len(js), chunk):
            jj = js[c0:c0 + chunk]
            qidx = ks.host_qidx(wl, np.full(len(jj), s), wl.q_pos[jj]).astype(np.float64)   # [c, Hi, D]
            w = ks.host_w(wl, np.full(len(jj), s), wl.q_pos[jj]).astype(np.float64)         # [c, Hi]
            for t, j in enumerate(jj):
                i = int(wl.q_pos[j])
                n_c = (i + 1) // P
                exact = O.indexer_scores(qidx[t], w[t], pooled, n_c)
                got = run.scores_row(int(j), n_c)
                np.testing.assert_array_equal(got, exact, err_msg=f"scores q{j} (seq {s}, pos {i})")
                sel, ns = run.sel_row(int(j))
                ref = O.select_pools(got, i, P, wl.k)
                assert ns == len(ref) and np.array_equal(sel[:ns], ref), f"selection q{j}"
                assert (sel[ns:] == -1).all(), f"padding q{j}"
    _say(f"  {wl.name}: all {wl.n_q} score rows and selections exact")
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
    check_run(run, list(range(wl.n_q)))                     # every query: scores, selection, output
    del run
    _free()


@pytest.mark.slow
def test_full_prefill64k():
    wl = ks.workloads()["prefill64k"]
    _say("[case prefill64k] 4096 queries on 65536 tokens")
    run = DeviceRun(wl).run()
    check_all_rows(run)                                     # all 4096 score rows and selections
    picks = sorted(set([0, 1, 2, 3, 4094, 4095] + np.random.default_rng(8).choice(4096, 26, replace=False).tolist()))
    check_run(run, picks, n_compress_check=1024)            # attention of 32 queries
    del run
    _free()


@pytest.mark.slow
def test_full_max_two_step_row():
    """One sequence at 2,097,152 tokens, paged: a row of 524,288 pools, the longest the two-step selection takes
    (16 chunks of 32,768 pools, merged as a tree of four groups of four), scored by the decode scorer and attended
    in 64 splits; every stage against the oracle."""
    T = 1 << 21
    wl = ks.scaled(ks.workloads()["decode32k"], name="max_row", ctx=[T], new_from=[T - 1],
                   q_seq=np.zeros(1, np.int32), q_pos=np.array([T - 1], np.int32), seed=6, page_perm_seed=66)
    _say(f"[case max_row] B=1 T={T}")
    run = DeviceRun(wl).run()
    check_run(run, [0])
    del run
    _free()


@pytest.mark.slow
def test_full_long1m():
    wl = ks.workloads()["long1m"]
    _say("[case long1m] B=8 T=1048576")
    run = DeviceRun(wl).run()
    check_run(run, list(range(wl.n_q)))                     # all 8 queries
    del run
    _free()
