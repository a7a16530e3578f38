#!/usr/bin/env python3
"""Benchmark of the KPool-DSA layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--legs decode,ceiling,32k,...]

A step is one pass of the whole layer -- kpool_compress (pools completing this step) -> dsa_indexer_score ->
dsa_topk_select -> sparse_mla_attn -- over one batch, enqueued on one stream through the C ABI (a decode step
pools and scores in one launch: dsa_compress_score).

Legs (inputs are seeded synthetic data already resident in HBM when timing starts):
  decode   the headline: 64 sequences, contexts U[8192, 131072] (seed 3, up to 128K), paged 64-token pages,
           full layer dims (index 32 x 128, pool 4, top-k 2048, 64 MLA heads on a 576 latent), bf16.
           `value` = decode tokens/s = 64 / step time.  Two copies of the caches alternate between steps so the
           256 MB Infinity Cache cannot serve one step from the previous one.
  ceiling  (with decode / long1m) the read-only gather of the step's own rows -- the attended tokens' 1 KiB value
           rows and the scanned 4 KiB pooled-key pages -- through kp_read_rows: what HBM delivers for these access
           patterns with nothing else running, the practical ceiling the stages are compared with.
  32k      one sequence at context 32,768 (latency-bound: its 10.6 MB is below what fills the machine),
           rotating 40 cache copies; also timed as a HIP graph replay.
  128k     one sequence at context 131,072 (the exact 128K point), rotating 40 cache copies.
  long1m   8 sequences at context 1,048,576.
  fp8      the 64-sequence decode over an fp8 (E4M3) latent cache.
  proj     the dense projections beside the path, at 64 and 4096 tokens.
  prefill  4096 new queries on 65,536 tokens: the indexer's TFLOP/s against the bf16 MFMA peak, and the
           whole prefill step.
  copy     a plain 1 GiB device-to-device copy: the achievable-bandwidth reference, and the kernel of known
           traffic against which the FETCH_SIZE / WRITE_SIZE counters are scaled.
Step times: `ms_per_step` is the mean over the whole timed region (the headline `value` is 64 / that); the median
and min of the per-step times come with it.  The CPU baseline is the oracle on this machine's host cores (see
`cpu_baseline`).  Rank 0 prints one JSON line.  Algorithmic bytes/flops count what the method must move or compute; the
derivation is in the docstrings of `decode_bytes` and `prefill_flops`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
METRIC = "KPool-DSA decode tokens/s + HBM GB/s at 128K ctx; prefill indexer TFLOP/s"


# ----------------------------------------------------------------------------------------------------------
# algorithmic work
# ----------------------------------------------------------------------------------------------------------
def attended(pos: int, P: int, k: int) -> int:
    """|S|: tokens a query at position pos attends (selected complete pools x P, plus the causal tail)."""
    n_c, r = (pos + 1) // P, (pos + 1) % P
    return min(k - (1 if r else 0), n_c) * P + r


def decode_bytes(wl) -> dict:
    """Bytes each stage must move, per step (bf16 storage, es = 2):
      compress  per completing pool: P key + P gate rows in (2*P*D*es), one pooled row out (D*es)
      score     per query: the pooled-key scan D*es*n_c, its index query Hi*D*es and weights Hi*4
      topk      per query: the selection written, k*4
      attend    per query: the V-wide value columns of every attended token V*les*|S| (les = 1 for an fp8
                latent cache, else es), the query's nope part H*V*es, the output H*V*es, the selection read k*4
    Score rows and split-KV partials are intermediate traffic, not algorithmic.  A decode step pools in its scoring
    launch (dsa_compress_score), so its score stage moves the compress bytes too (see fused_stage_bytes)."""
    es = 2 if wl.dtype == "bf16" else 4
    les = 1 if wl.latent_fp8 else es
    P, D, Hi, k, H, V = wl.P, wl.D, wl.Hi, wl.k, wl.H, wl.V
    n_complete = sum(t // P - nf // P for t, nf in zip(wl.ctx, wl.new_from))
    out = dict(compress=n_complete * (2 * P * D * es + D * es), score=0, topk=0, attend=0)
    for pos in wl.q_pos.tolist():
        n_c = (pos + 1) // P
        out["score"] += D * es * n_c + Hi * D * es + Hi * 4
        out["topk"] += k * 4
        out["attend"] += V * les * attended(pos, P, k) + 2 * H * V * es + k * 4
    return out


def fused_stage_bytes(by: dict) -> dict:
    """decode_bytes by stage as a decode step launches them: pooling folded into the scoring launch."""
    return {"score": by["score"] + by["compress"], "topk": by["topk"], "attend": by["attend"]}


def prefill_flops(wl) -> int:
    """Indexer flops: 2 * Hi * D per (query, visible complete pool) -- causal pools only."""
    return int(sum(2 * wl.Hi * wl.D * ((p + 1) // wl.P) for p in wl.q_pos.tolist()))


# ----------------------------------------------------------------------------------------------------------
# device legs
# ----------------------------------------------------------------------------------------------------------
class Leg:
    def __init__(self, wl, copies: int, group=None):
        import torch
        import kpool_synth as ks
        import sparse_attention_kpool_amd as K
        from sparse_attention_kpool_amd.layer import CompressInput, KPoolDSALayer
        self.torch, self.K = torch, K
        self.wl = wl
        d = ks.DeviceInputs(wl, "cuda")
        self.d = d
        self.dims = K.Dims(pool=wl.P, idx_dim=wl.D, idx_heads=wl.Hi, topk=wl.k, heads=wl.H, latent_dim=wl.L,
                           v_dim=wl.V, page_tokens=wl.page_tokens, dtype=wl.dtype, scale=wl.scale)
        self.caches = [K.Cache(latent=d.latent, pooled=d.pooled, block_table=d.block_table, latent_scale=wl.kv_scale)]
        for _ in range(copies - 1):
            self.caches.append(K.Cache(latent=d.latent.clone(), pooled=d.pooled.clone(), latent_scale=wl.kv_scale,
                                       block_table=d.block_table))
        if group is None:
            group = wl.n_q if len(set(wl.q_seq.tolist())) == 1 else 1
        self.queries = K.Queries(seq=d.q_seq, pos=d.q_pos, max_pos=wl.max_pos(), group=group)
        self.compress = None if d.c_keys is None else CompressInput(
            keys=d.c_keys, gates=d.c_gates, ape=d.ape, pool_seq=d.c_seq, pool_id=d.c_pool)
        self.layer = KPoolDSALayer(self.dims, "cuda", max_q=wl.n_q, max_pos=wl.max_pos())
        self.out = torch.empty((wl.n_q, wl.H, wl.V), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def step(self, i: int):
        self.layer.step(self.caches[i % len(self.caches)], self.queries, self.d.q_idx, self.d.w, self.d.q,
                        self.out, lse=self.lse, compress=self.compress)

    def time_steps(self, steps: int, warmup: int) -> dict:
        """ms per step over `steps` back-to-back steps: the mean over the whole timed region, and the median and min
        of the per-step times (HIP events recorded between the steps on the launch stream)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            self.step(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": float(np.median(per)), "min": min(per)}

    def time_steps_graph(self, steps: int, warmup: int, replays: int = 5) -> dict:
        """ms per step with `steps` steps captured in one HIP graph and replayed, as a serving loop replays its
        captured decode step: `mean` from the first timed replay (exactly `steps` steps, after three untimed
        replays: the first replays after a capture run a few per cent slower), `median` and `min` of the per-step
        times of `replays` timed replays."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                self.step(i)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(replays):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps)
        del g
        return {"mean": per[0], "median": float(np.median(per)), "min": min(per)}

    def time_stages(self, steps: int, split_compress: bool = False) -> dict:
        """Mean ms per stage, events recorded between the calls on the launch stream.  Stages as the layer step
        launches them: `score` is the step's pooling and scoring (dsa_compress_score: one launch for a decode
        batch); split_compress times kpool_compress on its own first (`compress`) and `score` without it.  The
        steps are enqueued back to back with one synchronisation at the end, so the host runs ahead of the device
        and no stage includes the device waiting for a launch."""
        torch, K, L = self.torch, self.K, self.layer
        n_q = self.wl.n_q
        names = (["compress"] if split_compress else []) + ["score", "topk", "attend"]
        c = self.compress
        evs = []
        torch.cuda.synchronize()
        for i in range(steps):
            cache = self.caches[i % len(self.caches)]
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
            ev[0].record()
            if split_compress:
                if c is not None:
                    K.kpool_compress(self.dims, cache, c.keys, c.gates, c.ape, c.pool_seq, c.pool_id, src=c.src)
                ev[1].record()
                K.dsa_indexer_score(self.dims, cache, self.queries, self.d.q_idx, self.d.w, L.scores[:n_q])
            else:
                L._compress_score(cache, c, self.queries, self.d.q_idx, self.d.w, L.scores[:n_q])
            ev[len(names) - 2].record()
            K.dsa_topk_select(self.dims, self.queries, L.scores[:n_q], L.sel[:n_q], L.n_sel[:n_q],
                              workspace=L.ws_topk)
            ev[len(names) - 1].record()
            if cache.latent.dtype == torch.uint8:
                K.sparse_mla_attn_fp8(self.dims, cache, self.queries, self.d.q, L.sel[:n_q], L.n_sel[:n_q],
                                      cache.latent_scale, self.out, lse=self.lse, workspace=L.ws_attn)
            else:
                K.sparse_mla_attn(self.dims, cache, self.queries, self.d.q, L.sel[:n_q], L.n_sel[:n_q], self.out,
                                  lse=self.lse, workspace=L.ws_attn)
            ev[len(names)].record()
            evs.append(ev)
        torch.cuda.synchronize()
        acc = dict.fromkeys(names, 0.0)
        for ev in evs:
            for j, n in enumerate(names):
                acc[n] += ev[j].elapsed_time(ev[j + 1])
        return {n: acc[n] / steps for n in names}

    def attended_rows(self):
        """Physical latent rows of every token the last step attended (int32, in each query's selection order).
        Raises unless a step has run: the selection is checked on the host before it indexes the block table."""
        torch, wl = self.torch, self.wl
        P, pt = wl.P, wl.page_tokens
        bt = self.d.block_table.long()
        out = []
        for j in range(wl.n_q):
            s, pos = int(wl.q_seq[j]), int(wl.q_pos[j])
            ns = int(self.layer.n_sel[j].item())
            if not 0 <= ns <= wl.k:
                raise RuntimeError("attended_rows: no step has written the selection")
            p = self.layer.sel[j, :ns].long()
            if ns and (int(p.min().item()) < 0 or int(p.max().item()) > pos // P):
                raise RuntimeError("attended_rows: no step has written the selection")
            tok = (p[:, None] * P + torch.arange(P, device="cuda")[None, :]).reshape(-1)
            tok = tok[tok <= pos]
            out.append(bt[s, tok // pt] * pt + tok % pt)
        return torch.cat(out).to(torch.int32).contiguous()

    def scanned_pages(self):
        """Physical pages of every query's visible complete pools (the pooled-key pages the scorer streams)."""
        torch, wl = self.torch, self.wl
        ppp = wl.page_tokens // wl.P
        out = []
        for j in range(wl.n_q):
            s, n_c = int(wl.q_seq[j]), (int(wl.q_pos[j]) + 1) // wl.P
            out.append(self.d.block_table[s, :(n_c + ppp - 1) // ppp])
        return torch.cat(out).to(torch.int32).contiguous()

    def time_read_rows(self, which: str, reps: int = 20) -> dict:
        """The gather-bandwidth reference (kp_read_rows) over this workload's own rows: 'attend' = the attended
        tokens' 1 KiB value rows of the latent cache, 'score' = the scanned 4 KiB pages of the pooled cache;
        alternating cache copies, as the steps do."""
        torch, K = self.torch, self.K
        if which == "attend":
            rows, nbytes, bufs = self.attended_rows(), 1024, [c.latent.view(-1, self.wl.L) for c in self.caches]
        else:
            rows, nbytes, bufs = self.scanned_pages(), 4096, [c.pooled for c in self.caches]
        for i in range(3):
            K.read_rows(bufs[i % len(bufs)], nbytes, rows)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            K.read_rows(bufs[i % len(bufs)], nbytes, rows)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        b = rows.numel() * nbytes
        return {"rows": int(rows.numel()), "bytes": int(b), "ms": round(ms, 5), "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    def free(self):
        del self.caches, self.layer, self.d
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


# the batch-64 decode step's kernels by stage (the scorer pools the step's completed pools in the same launch)
STAGE_KERNELS = {"score": ["kp::score_decode_kernel<kp::bf16, 128, true>"],
                 "topk": ["kp::topk_chunk_kernel<16>", "kp::topk_merge_kernel<16, true>"],
                 "attend": ["kp::attn_dma_kernel<4, false, false>", "kp::attn_combine_kernel<kp::bf16, 8, 1>"]}


def mtp_leg(W, steps: int) -> dict:
    """MTP verification attention: 32 sequences of the batch-64 decode workload, each with a target query at T-2 and
    its draft at T-1 sharing the target's selection.  The same attention done two ways -- sparse_mla_attn_shared
    (each query gathers its own rows) and sparse_mla_attn_mtp (one gather per pair) -- timed as graph replays of
    `steps` calls over alternating cache copies, with the latent bytes each way gathers per query."""
    import torch
    import kpool_synth as ks
    import sparse_attention_kpool_amd as K
    base = W["batch64"]
    ctx = [int(t) for t in base.ctx[:32]]
    q_seq = np.repeat(np.arange(32, dtype=np.int32), 2)
    q_pos = np.array([[t - 2, t - 1] for t in ctx], np.int32).reshape(-1)
    wl = ks.scaled(base, name="mtp_verify", ctx=ctx, new_from=[t - 2 for t in ctx], q_seq=q_seq, q_pos=q_pos)
    leg = Leg(wl, copies=2)
    leg.step(0)
    torch.cuda.synchronize()
    n_q = wl.n_q
    sel = leg.layer.sel[:n_q][0::2].contiguous()            # the targets' rows, one per pair
    n_sel = leg.layer.n_sel[:n_q][0::2].contiguous()
    sel_row = torch.arange(n_q, device="cuda", dtype=torch.int32) // 2
    out = torch.empty((n_q, wl.H, wl.V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n_q, wl.H), dtype=torch.float32, device="cuda")
    ws_s = torch.empty(max(K.sparse_mla_workspace_size(leg.dims, leg.queries) // 4, 4), dtype=torch.float32,
                       device="cuda")
    ws_m = torch.empty(max(K.sparse_mla_mtp_workspace_size(leg.dims, leg.queries) // 4, 4), dtype=torch.float32,
                       device="cuda")

    def shared(i):
        K.sparse_mla_attn_shared(leg.dims, leg.caches[i % 2], leg.queries, leg.d.q, sel, n_sel, sel_row, out,
                                 lse=lse, workspace=ws_s)

    def mtp(i):
        K.sparse_mla_attn_mtp(leg.dims, leg.caches[i % 2], leg.queries, leg.d.q, sel, n_sel, out, lse=lse,
                              workspace=ws_m)

    def graph_ms(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(5):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps)
        del g
        return float(np.median(per))

    ms_s, ms_m = graph_ms(shared), graph_ms(mtp)
    # tokens each query attends (its target's selected pools cut at its position, plus its own incomplete tail),
    # and per pair the union the one-gather call reads
    P = wl.P
    sel_h, ns_h = sel.cpu().numpy(), n_sel.cpu().numpy()
    per_query = 0
    per_pair = 0
    for r in range(len(ctx)):
        sets = []
        for i in (2 * r, 2 * r + 1):
            pos = int(q_pos[i])
            pools = set(int(x) for x in sel_h[r, :min(int(ns_h[r]), wl.k)])
            if (pos + 1) % P:
                pools.add(pos // P)
            toks = {P * p + t for p in pools for t in range(P) if P * p + t <= pos}
            sets.append(toks)
            per_query += len(toks)
        per_pair += len(sets[0] | sets[1])
    row_b = wl.V * 2
    leg.free()
    return {"queries": n_q, "pairs": len(ctx), "shared_ms": round(ms_s, 5), "mtp_ms": round(ms_m, 5),
            "speedup": round(ms_s / ms_m, 3),
            "latent_mb_gathered": {"shared": round(per_query * row_b / 1e6, 2), "mtp": round(per_pair * row_b / 1e6, 2)},
            "latent_kb_per_query": {"shared": round(per_query * row_b / n_q / 1e3, 1),
                                    "mtp": round(per_pair * row_b / n_q / 1e3, 1)}}


def eager_stats(t: dict, n_q: int) -> dict:
    """The same steps launched one call at a time (no graph): ms per step (mean, median, min) and tokens/s."""
    return {"ms_per_step": round(t["mean"], 5), "ms_per_step_median": round(t["median"], 5),
            "ms_per_step_min": round(t["min"], 5), "tokens_per_s": round(n_q / (t["mean"] * 1e-3), 1)}


def measured_traffic(stage: str):
    """HBM bytes per launch of a stage's kernels from the committed counter record (profiles/), scaled by the
    copy-kernel calibration; None when any of those kernels' sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_batch64_decode.json")
    try:
        rec = json.load(open(path))
        total = 0.0
        for k in STAGE_KERNELS[stage]:
            e = rec["kernels"][k]
            h = hashlib.sha256()
            for src in e["sources"]:                      # the kernel's source file, then the shared device header
                h.update(open(os.path.join(ROOT, src), "rb").read())
            if h.hexdigest()[:16] != e["sha256_16"]:
                return None
            total += e["read_bytes"] + e["write_bytes"]
        return int(total)
    except (OSError, KeyError, ValueError):
        return None


def roofline(stage_ms: dict, stage_bytes: dict) -> dict:
    dom = max(("score", "attend"), key=lambda s: stage_ms[s])
    achieved = stage_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    return {"bound": "hbm", "stage": dom, "kernel": " + ".join(STAGE_KERNELS[dom]), "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": int(stage_bytes[dom]), "ms_per_launch": round(stage_ms[dom], 5),
            "traffic": measured_traffic(dom)}


# ----------------------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the decode step
# ----------------------------------------------------------------------------------------------------------
def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the host's CPU count
        return os.cpu_count() or 1


def _oracle_inputs(wl, j: int, ape):
    """Host inputs of decode query j (regenerated outside any timed region): pre-filled pooled keys, the key / gate
    rows of a pool completing this step, the queries, and the latent rows the query attends (found by one untimed
    selection pass) with a token -> row map, so the timed pass can gather through it."""
    import kpool_synth as ks
    import oracle as O
    s, i = int(wl.q_seq[j]), int(wl.q_pos[j])
    n_c, r, tau = O.pool_geometry(i, wl.P)
    first_new = wl.new_from[s] // wl.P
    pre = np.zeros((n_c, wl.D))
    pre[:min(first_new, n_c)] = ks.host_pool_keys(wl, s, np.arange(min(first_new, n_c))).astype(np.float64)
    comp = None
    if n_c > first_new:                                       # pools completing this step
        toks = np.arange(first_new * wl.P, n_c * wl.P)
        comp = (ks.host_token_keys(wl, s, toks).reshape(-1, wl.P, wl.D).astype(np.float64),
                ks.host_gates(wl, s, toks).reshape(-1, wl.P, wl.D).astype(np.float64), first_new)
        pre[first_new:] = O.store_round(O.pool_compress(comp[0], comp[1], ape), wl.dtype)
    qidx = ks.host_qidx(wl, s, i)[0].astype(np.float64)
    w = ks.host_w(wl, s, i)[0].astype(np.float64)
    q = ks.host_q(wl, s, i)[0].astype(np.float64)
    sel0 = O.select_pools(O.indexer_scores(qidx, w, pre, n_c), i, wl.P, wl.k)
    toks0 = O.attended_tokens(sel0, i, wl.P)
    rows = ks.host_latent(wl, s, toks0).astype(np.float64)
    tmap = np.full(i + 1, -1, dtype=np.int64)
    tmap[toks0] = np.arange(len(toks0))
    return (i, pre, comp, qidx, w, q, rows, tmap)


def _oracle_pass(wl, prepared, ape, stage: dict) -> None:
    """One pass of the whole layer per prepared query (pool, score, select, attend) in float64 numpy, adding each
    stage's wall time to `stage`."""
    import oracle as O
    for (i, pre, comp, qidx, w, q, rows, tmap) in prepared:
        n_c = (i + 1) // wl.P
        t0 = time.perf_counter()
        pooled = pre
        if comp is not None:
            pooled = pre.copy()
            pooled[comp[2]:n_c] = O.store_round(O.pool_compress(comp[0], comp[1], ape), wl.dtype)
        t1 = time.perf_counter()
        s_ = O.indexer_scores(qidx, w, pooled, n_c)
        t2 = time.perf_counter()
        sel = O.select_pools(s_, i, wl.P, wl.k)
        t3 = time.perf_counter()
        toks = O.attended_tokens(sel, i, wl.P)
        O.sparse_mla(q, rows[tmap[toks]], wl.scale, wl.V)
        t4 = time.perf_counter()
        for k, a, b in (("pool", t0, t1), ("score", t1, t2), ("select", t2, t3), ("attend", t3, t4)):
            stage[k] = stage.get(k, 0.0) + (b - a)


def _time_oracle(wl, queries, min_seconds: float) -> dict:
    import kpool_synth as ks
    ape = ks.host_ape(wl).astype(np.float64)
    prepared = [_oracle_inputs(wl, j, ape) for j in queries]
    stage, reps, t0 = {}, 0, time.perf_counter()
    while True:                                                 # repeat the sample to >= min_seconds of work
        _oracle_pass(wl, prepared, ape, stage)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    n = reps * len(queries)
    return {"tokens_per_s": round(n / dt, 3), "queries": n, "seconds": round(dt, 3),
            "stage_ms_per_query": {k: round(v / n * 1e3, 3) for k, v in stage.items()}}


def cpu_baseline(wl, n_sample: int, min_seconds: float = 10.0, extra: bool = True) -> dict:
    """The oracle as it stands, timed on this machine's host cores: a bounded sample of the decode workload with
    numpy's BLAS on all its threads (the reported baseline), then the tiny prefill (all 64 queries) and the
    32K-context decode single-threaded."""
    threads = _blas_threads()
    main = _time_oracle(wl, list(range(n_sample)), min_seconds)
    out = {"value": main["tokens_per_s"], "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "host_cpus": os.cpu_count(), "blas_threads": int(threads), "seconds": main["seconds"],
           "stage_ms_per_query": main["stage_ms_per_query"],
           "sample": f"{n_sample} of the 64 decode queries (sequences 0..{n_sample - 1}), repeated to "
                     f"{main['queries']} queries, the whole layer per query (pool, score, select, attend) in float64 "
                     f"numpy; host input regeneration not timed"}
    if extra:
        import kpool_synth as ks
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:
            threadpool_limits = None
        if threadpool_limits is not None:
            W = ks.workloads()
            with threadpool_limits(limits=1):
                out["single_thread"] = {
                    "tiny": dict(_time_oracle(W["tiny"], list(range(64)), 2.0), unit="queries/s"),
                    "decode32k": dict(_time_oracle(W["decode32k"], [0], 3.0), unit="tokens/s"),
                }
    return out

# the dense projections beside the path (kp_linear) at the layer's shapes: hidden 4096, q_lora 1536, 32 index heads
# x 128, 64 MLA heads, kv_lora 512, qk_nope = v_head = 256
PROJ_HIDDEN, PROJ_QRANK, PROJ_HI, PROJ_D, PROJ_H, PROJ_V, PROJ_DN, PROJ_DV, PROJ_L = 4096, 1536, 32, 128, 64, 512, \
    256, 256, 576


def proj_leg(T: int, reps: int, split: bool = True) -> dict:
    """Time each projection of a T-token step (HIP events around a graph replay of `reps` calls, mean per call),
    then the step's five as a layer launches them (one grouped launch before attention, the un-absorb after).
    Inputs: seeded N(0, 1) draws (weights x 2^-6) rounded to bf16."""
    import torch
    import sparse_attention_kpool_amd as K
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234 + T)

    def mat(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)
    hid, qr, Hi, D, H, V, dn, dv, L = (PROJ_HIDDEN, PROJ_QRANK, PROJ_HI, PROJ_D, PROJ_H, PROJ_V, PROJ_DN, PROJ_DV,
                                       PROJ_L)
    x, cq = mat(T, hid), mat(T, qr)
    w_q, w_w, w_kg = mat(Hi * D, qr, scale=2 ** -6), mat(Hi, hid, scale=2 ** -6), mat(2 * D, hid, scale=2 ** -6)
    q_nope, w_uk_t, w_uv = mat(T, H, dn), mat(H, V, dn, scale=2 ** -6), mat(H, dv, V, scale=2 ** -6)
    o_lat = mat(T, H, V)
    q_idx = torch.empty(T, Hi * D, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(T, Hi, dtype=torch.float32, device="cuda")
    keys = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    gates = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(T, H, L, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(T, H, dv, dtype=torch.bfloat16, device="cuda")
    # one split-K workspace for all five
    ws_n = max(K.linear_workspace_size(1, T, Hi * D, qr), K.linear_workspace_size(1, T, Hi, hid),
               K.linear_workspace_size(1, T, D, hid), K.linear_workspace_size(H, T, V, dn),
               K.linear_workspace_size(H, T, dv, V))
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device="cuda") if (ws_n and split) else None
    # name: (call, flops, algorithmic bytes = operands read once + output written once)
    calls = {
        "index_query": (lambda: K.linear(cq, w_q, q_idx, workspace=ws), 2 * T * Hi * D * qr,
                        2 * (T * qr + Hi * D * qr + T * Hi * D)),
        "head_weights": (lambda: K.linear(x, w_w, w, workspace=ws), 2 * T * Hi * hid, 2 * (T * hid + Hi * hid) + 4 * T * Hi),
        "key_gate": (lambda: (K.linear(x, w_kg[:D], keys, workspace=ws), K.linear(x, w_kg[D:], gates, workspace=ws)),
                     2 * T * 2 * D * hid,
                     2 * (2 * T * hid + 2 * D * hid + 2 * T * D)),
        "absorb": (lambda: K.mla_absorb_q(q_nope, w_uk_t, q, workspace=ws), 2 * T * H * V * dn,
                   2 * (T * H * dn + H * V * dn + T * H * V)),
        "unabsorb": (lambda: K.mla_unabsorb_o(o_lat, w_uv, o, workspace=ws), 2 * T * H * dv * V,
                     2 * (T * H * V + H * dv * V + T * H * dv)),
    }

    def timed(f):
        # `reps` calls captured in one HIP graph and replayed: a decode-sized product runs for less time than one
        # Python call takes to launch it, so timing eager calls would time the host
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / reps * 1e3  # us
    out = {"tokens": T, "calls": {}}
    for name, (f, fl, by) in calls.items():
        us = timed(f)
        out["calls"][name] = {"us": round(us, 2), "tflops": round(fl / (us * 1e-6) / 1e12, 2),
                              "gbs": round(by / (us * 1e-6) / 1e9, 1)}
    # as a layer step launches them: the four indexer products and the query absorb (all inputs ready before
    # attention) in one grouped launch, the un-absorb after attention on its own
    group = K.indexer_products(x, cq, w_q, w_w, w_kg, q_idx, w, keys, gates) + [K.absorb_product(q_nope, w_uk_t, q)]
    gws_n = K.linear_group_workspace_size(group)
    gws = torch.empty(max(gws_n, 16), dtype=torch.uint8, device="cuda") if (gws_n and split) else None
    f_group = lambda: K.linear_group(group, workspace=gws)  # noqa: E731
    us_g = timed(f_group)
    fl_g = sum(calls[c][1] for c in ("index_query", "head_weights", "key_gate", "absorb"))
    by_g = sum(calls[c][2] for c in ("index_query", "head_weights", "key_gate", "absorb"))
    out["calls"]["pre_attention_group"] = {"us": round(us_g, 2), "tflops": round(fl_g / (us_g * 1e-6) / 1e12, 2),
                                           "gbs": round(by_g / (us_g * 1e-6) / 1e9, 1)}
    f_un = calls["unabsorb"][0]
    us = timed(lambda: (f_group(), f_un()))
    fl = sum(c[1] for c in calls.values())
    by = sum(c[2] for c in calls.values())
    out.update(us=round(us, 2), flops=fl, bytes=by, tflops=round(fl / (us * 1e-6) / 1e12, 2),
               frac_of_bf16_peak=round(fl / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
               gbs=round(by / (us * 1e-6) / 1e9, 1), hbm_frac=round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
    del x, cq, w_q, w_w, w_kg, q_nope, w_uk_t, w_uv, o_lat, q_idx, w, keys, gates, q, o, ws, gws, group
    torch.cuda.empty_cache()
    return out



# ----------------------------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="decode,ceiling,32k,128k,long1m,fp8,mtp,prefill,proj,copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=16)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the KPool-DSA layer here is a single-GPU kernel path with no "
              "collectives; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import kpool_synth as ks
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    legs = set(args.legs.split(","))
    W = ks.workloads()
    res = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded generator; integer index data, N(0,1) "
                                                            "latents rounded to bf16)"}
    wl = W["batch64"]
    if "decode" in legs:
        print("[bench] decode leg: 64 sequences, contexts up to 128K", file=sys.stderr, flush=True)
        leg = Leg(wl, copies=2)
        te = leg.time_steps(args.steps, args.warmup)
        t = leg.time_steps_graph(args.steps, args.warmup)
        ms = t["mean"]
        st = leg.time_stages(args.steps)
        by = fused_stage_bytes(decode_bytes(wl))
        tot = sum(by.values())
        res.update(value=round(wl.n_q / (ms * 1e-3), 1), ms_per_step=round(ms, 5))
        res["ms_per_step_median"], res["ms_per_step_min"] = round(t["median"], 5), round(t["min"], 5)
        res["launch"] = "the timed steps captured in one HIP graph, replayed"
        res["eager"] = eager_stats(te, wl.n_q)
        res["hbm_gbs"] = round(tot / (ms * 1e-3) / 1e9, 1)
        res["hbm_frac"] = round(res["hbm_gbs"] / HBM_PEAK_GBS, 4)
        res["stages_ms"] = {k: round(v, 5) for k, v in st.items()}
        res["stage_bytes"] = by
        res["roofline"] = roofline(st, by)
        meas = [measured_traffic(k) for k in STAGE_KERNELS]
        # the step's HBM bytes as the counters measured them (profiles/), over the same step time; None once any of
        # the step's kernels changed since the counters were taken
        res["hbm_gbs_measured"] = (round(sum(meas) / (ms * 1e-3) / 1e9, 1) if all(m is not None for m in meas)
                                   else None)
        if "ceiling" in legs:
            # what HBM delivers for the step's own access patterns, read-only, nothing else running: the
            # attended tokens' value rows and the scanned pooled-key pages
            print("[bench] ceiling leg: read-only gathers of the decode step's own rows", file=sys.stderr, flush=True)
            ca, cs = leg.time_read_rows("attend"), leg.time_read_rows("score")
            res["ceiling"] = {"attend_rows": ca, "score_pages": cs,
                              "attend_stage_vs_ceiling": round(ca["ms"] / st["attend"], 4),
                              "score_stage_vs_ceiling": round(cs["ms"] / st["score"], 4),
                              "step_at_ceiling_ms": round(ca["ms"] + cs["ms"], 5),
                              "step_frac_at_ceiling": round(tot / ((ca["ms"] + cs["ms"]) * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                            4)}
        leg.free()
    res["config"] = {"workload": "batch64-decode-128k: 64 sequences, context U[8192,131072] seed 3 (sum 4,151,643),"
                                 " paged 64-token pages in a seeded random order, full layer dims",
                     "global_batch": wl.n_q, "seq_len": int(max(wl.ctx)), "parallelism": "none (1 GPU)",
                     "index_heads": wl.Hi, "index_dim": wl.D, "pool": wl.P, "topk": wl.k, "mla_heads": wl.H,
                     "latent": wl.L}

    def single(name, key, copies):
        w1 = W[name]
        leg = Leg(w1, copies=copies)
        n = max(args.steps, 50)
        te = leg.time_steps(n, args.warmup)
        t = leg.time_steps_graph(n, args.warmup)
        ms = t["mean"]
        st = leg.time_stages(n)
        by = fused_stage_bytes(decode_bytes(w1))
        gbs = sum(by.values()) / (ms * 1e-3) / 1e9
        res[key] = {"tokens_per_s": round(1 / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                    "ms_per_step_median": round(t["median"], 5), "ms_per_step_min": round(t["min"], 5),
                    "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "stages_ms": {k: round(v, 5) for k, v in st.items()}, "bytes": int(sum(by.values())),
                    "eager": eager_stats(te, 1)}
        leg.free()
    if "32k" in legs:
        print("[bench] 32k leg: one sequence at context 32768", file=sys.stderr, flush=True)
        single("decode32k", "decode32k", 40)
    if "128k" in legs:
        print("[bench] 128k leg: one sequence at context 131072", file=sys.stderr, flush=True)
        single("decode128k", "decode128k", 40)
    if "long1m" in legs:
        print("[bench] long1m leg: 8 sequences at context 1048576", file=sys.stderr, flush=True)
        w5 = W["long1m"]
        leg = Leg(w5, copies=2)
        te = leg.time_steps(args.steps, args.warmup)
        t = leg.time_steps_graph(args.steps, args.warmup)
        ms = t["mean"]
        st = leg.time_stages(args.steps)
        by = fused_stage_bytes(decode_bytes(w5))
        gbs = sum(by.values()) / (ms * 1e-3) / 1e9
        res["long1m"] = {"tokens_per_s": round(w5.n_q / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                         "ms_per_step_median": round(t["median"], 5), "ms_per_step_min": round(t["min"], 5),
                         "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "stages_ms": {k: round(v, 5) for k, v in st.items()}, "stage_bytes": by,
                         "eager": eager_stats(te, w5.n_q)}
        if "ceiling" in legs:
            ca, cs = leg.time_read_rows("attend"), leg.time_read_rows("score")
            res["long1m"]["ceiling"] = {"attend_rows": ca, "score_pages": cs,
                                        "step_frac_at_ceiling": round(sum(by.values()) / ((ca["ms"] + cs["ms"]) * 1e-3)
                                                                      / 1e9 / HBM_PEAK_GBS, 4)}
        leg.free()
    if "mtp" in legs:
        print("[bench] mtp leg: 32 targets at T-2 and their drafts at T-1, one selection per pair", file=sys.stderr,
              flush=True)
        res["mtp_verify"] = mtp_leg(W, args.steps)
    if "fp8" in legs:
        print("[bench] fp8 leg: the 64-sequence decode over an fp8 (E4M3) latent cache", file=sys.stderr, flush=True)
        w8 = W["batch64_fp8"]
        leg = Leg(w8, copies=2)
        te = leg.time_steps(args.steps, args.warmup)
        t = leg.time_steps_graph(args.steps, args.warmup)
        ms = t["mean"]
        st = leg.time_stages(args.steps)
        by = fused_stage_bytes(decode_bytes(w8))
        gbs = sum(by.values()) / (ms * 1e-3) / 1e9
        res["decode_fp8_latent"] = {"tokens_per_s": round(w8.n_q / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                                    "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                    "kv_scale": w8.kv_scale, "stages_ms": {k: round(v, 5) for k, v in st.items()},
                                    "stage_bytes": by, "eager": eager_stats(te, w8.n_q)}
        leg.free()
    if "prefill" in legs:
        print("[bench] prefill leg: 4096 queries on 65536 tokens", file=sys.stderr, flush=True)
        wp = W["prefill64k"]
        leg = Leg(wp, copies=1)
        ms = leg.time_steps(max(3, args.steps // 4), 2)["mean"]
        st = leg.time_stages(max(3, args.steps // 4), split_compress=True)
        fl = prefill_flops(wp)
        tf = fl / (st["score"] * 1e-3) / 1e12
        res["prefill_indexer"] = {"tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                                  "ms": round(st["score"], 4), "flops": fl, "step_ms": round(ms, 4),
                                  "stages_ms": {k: round(v, 4) for k, v in st.items()}}
        # the prefill attention: 2 H (V + V) flop per (query, attended token), tokens counted from the step's own
        # selection (each selected pool cut at the query)
        L = leg.layer
        sel = L.sel[:wp.n_q].long()
        pos = leg.d.q_pos.long()[:, None]
        nt = torch.clamp(pos - wp.P * sel + 1, 0, wp.P) * (sel >= 0)
        pairs = int(nt.sum().item())
        afl = 2 * wp.H * 2 * wp.V * pairs
        atf = afl / (st["attend"] * 1e-3) / 1e12
        res["prefill_attention"] = {"tflops": round(atf, 2), "frac_of_bf16_peak": round(atf / BF16_PEAK_TFLOPS, 4),
                                    "ms": round(st["attend"], 4), "flops": afl, "query_token_pairs": pairs}
        leg.free()
    if "proj" in legs:
        print("[bench] proj leg: the five projections at 64 tokens (decode) and 4096 tokens (prefill)",
              file=sys.stderr, flush=True)
        res["projections"] = {"decode64": proj_leg(64, 200), "prefill4096": proj_leg(4096, 20)}
    if "copy" in legs:
        print("[bench] copy leg: 1 GiB device copy", file=sys.stderr, flush=True)
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res["copy"] = {"bytes_moved": 2 * 4 * n, "ms": round(ms, 4),
                       "gbs": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1)}
        if res.get("hbm_gbs"):   # the decode step against what a plain copy reaches on this machine
            res["hbm_frac_of_copy"] = round(res["hbm_gbs"] / res["copy"]["gbs"], 4)
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
