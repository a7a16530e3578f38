#!/usr/bin/env python3
"""Benchmark of the KPool-DSA layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--legs decode,128k,long1m,prefill]

A step is one pass of the whole layer -- kpool_compress (pools completing this step) -> dsa_indexer_score ->
dsa_topk_select -> sparse_mla_attn -- over one batch, enqueued on one stream through the C ABI.

Legs (inputs are seeded synthetic data already resident in HBM when timing starts):
  decode   the headline: 64 sequences, contexts U[8192, 131072] (seed 3, up to 128K), paged 64-token pages,
           full layer dims (index 32 x 128, pool 4, top-k 2048, 64 MLA heads on a 576 latent), bf16.
           `value` = decode tokens/s = 64 / step time.  Two copies of the caches alternate between steps so the
           256 MB Infinity Cache cannot serve one step from the previous one.
  128k     one sequence at context 131,072 (the exact 128K point), rotating 40 cache copies.
  prefill  4096 new queries on 65,536 tokens: the indexer's TFLOP/s against the bf16 MFMA peak, and the
           whole prefill step.
  copy     a plain 1 GiB device-to-device copy: the achievable-bandwidth reference, and the kernel of known
           traffic against which the FETCH_SIZE / WRITE_SIZE counters are scaled.
Rank 0 prints one JSON line.  Algorithmic bytes/flops count what the method must move or compute; the
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
    Score rows and split-KV partials are intermediate traffic, not algorithmic."""
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

    def time_steps(self, steps: int, warmup: int) -> float:
        """Mean ms per step over `steps` back-to-back steps (HIP events on the launch stream)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            self.step(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_steps_graph(self, steps: int) -> float:
        """Mean ms per step with `steps` steps captured in one HIP graph and replayed: the GPU time of a step whose
        kernels finish faster than Python can enqueue them (a single query)."""
        torch = self.torch
        for i in range(3):
            self.step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                self.step(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / steps

    def time_stages(self, steps: int) -> dict:
        """Mean ms per stage, events recorded between the four calls on the launch stream."""
        torch, K, L = self.torch, self.K, self.layer
        n_q = self.wl.n_q
        names = ["compress", "score", "topk", "attend"]
        acc = dict.fromkeys(names, 0.0)
        for i in range(steps):
            cache = self.caches[i % len(self.caches)]
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record()
            c = self.compress
            if c is not None:
                K.kpool_compress(self.dims, cache, c.keys, c.gates, c.ape, c.pool_seq, c.pool_id, src=c.src)
            ev[1].record()
            K.dsa_indexer_score(self.dims, cache, self.queries, self.d.q_idx, self.d.w, L.scores[:n_q])
            ev[2].record()
            K.dsa_topk_select(self.dims, self.queries, L.scores[:n_q], L.sel[:n_q], L.n_sel[:n_q],
                              workspace=L.ws_topk)
            ev[3].record()
            if cache.latent.dtype == torch.uint8:
                K.sparse_mla_attn_fp8(self.dims, cache, self.queries, self.d.q, L.sel[:n_q], L.n_sel[:n_q],
                                      cache.latent_scale, self.out, lse=self.lse, workspace=L.ws_attn)
            else:
                K.sparse_mla_attn(self.dims, cache, self.queries, self.d.q, L.sel[:n_q], L.n_sel[:n_q], self.out,
                                  lse=self.lse, workspace=L.ws_attn)
            ev[4].record()
            torch.cuda.synchronize()
            for j, n in enumerate(names):
                acc[n] += ev[j].elapsed_time(ev[j + 1])
        return {n: acc[n] / steps for n in names}

    def free(self):
        del self.caches, self.layer, self.d
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


STAGE_KERNELS = {"score": ["kp::score_decode_kernel<kp::bf16, 128>"],
                 "attend": ["kp::attn_dma_kernel<4, false>", "kp::attn_combine_kernel<kp::bf16, 8>"]}


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
            cur = hashlib.sha256(open(os.path.join(ROOT, e["source"]), "rb").read()).hexdigest()[:16]
            if cur != e["sha256_16"]:
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
def cpu_baseline(wl, n_sample: int, min_seconds: float = 10.0) -> dict:
    import kpool_synth as ks
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS thread count is not reported
        threads = os.cpu_count() or 1
    ape = ks.host_ape(wl).astype(np.float64)
    prepared = []
    for j in range(n_sample):                                   # host inputs, outside the timed region
        s, i = int(wl.q_seq[j]), int(wl.q_pos[j])
        n_c, r, tau = O.pool_geometry(i, wl.P)
        pre = ks.host_pool_keys(wl, s, np.arange(n_c)).astype(np.float64)
        comp = None
        if wl.ctx[s] % wl.P == 0:                               # this step completes pool n_c - 1
            toks = np.arange((n_c - 1) * wl.P, n_c * wl.P)
            comp = (ks.host_token_keys(wl, s, toks)[None].astype(np.float64),
                    ks.host_gates(wl, s, toks)[None].astype(np.float64))
        qidx = ks.host_qidx(wl, s, i)[0].astype(np.float64)
        w = ks.host_w(wl, s, i)[0].astype(np.float64)
        q = ks.host_q(wl, s, i)[0].astype(np.float64)
        # regenerate only the latent rows this query attends (found by an untimed selection pass); the timed
        # pass below redoes the whole layer and gathers its rows through the token -> row map
        sel0 = O.select_pools(O.indexer_scores(qidx, w, pre, n_c), i, wl.P, wl.k)
        toks0 = O.attended_tokens(sel0, i, wl.P)
        rows = ks.host_latent(wl, s, toks0).astype(np.float64)
        tmap = np.full(i + 1, -1, dtype=np.int64)
        tmap[toks0] = np.arange(len(toks0))
        prepared.append((i, pre, comp, qidx, w, q, rows, tmap))
    t0 = time.perf_counter()
    reps = 0
    while True:                                                 # repeat the sample to >= min_seconds of work
        for (i, pre, comp, qidx, w, q, rows, tmap) in prepared:
            n_c = (i + 1) // wl.P
            pooled = pre
            if comp is not None:
                pooled = pre.copy()
                pooled[n_c - 1] = O.store_round(O.pool_compress(comp[0], comp[1], ape), wl.dtype)[0]
            s_ = O.indexer_scores(qidx, w, pooled, n_c)
            sel = O.select_pools(s_, i, wl.P, wl.k)
            toks = O.attended_tokens(sel, i, wl.P)
            O.sparse_mla(q, rows[tmap[toks]], wl.scale, wl.V)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(reps * n_sample / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{n_sample} of the 64 decode queries (sequences 0..{n_sample - 1}) x {reps} passes, the whole "
                      f"layer per query (pool, score, select, attend) in float64 numpy; host input regeneration "
                      f"not timed"}

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
    ap.add_argument("--legs", default="decode,128k,long1m,fp8,prefill,proj,copy")
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
        ms = leg.time_steps(args.steps, args.warmup)
        st = leg.time_stages(args.steps)
        by = decode_bytes(wl)
        tot = sum(by.values())
        res.update(value=round(wl.n_q / (ms * 1e-3), 1), ms_per_step=round(ms, 5))
        res["hbm_gbs"] = round(tot / (ms * 1e-3) / 1e9, 1)
        res["hbm_frac"] = round(res["hbm_gbs"] / HBM_PEAK_GBS, 4)
        res["stages_ms"] = {k: round(v, 5) for k, v in st.items()}
        res["stage_bytes"] = by
        res["roofline"] = roofline(st, by)
        leg.free()
    res["config"] = {"workload": "batch64-decode-128k: 64 sequences, context U[8192,131072] seed 3 (sum 4,151,643),"
                                 " paged 64-token pages in a seeded random order, full layer dims",
                     "global_batch": wl.n_q, "seq_len": int(max(wl.ctx)), "parallelism": "none (1 GPU)",
                     "index_heads": wl.Hi, "index_dim": wl.D, "pool": wl.P, "topk": wl.k, "mla_heads": wl.H,
                     "latent": wl.L}
    if "128k" in legs:
        print("[bench] 128k leg: one sequence at context 131072", file=sys.stderr, flush=True)
        w1 = W["decode128k"]
        leg = Leg(w1, copies=40)
        ms = leg.time_steps(max(args.steps, 50), args.warmup)
        st = leg.time_stages(max(args.steps, 50))
        by = decode_bytes(w1)
        msg = leg.time_steps_graph(max(args.steps, 50))
        res["decode128k"] = {"tokens_per_s": round(1 / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                             "hbm_gbs": round(sum(by.values()) / (ms * 1e-3) / 1e9, 1),
                             "stages_ms": {k: round(v, 5) for k, v in st.items()},
                             "graph": {"ms_per_step": round(msg, 5), "tokens_per_s": round(1 / (msg * 1e-3), 1),
                                       "hbm_gbs": round(sum(by.values()) / (msg * 1e-3) / 1e9, 1)}}
        leg.free()
    if "long1m" in legs:
        print("[bench] long1m leg: 8 sequences at context 1048576", file=sys.stderr, flush=True)
        w5 = W["long1m"]
        leg = Leg(w5, copies=2)
        ms = leg.time_steps(args.steps, args.warmup)
        st = leg.time_stages(args.steps)
        by = decode_bytes(w5)
        gbs = sum(by.values()) / (ms * 1e-3) / 1e9
        res["long1m"] = {"tokens_per_s": round(w5.n_q / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                         "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "stages_ms": {k: round(v, 5) for k, v in st.items()}, "stage_bytes": by}
        leg.free()
    if "fp8" in legs:
        print("[bench] fp8 leg: the 64-sequence decode over an fp8 (E4M3) latent cache", file=sys.stderr, flush=True)
        w8 = W["batch64_fp8"]
        leg = Leg(w8, copies=2)
        ms = leg.time_steps(args.steps, args.warmup)
        st = leg.time_stages(args.steps)
        by = decode_bytes(w8)
        gbs = sum(by.values()) / (ms * 1e-3) / 1e9
        res["decode_fp8_latent"] = {"tokens_per_s": round(w8.n_q / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                                    "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                    "kv_scale": w8.kv_scale, "stages_ms": {k: round(v, 5) for k, v in st.items()},
                                    "stage_bytes": by}
        leg.free()
    if "prefill" in legs:
        print("[bench] prefill leg: 4096 queries on 65536 tokens", file=sys.stderr, flush=True)
        wp = W["prefill64k"]
        leg = Leg(wp, copies=1)
        ms = leg.time_steps(max(3, args.steps // 4), 2)
        st = leg.time_stages(max(3, args.steps // 4))
        fl = prefill_flops(wp)
        tf = fl / (st["score"] * 1e-3) / 1e12
        res["prefill_indexer"] = {"tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                                  "ms": round(st["score"], 4), "flops": fl, "step_ms": round(ms, 4),
                                  "stages_ms": {k: round(v, 4) for k, v in st.items()}}
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
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
