"""Test-only glue: builds a workload's inputs on the device through the seeded generator, runs the layer through
the C ABI, and recomputes sampled queries with the CPU oracle from host-regenerated inputs.

Nothing here is imported by the product path."""
from __future__ import annotations

import numpy as np
import torch

import kpool_synth as ks
import oracle as O
import sparse_attention_kpool_amd as K
from sparse_attention_kpool_amd.layer import CompressInput, KPoolDSALayer


# Guard bands: every output buffer of a parity run sits inside a larger allocation filled with a sentinel; after the
# run, the words before and after it must be untouched (a kernel writing out of bounds fails the test).
GUARD_ELEMS = 256
SENTINEL = {torch.float32: 0x7FC0DEAD, torch.int32: 0x5A5A5A5A, torch.bfloat16: 0x7FC1}


class Guarded:
    """A tensor of `shape` placed GUARD_ELEMS elements into a sentinel-filled buffer of GUARD_ELEMS extra elements on
    each side."""

    def __init__(self, shape, dtype, device):
        n = 1
        for e in shape:
            n *= int(e)
        self.n, self.dtype = n, dtype
        raw = torch.empty(n + 2 * GUARD_ELEMS, dtype=dtype, device=device)
        self._bits(raw).fill_(SENTINEL[dtype])
        self.raw = raw
        self.t = raw[GUARD_ELEMS:GUARD_ELEMS + n].view(*shape)

    @staticmethod
    def _bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)

    def intact(self) -> bool:
        b = self._bits(self.raw)
        pre, post = b[:GUARD_ELEMS], b[GUARD_ELEMS + self.n:]
        ref = SENTINEL[self.dtype]
        if self.dtype == torch.bfloat16:
            ref = ref - (1 << 16) if ref >= (1 << 15) else ref
        return bool((pre == ref).all().item() and (post == ref).all().item())


def dims_of(wl: ks.Workload) -> K.Dims:
    return K.Dims(pool=wl.P, idx_dim=wl.D, idx_heads=wl.Hi, topk=wl.k, heads=wl.H, latent_dim=wl.L, v_dim=wl.V,
                  page_tokens=wl.page_tokens, dtype=wl.dtype, scale=wl.scale)


class DeviceRun:
    """Device-side inputs of one workload (from the seeded generator) plus the layer's outputs after `run()`."""

    def __init__(self, wl: ks.Workload, device="cuda", group=None):
        self.wl = wl
        self.dev = torch.device(device)
        self.dims = dims_of(wl)
        d = ks.DeviceInputs(wl, self.dev)
        self.inputs = d
        self.bt_np = d.block_table_np
        self.latent, self.pooled = d.latent, d.pooled
        self.cache = K.Cache(latent=d.latent, pooled=d.pooled, block_table=d.block_table, latent_scale=wl.kv_scale)
        if group is None:
            group = wl.n_q if len(set(wl.q_seq.tolist())) == 1 else 1
        self.queries = K.Queries(seq=d.q_seq, pos=d.q_pos, max_pos=wl.max_pos(), group=group)
        self.q_idx, self.w, self.q = d.q_idx, d.w, d.q
        self.cpools = d.cpools
        self.compress = None if d.c_keys is None else CompressInput(
            keys=d.c_keys, gates=d.c_gates, ape=d.ape, pool_seq=d.c_seq, pool_id=d.c_pool)
        self.layer = KPoolDSALayer(self.dims, self.dev, max_q=wl.n_q, max_pos=max(wl.max_pos(), 0))
        tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        # every output the step writes sits between guard bands; the layer's own intermediates are swapped for
        # guarded ones of the same shape, and the score rows start out as the sentinel, so columns a query cannot
        # see (p >= n_c) are checked to stay unwritten
        L = self.layer
        self.guards = {
            "scores": Guarded(tuple(L.scores.shape), torch.float32, self.dev),
            "sel": Guarded(tuple(L.sel.shape), torch.int32, self.dev),
            "n_sel": Guarded(tuple(L.n_sel.shape), torch.int32, self.dev),
            "out": Guarded((wl.n_q, wl.H, wl.V), tdt, self.dev),
            "lse": Guarded((wl.n_q, wl.H), torch.float32, self.dev),
        }
        L.scores, L.sel, L.n_sel = self.guards["scores"].t, self.guards["sel"].t, self.guards["n_sel"].t
        self.out, self.lse = self.guards["out"].t, self.guards["lse"].t

    def run(self):
        self.layer.step(self.cache, self.queries, self.q_idx, self.w, self.q, self.out, lse=self.lse,
                        compress=self.compress)
        torch.cuda.synchronize()
        return self

    def check_guards(self):
        """Every guard band intact, and no score written at or past a query's visible complete pools."""
        for name, g in self.guards.items():
            assert g.intact(), f"{name}: a kernel wrote outside the buffer"
        wl = self.wl
        n_c = torch.from_numpy(((wl.q_pos.astype(np.int64) + 1) // wl.P)).to(self.dev)
        sc = self.layer.scores[:wl.n_q].view(torch.int32)
        col = torch.arange(sc.shape[1], device=self.dev)[None, :]
        tail = col >= n_c[:, None]
        assert bool((sc[tail] == SENTINEL[torch.float32]).all().item()), "a score was written past n_c"

    # ---- host copies of what the device produced -----------------------------------------------------
    def pooled_rows(self, s: int, pools) -> np.ndarray:
        wl = self.wl
        ppp = wl.page_tokens // wl.P
        pools = np.asarray(pools, dtype=np.int64)
        pages = torch.from_numpy(self.bt_np[s, pools // ppp].astype(np.int64)).to(self.dev)
        slots = torch.from_numpy(pools % ppp).to(self.dev)
        return self.pooled[pages, slots].float().cpu().numpy().astype(np.float64)

    def scores_row(self, j: int, n_c: int) -> np.ndarray:
        return self.layer.scores[j, :n_c].cpu().numpy().astype(np.float64)

    def sel_row(self, j: int):
        ns = int(self.layer.n_sel[j].item())
        return self.layer.sel[j].cpu().numpy(), ns


# ----------------------------------------------------------------------------------------------------------
# oracle side (host regeneration)
# ----------------------------------------------------------------------------------------------------------
def oracle_pooled(wl: ks.Workload, s: int, n_c: int) -> np.ndarray:
    """Pooled keys of sequence s, pools < n_c, as the cache holds them after the step (storage precision)."""
    P, D = wl.P, wl.D
    out = np.zeros((n_c, D), dtype=np.float64)
    first_new = wl.new_from[s] // P
    old = min(first_new, n_c)
    if old:
        out[:old] = ks.host_pool_keys(wl, s, np.arange(old))        # pre-filled constant-key pools
    if n_c > old:
        toks = np.arange(old * P, n_c * P)
        keys = ks.host_token_keys(wl, s, toks).reshape(-1, P, D)
        gates = ks.host_gates(wl, s, toks).reshape(-1, P, D)
        out[old:] = O.store_round(O.pool_compress(keys, gates, ks.host_ape(wl)), wl.dtype)
    return out


def oracle_query(wl: ks.Workload, j: int, pooled=None, sel=None):
    """Oracle result for query j.  `pooled` / `sel` override the oracle's own stage outputs (stage parity)."""
    s, i = int(wl.q_seq[j]), int(wl.q_pos[j])
    n_c, r, tau = O.pool_geometry(i, wl.P)
    if pooled is None:
        pooled = oracle_pooled(wl, s, n_c)
    qidx = ks.host_qidx(wl, s, i)[0]
    w = ks.host_w(wl, s, i)[0]
    scores = O.indexer_scores(qidx, w, pooled, n_c)
    own_sel = O.select_pools(scores, i, wl.P, wl.k)
    use_sel = own_sel if sel is None else sel
    toks = O.attended_tokens(use_sel, i, wl.P)
    q = ks.host_q(wl, s, i)[0]
    if wl.latent_fp8:   # the cache holds E4M3 codes; a row's values are the decoded codes times the cache scale
        rows = O.fp8_e4m3_decode(ks.host_latent_codes(wl, s, toks)) * wl.kv_scale
    else:
        rows = ks.host_latent(wl, s, toks)
    out, lse = O.sparse_mla(q, rows, wl.scale, wl.V)
    return dict(scores=scores, sel=own_sel, tokens=toks, out=out, lse=lse, n_c=n_c, r=r, tau=tau)


def attn_tolerance(dtype: str):
    """(max-abs, rel-RMS) bounds for the attention output."""
    return (3e-2, 1e-2) if dtype == "bf16" else (1e-4, 1e-5)


def rel_rms(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.sqrt(((a - b) ** 2).sum()) / max(np.sqrt((b ** 2).sum()), 1e-30))
