"""Seeded synthetic inputs for the KPool-DSA sparse-attention layer.

Test and benchmark infrastructure, shared by the oracle side and the device side.  It holds none of the layer's
arithmetic: it only decides which input values exist.

Every value is a pure function of (workload seed, stream name, logical index).  The hash is integer-only
(Wellons' "lowbias32" 32-bit mixer, applied twice over the low and high halves of a 64-bit counter), so the
same function evaluated with numpy on the host and with torch integer ops on the device gives bit-identical
values.  That lets a test regenerate, on the host, exactly the rows an oracle check needs (one sequence's pooled
keys, the selected latent rows) while the device fills multi-gigabyte paged caches in place.

Value recipes (the workload shapes come from the layer's published configuration; see ``workloads``):
  * small integers U{lo..hi}: ``(h * n) >> 32`` with n = hi - lo + 1;
  * N(0, 1): a 65536-entry table of normal quantiles at (j + 1/2) / 65536, rounded once to the storage dtype
    (bf16 round-to-nearest-even, or fp32), indexed by the top 16 hash bits;
  * U(0,1) head weights on a 2^-8 grid: U{0..255} / 256 (exact in bf16 and fp32).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

M32 = 0xFFFFFFFF
TMAX = 1 << 21          # logical token stride per sequence in the counter (> 1,048,576 tokens)


# ----------------------------------------------------------------------------------------------------------
# integer hash, written once over a tiny backend shim so numpy and torch evaluate the same expression
# ----------------------------------------------------------------------------------------------------------
def _mulmod32(x, c: int):
    """(x * c) mod 2^32 for 0 <= x < 2^32 without ever leaving int64 range."""
    c_lo, c_hi = c & 0xFFFF, c >> 16
    return (x * c_lo + (((x * c_hi) & 0xFFFF) << 16)) & M32


def _mix32(x):
    x = x ^ (x >> 16)
    x = _mulmod32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mulmod32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def stream_key(seed: int, stream: str) -> int:
    """32-bit key for one named stream of one workload seed (host side, hashlib)."""
    d = hashlib.blake2b(f"{seed}:{stream}".encode(), digest_size=8).digest()
    return int.from_bytes(d, "little") & M32


def hash32(key: int, idx):
    """Hash of a non-negative int64 counter array (numpy int64 or torch int64); values in [0, 2^32)."""
    k1 = key
    k2 = _mix32_int(key ^ 0x9E3779B9)
    lo = idx & M32
    hi = idx >> 32
    h = _mix32(lo ^ k1)
    h = _mix32(h ^ hi ^ k2)
    return h


def _mix32_int(x: int) -> int:
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def uniform_int(key: int, idx, lo: int, hi: int):
    n = hi - lo + 1
    return ((hash32(key, idx) * n) >> 32) + lo


def _f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32)


_TABLES: dict = {}


def normal_table(dtype: str) -> np.ndarray:
    """65536 normal quantiles at (j + 1/2)/65536 rounded to ``dtype`` ('bf16' or 'f32'), as float32."""
    if dtype not in _TABLES:
        from scipy.special import ndtri
        q = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
        _TABLES[dtype] = _f32_to_bf16_rne(q) if dtype == "bf16" else q
    return _TABLES[dtype]


def fp8_codes(key: int, idx):
    """E4M3 codes from the hash: random sign, exponent field 4..7, random 3-bit mantissa -- magnitudes in
    [0.125, 1.875], never NaN.  uint8 numpy array, or an int64 torch tensor for a torch ``idx``."""
    h = hash32(key, idx)
    c = (((h >> 31) & 1) << 7) | ((4 + ((h >> 24) & 3)) << 3) | ((h >> 16) & 7)
    return c.astype(np.uint8) if isinstance(c, np.ndarray) else c


def normal(key: int, idx, dtype: str, table=None):
    """N(0,1) draws (numpy float32 on the host; pass ``table`` as a device tensor for torch)."""
    h = hash32(key, idx) >> 16
    if table is None:
        return normal_table(dtype)[h]
    return table[h]


def host_matrix(seed: int, name: str, shape, kind: str = "normal", scale: float = 1.0) -> np.ndarray:
    """Seeded float32 array of bf16 values for one named operand.  kind 'int': integers in [-4, 4] (exact in
    bf16, and any sum of up to 2^20 of their products is exact in fp32); 'normal': N(0, 1) draws times `scale`
    (a power of two keeps them bf16 values)."""
    key = stream_key(seed, "matrix:" + name)
    idx = np.arange(int(np.prod(shape)), dtype=np.int64)
    if kind == "int":
        v = uniform_int(key, idx, -4, 4).astype(np.float32)
    else:
        v = normal(key, idx, "bf16") * np.float32(scale)
    return v.reshape(shape)


# ----------------------------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------------------------
@dataclass
class Workload:
    """One synthetic workload of the layer.

    Sequences hold ``ctx[s]`` tokens in both caches after the step.  Queries are (seq, pos) pairs; a decode
    query sits at the last token, ``pos = ctx - 1``.  Tokens ``new_from[s] ... ctx[s]-1`` are new this step:
    their pools are compressed in-step when they complete; older pools are pre-filled in the pooled cache.
    """
    name: str
    dtype: str                       # 'f32' or 'bf16' storage dtype
    P: int                           # tokens per pool
    D: int                           # index head dim
    Hi: int                          # index heads
    k: int                           # top-k, in pools
    H: int                           # MLA heads
    L: int                           # latent row width
    V: int                           # value (nope) width; columns V..L-1 are zero
    scale: float                     # attention softmax scale
    page_tokens: int                 # tokens per page of both caches
    ctx: list                        # tokens per sequence after this step
    new_from: list                   # first new token per sequence
    q_seq: np.ndarray                # [n_q] int32
    q_pos: np.ndarray                # [n_q] int32
    seed: int = 0
    w_int: bool = False              # head weights U{-4..4} (tiny fp32 case) instead of U{0..255}/256
    latent_int: bool = False         # q and latents U{-4..4} instead of N(0,1)
    key_per_token: bool = False      # general instance: keys drawn per token (else constant per pool)
    page_perm_seed: Optional[int] = None   # None: pages placed in order; else a seeded random permutation
    w_scale: float = 1.0             # multiplies the head weights (0 makes every score 0: a pure tie-break case)
    latent_fp8: bool = False         # latent cache of OCP E4M3 codes (value = code value * kv_scale)
    kv_scale: float = 1.0            # scale of the fp8 latent cache
    extra: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return len(self.ctx)

    @property
    def n_q(self) -> int:
        return int(len(self.q_pos))

    def pages_per_seq(self) -> list:
        pt = self.page_tokens
        return [(t + pt - 1) // pt for t in self.ctx]

    def block_table(self) -> np.ndarray:
        """[B, max_pages] int32 physical page ids (-1 past a sequence's last page)."""
        pps = self.pages_per_seq()
        total = sum(pps)
        if self.page_perm_seed is None:
            phys = np.arange(total, dtype=np.int64)
        else:
            phys = np.random.default_rng(self.page_perm_seed).permutation(total)
        bt = np.full((self.B, max(pps)), -1, dtype=np.int32)
        o = 0
        for s, n in enumerate(pps):
            bt[s, :n] = phys[o:o + n]
            o += n
        return bt

    def n_pages(self) -> int:
        return sum(self.pages_per_seq())

    def max_pos(self) -> int:
        return int(self.q_pos.max()) if self.n_q else 0

    # ---- keys -----------------------------------------------------------------------------------------
    def key(self, stream: str) -> int:
        return stream_key(self.seed, stream)


def _decode(name, dtype, ctx, seed, **kw) -> Workload:
    ctx = [int(t) for t in ctx]
    full = dict(P=4, D=128, Hi=32, k=2048, H=64, L=576, V=512, scale=1.0 / 16.0, page_tokens=64)
    full.update(kw)
    return Workload(name=name, dtype=dtype, ctx=ctx, new_from=[t - 1 for t in ctx],
                    q_seq=np.arange(len(ctx), dtype=np.int32),
                    q_pos=np.array([t - 1 for t in ctx], dtype=np.int32), seed=seed, **full)


def cfg3_contexts() -> np.ndarray:
    """Per-sequence contexts of the batch-64 decode workload: U[8192, 131072], seed 3."""
    return np.random.default_rng(3).integers(8192, 131072, 64, endpoint=True)


def workloads() -> dict:
    """The five published workload shapes, plus the 128K single-sequence decode point and the batch-64 decode over
    an fp8 latent cache."""
    w = {}
    # tiny prefill, fp32: all 64 positions of one sequence are queries and all tokens are new
    w["tiny"] = Workload(name="tiny", dtype="f32", P=4, D=32, Hi=2, k=8, H=4, L=80, V=64, scale=1.0 / 8.0,
                         page_tokens=16, ctx=[64], new_from=[0], q_seq=np.zeros(64, np.int32),
                         q_pos=np.arange(64, dtype=np.int32), seed=1, w_int=True, latent_int=True,
                         page_perm_seed=11)
    w["decode32k"] = _decode("decode32k", "bf16", [32768], seed=2)
    w["decode128k"] = _decode("decode128k", "bf16", [131072], seed=22)
    w["batch64"] = _decode("batch64", "bf16", cfg3_contexts(), seed=3, page_perm_seed=33)
    w["prefill64k"] = Workload(name="prefill64k", dtype="bf16", P=4, D=128, Hi=32, k=2048, H=64, L=576, V=512,
                               scale=1.0 / 16.0, page_tokens=64, ctx=[65536], new_from=[61440],
                               q_seq=np.zeros(4096, np.int32), q_pos=np.arange(61440, 65536, dtype=np.int32),
                               seed=4)
    w["long1m"] = _decode("long1m", "bf16", [1 << 20] * 8, seed=5, page_perm_seed=55)
    # the batch-64 decode over an fp8 (E4M3) latent cache with scale 1/2
    w["batch64_fp8"] = scaled(w["batch64"], name="batch64_fp8", latent_fp8=True, kv_scale=0.5)
    return w


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of ``wl`` with fields replaced (e.g. smaller contexts for a quick parity case)."""
    import dataclasses
    return dataclasses.replace(wl, **changes)


# ----------------------------------------------------------------------------------------------------------
# host (numpy) generation of logical arrays
# ----------------------------------------------------------------------------------------------------------
def _seqtok(seq, tok):
    return np.asarray(seq, dtype=np.int64) * TMAX + np.asarray(tok, dtype=np.int64)


def host_pool_keys(wl: Workload, seq: int, pools: np.ndarray) -> np.ndarray:
    """Per-pool integer keys [len(pools), D] (the constant-per-pool parity instance)."""
    idx = _seqtok(seq, pools)[:, None] * wl.D + np.arange(wl.D, dtype=np.int64)[None, :]
    return uniform_int(wl.key("kpool"), idx, -4, 4).astype(np.float32)


def host_token_keys(wl: Workload, seq: int, toks: np.ndarray) -> np.ndarray:
    """Per-token index keys [len(toks), D]."""
    toks = np.asarray(toks, dtype=np.int64)
    if not wl.key_per_token:
        return host_pool_keys(wl, seq, toks // wl.P)
    idx = _seqtok(seq, toks)[:, None] * wl.D + np.arange(wl.D, dtype=np.int64)[None, :]
    return uniform_int(wl.key("ktok"), idx, -4, 4).astype(np.float32)


def host_gates(wl: Workload, seq: int, toks: np.ndarray) -> np.ndarray:
    idx = _seqtok(seq, toks)[:, None] * wl.D + np.arange(wl.D, dtype=np.int64)[None, :]
    return normal(wl.key("gate"), idx, wl.dtype)


def host_ape(wl: Workload) -> np.ndarray:
    idx = np.arange(wl.P * wl.D, dtype=np.int64).reshape(wl.P, wl.D)
    return normal(wl.key("ape"), idx, wl.dtype)


def host_qidx(wl: Workload, seq, pos) -> np.ndarray:
    """Index queries [n, Hi, D] for queries (seq[j], pos[j])."""
    st = _seqtok(seq, pos).reshape(-1)
    idx = (st[:, None, None] * wl.Hi + np.arange(wl.Hi)[None, :, None]) * wl.D + np.arange(wl.D)[None, None, :]
    return uniform_int(wl.key("qidx"), idx, -4, 4).astype(np.float32)


def host_w(wl: Workload, seq, pos) -> np.ndarray:
    st = _seqtok(seq, pos).reshape(-1)
    idx = st[:, None] * wl.Hi + np.arange(wl.Hi)[None, :]
    if wl.w_int:
        w = uniform_int(wl.key("w"), idx, -4, 4).astype(np.float32)
    else:
        w = (uniform_int(wl.key("w"), idx, 0, 255).astype(np.float32) / 256.0).astype(np.float32)
    return (w * np.float32(wl.w_scale)).astype(np.float32)


def host_q(wl: Workload, seq, pos) -> np.ndarray:
    """MLA queries [n, H, L]; columns V..L-1 are zero."""
    st = _seqtok(seq, pos).reshape(-1)
    idx = (st[:, None, None] * wl.H + np.arange(wl.H)[None, :, None]) * wl.L + np.arange(wl.L)[None, None, :]
    if wl.latent_int:
        v = uniform_int(wl.key("q"), idx, -4, 4).astype(np.float32)
    else:
        v = normal(wl.key("q"), idx, wl.dtype)
    v[..., wl.V:] = 0.0
    return v


def host_latent_codes(wl: Workload, seq: int, toks: np.ndarray) -> np.ndarray:
    """Fp8 latent rows [len(toks), L] as E4M3 codes (uint8); columns V..L-1 hold code 0."""
    idx = _seqtok(seq, toks)[:, None] * wl.L + np.arange(wl.L, dtype=np.int64)[None, :]
    c = fp8_codes(wl.key("lat8"), idx)
    c[:, wl.V:] = 0
    return c


def host_latent(wl: Workload, seq: int, toks: np.ndarray) -> np.ndarray:
    """Latent rows [len(toks), L]; columns V..L-1 are zero."""
    idx = _seqtok(seq, toks)[:, None] * wl.L + np.arange(wl.L, dtype=np.int64)[None, :]
    if wl.latent_int:
        v = uniform_int(wl.key("lat"), idx, -4, 4).astype(np.float32)
    else:
        v = normal(wl.key("lat"), idx, wl.dtype)
    v[:, wl.V:] = 0.0
    return v


# ----------------------------------------------------------------------------------------------------------
# device (torch) generation straight into the physical paged layout
# ----------------------------------------------------------------------------------------------------------
def _torch_dtype(wl: Workload):
    import torch
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def page_owner(wl: Workload):
    """(seq, logical page) of every physical page, as int64 numpy arrays of length n_pages."""
    bt = wl.block_table()
    n = wl.n_pages()
    seq = np.zeros(n, np.int64)
    lpg = np.zeros(n, np.int64)
    for s, npg in enumerate(wl.pages_per_seq()):
        seq[bt[s, :npg]] = s
        lpg[bt[s, :npg]] = np.arange(npg)
    return seq, lpg


def device_caches(wl: Workload, device, chunk_pages: int = 1024):
    """Fill the paged latent cache [n_pages, page_tokens, L] and the pooled-key cache
    [n_pages, page_tokens / P, D] on ``device``.  Pooled rows of pools that complete before ``new_from`` hold the
    constant-per-pool integer keys (what compression yields on such pools); rows of newer pools are zero and get
    written by compression in-step."""
    import torch
    dt = _torch_dtype(wl)
    seq_np, lpg_np = page_owner(wl)
    n_pages, pt, P = wl.n_pages(), wl.page_tokens, wl.P
    ppp = pt // P
    latent = torch.empty((n_pages, pt, wl.L), dtype=torch.uint8 if wl.latent_fp8 else dt, device=device)
    pooled = torch.zeros((n_pages, ppp, wl.D), dtype=dt, device=device)
    table = torch.from_numpy(normal_table(wl.dtype)).to(device)
    seq_t = torch.from_numpy(seq_np).to(device)
    lpg_t = torch.from_numpy(lpg_np).to(device)
    first_new_pool = torch.tensor([nf // P for nf in wl.new_from], dtype=torch.int64, device=device)
    klat, kpool = wl.key("lat"), wl.key("kpool")
    colL = torch.arange(wl.L, dtype=torch.int64, device=device)
    colD = torch.arange(wl.D, dtype=torch.int64, device=device)
    tok_in_page = torch.arange(pt, dtype=torch.int64, device=device)
    pool_in_page = torch.arange(ppp, dtype=torch.int64, device=device)
    for p0 in range(0, n_pages, chunk_pages):
        p1 = min(n_pages, p0 + chunk_pages)
        s = seq_t[p0:p1]
        tok = lpg_t[p0:p1, None] * pt + tok_in_page[None, :]                       # [c, pt]
        idx = ((s[:, None] * TMAX + tok)[:, :, None] * wl.L + colL[None, None, :])  # [c, pt, L]
        if wl.latent_fp8:
            c = fp8_codes(wl.key("lat8"), idx)
            c[:, :, wl.V:] = 0
            latent[p0:p1] = c.to(torch.uint8)
            del idx, c
        else:
            if wl.latent_int:
                v = uniform_int(klat, idx, -4, 4).to(torch.float32)
            else:
                v = table[hash32(klat, idx) >> 16]
            v[:, :, wl.V:] = 0
            latent[p0:p1] = v.to(dt)
            del idx, v
        pool = lpg_t[p0:p1, None] * ppp + pool_in_page[None, :]                      # [c, ppp]
        idx = ((s[:, None] * TMAX + pool)[:, :, None] * wl.D + colD[None, None, :])
        kv = uniform_int(kpool, idx, -4, 4).to(torch.float32)
        keep = (pool < first_new_pool[s][:, None]).to(torch.float32)[:, :, None]
        pooled[p0:p1] = (kv * keep).to(dt)
        del idx, kv
    return latent, pooled


def device_tokens(wl: Workload, seq: int, toks, device):
    """Index keys and gates [len(toks), D] for one sequence's tokens, on ``device``."""
    import torch
    dt = _torch_dtype(wl)
    toks = torch.as_tensor(np.asarray(toks, dtype=np.int64), device=device)
    colD = torch.arange(wl.D, dtype=torch.int64, device=device)
    base = (seq * TMAX + toks)[:, None] * wl.D + colD[None, :]
    if wl.key_per_token:
        keys = uniform_int(wl.key("ktok"), base, -4, 4)
    else:
        pidx = (seq * TMAX + toks // wl.P)[:, None] * wl.D + colD[None, :]
        keys = uniform_int(wl.key("kpool"), pidx, -4, 4)
    table = torch.from_numpy(normal_table(wl.dtype)).to(device)
    gates = table[hash32(wl.key("gate"), base) >> 16]
    return keys.to(torch.float32).to(dt), gates.to(dt)


def device_queries(wl: Workload, device):
    """(q_idx [n_q, Hi, D], w [n_q, Hi] fp32, q [n_q, H, L]) on ``device``."""
    import torch
    dt = _torch_dtype(wl)
    st = torch.as_tensor(_seqtok(wl.q_seq, wl.q_pos), device=device)
    hi = torch.arange(wl.Hi, dtype=torch.int64, device=device)
    d = torch.arange(wl.D, dtype=torch.int64, device=device)
    qidx = uniform_int(wl.key("qidx"), (st[:, None, None] * wl.Hi + hi[None, :, None]) * wl.D + d[None, None, :],
                       -4, 4).to(torch.float32).to(dt)
    widx = st[:, None] * wl.Hi + hi[None, :]
    if wl.w_int:
        w = uniform_int(wl.key("w"), widx, -4, 4).to(torch.float32)
    else:
        w = uniform_int(wl.key("w"), widx, 0, 255).to(torch.float32) / 256.0
    w = w * float(wl.w_scale)
    h = torch.arange(wl.H, dtype=torch.int64, device=device)
    lc = torch.arange(wl.L, dtype=torch.int64, device=device)
    qi = (st[:, None, None] * wl.H + h[None, :, None]) * wl.L + lc[None, None, :]
    if wl.latent_int:
        q = uniform_int(wl.key("q"), qi, -4, 4).to(torch.float32)
    else:
        table = torch.from_numpy(normal_table(wl.dtype)).to(device)
        q = table[hash32(wl.key("q"), qi) >> 16]
    q[:, :, wl.V:] = 0
    return qidx, w.contiguous(), q.to(dt).contiguous()


def device_ape(wl: Workload, device):
    import torch
    return torch.from_numpy(host_ape(wl)).to(device).to(_torch_dtype(wl))


def compress_pools(wl: Workload):
    """(seq, pool) of every pool that completes during the step: pools [new_from // P, ctx // P)."""
    out = []
    for s in range(wl.B):
        for p in range(wl.new_from[s] // wl.P, wl.ctx[s] // wl.P):
            out.append((s, p))
    return out


class DeviceInputs:
    """Every device-side input of one workload step: the two paged caches and their block table, the queries,
    and the key/gate rows of the pools that complete in-step (as [n, P, D] blocks with their destinations)."""

    def __init__(self, wl: Workload, device):
        import torch
        self.wl = wl
        self.device = torch.device(device)
        self.block_table_np = wl.block_table()
        self.latent, self.pooled = device_caches(wl, self.device)
        self.block_table = torch.from_numpy(self.block_table_np).to(self.device)
        self.q_seq = torch.from_numpy(wl.q_seq.astype(np.int32)).to(self.device)
        self.q_pos = torch.from_numpy(wl.q_pos.astype(np.int32)).to(self.device)
        self.q_idx, self.w, self.q = device_queries(wl, self.device)
        self.cpools = compress_pools(wl)
        self.ape = device_ape(wl, self.device)
        if self.cpools:
            ks_, gs_ = [], []
            for s in sorted(set(s for s, _ in self.cpools)):
                ps = [p for ss, p in self.cpools if ss == s]
                toks = np.concatenate([np.arange(p * wl.P, p * wl.P + wl.P) for p in ps])
                kk, gg = device_tokens(wl, s, toks, self.device)
                ks_.append(kk.view(len(ps), wl.P, wl.D))
                gs_.append(gg.view(len(ps), wl.P, wl.D))
            order = sorted(self.cpools)
            self.c_keys = torch.cat(ks_).contiguous()
            self.c_gates = torch.cat(gs_).contiguous()
            self.c_seq = torch.tensor([s for s, _ in order], dtype=torch.int32, device=self.device)
            self.c_pool = torch.tensor([p for _, p in order], dtype=torch.int32, device=self.device)
        else:
            self.c_keys = self.c_gates = self.c_seq = self.c_pool = None
