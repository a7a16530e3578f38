"""One KPool-DSA layer step over the C ABI: compress -> score -> select -> attend, and the dense projections on
either side of it.

``KPoolDSALayer`` sizes and owns the intermediate buffers (scores, selection, workspaces) once, at
construction, for a maximum batch shape; ``step`` then only enqueues the four library calls on the current
stream -- no allocation, no host synchronisation.  ``LayerProjections`` does the same for the projections: one
grouped launch before attention (index query, head weights, key | gate, query absorb) and the output un-absorb
after it.  Caches, queries, weights and outputs belong to the caller.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (KP_DTYPE_BF16, KP_DTYPE_F32, Cache, Dims, Queries, absorb_product, dsa_compress_score,
               dsa_indexer_score,
               dsa_topk_select, dsa_topk_workspace_size, indexer_products, linear_group,
               linear_shapes_workspace_size, mla_unabsorb_o, sparse_mla_attn, sparse_mla_attn_fp8,
               sparse_mla_attn_mtp, sparse_mla_mtp_workspace_size, sparse_mla_workspace_size)


@dataclass
class CompressInput:
    """Pools that complete this step: keys/gates [n_src, P, D] rows, selected by ``src`` (None: row i)."""
    keys: torch.Tensor
    gates: torch.Tensor
    ape: torch.Tensor
    pool_seq: torch.Tensor
    pool_id: torch.Tensor
    src: Optional[torch.Tensor] = None


class KPoolDSALayer:
    """``mtp=True`` also sizes the workspace of ``verify_step`` (MTP verification: targets and their drafts)."""

    def __init__(self, dims: Dims, device, max_q: int, max_pos: int, mtp: bool = False):
        self.dims = dims
        self.device = torch.device(device)
        n_pool_max = (max_pos + 1) // dims.pool
        self.ld = max(4, (n_pool_max + 3) // 4 * 4)     # 16-byte aligned score rows
        self.scores = torch.empty((max_q, self.ld), dtype=torch.float32, device=self.device)
        self.sel = torch.empty((max_q, dims.topk), dtype=torch.int32, device=self.device)
        self.n_sel = torch.empty((max_q,), dtype=torch.int32, device=self.device)
        probe = Queries(seq=torch.empty(max_q, dtype=torch.int32), pos=torch.empty(max_q, dtype=torch.int32),
                        max_pos=max_pos)
        # how rows and selections are split depends on the number of queries: size each workspace for the
        # largest need over 1..max_q
        need_topk = need_attn = 0
        for n in range(1, max_q + 1):
            qn = Queries(seq=probe.seq[:n], pos=probe.pos[:n], max_pos=max_pos)
            need_topk = max(need_topk, dsa_topk_workspace_size(dims, qn))
            need_attn = max(need_attn, sparse_mla_workspace_size(dims, qn))
        self.ws_topk = self._ws(need_topk)
        self.ws_attn = self._ws(need_attn)
        self.ws_mtp = None
        if mtp:
            need_mtp = max(sparse_mla_mtp_workspace_size(dims, Queries(seq=probe.seq[:n], pos=probe.pos[:n],
                                                                       max_pos=max_pos))
                           for n in range(1, max_q + 1))
            self.ws_mtp = self._ws(need_mtp)
        self.mtp = mtp
        self.max_q, self.max_pos = max_q, max_pos

    def _ws(self, nbytes: int):
        if nbytes == 0:
            return None
        return torch.empty(((nbytes + 15) // 16 * 4,), dtype=torch.float32, device=self.device)

    def _compress_score(self, cache: Cache, compress: Optional[CompressInput], queries: Queries, q_idx, w,
                        scores) -> None:
        # the step's completed pools, then the scores (one launch for a decode batch: dsa_compress_score)
        if compress is not None and compress.pool_seq.numel() > 0:
            dsa_compress_score(self.dims, cache, compress.keys, compress.gates, compress.ape, compress.pool_seq,
                               compress.pool_id, queries, q_idx, w, scores, src=compress.src)
        else:
            dsa_indexer_score(self.dims, cache, queries, q_idx, w, scores)

    def step(self, cache: Cache, queries: Queries, q_idx, w, q, out, lse=None,
             compress: Optional[CompressInput] = None) -> None:
        n_q = int(queries.seq.numel())
        if n_q > self.max_q or queries.max_pos > self.max_pos:
            raise ValueError("call shape exceeds the layer's allocation")
        scores = self.scores[:n_q]
        self._compress_score(cache, compress, queries, q_idx, w, scores)
        dsa_topk_select(self.dims, queries, scores, self.sel[:n_q], self.n_sel[:n_q], workspace=self.ws_topk)
        if cache.latent.dtype == torch.uint8:   # an fp8 (E4M3) latent cache
            sparse_mla_attn_fp8(self.dims, cache, queries, q, self.sel[:n_q], self.n_sel[:n_q], cache.latent_scale,
                                out, lse=lse, workspace=self.ws_attn)
        else:
            sparse_mla_attn(self.dims, cache, queries, q, self.sel[:n_q], self.n_sel[:n_q], out, lse=lse,
                            workspace=self.ws_attn)

    def verify_step(self, cache: Cache, queries: Queries, targets: Queries, q_idx, w, q, out, lse=None,
                    compress: Optional[CompressInput] = None) -> None:
        """MTP verification: ``queries`` holds runs of a target (entry 2r) and its draft (entry 2r + 1); ``targets``
        holds the targets alone (entry r = queries' entry 2r), with their index queries ``q_idx`` and head weights
        ``w``.  The targets are scored and selected; then every query attends its run's selection through
        sparse_mla_attn_mtp (one gather per run).  ``q``, ``out``, ``lse`` are per query of ``queries``."""
        if not self.mtp:
            raise ValueError("verify_step needs a layer built with mtp=True")
        n_q, n_t = int(queries.seq.numel()), int(targets.seq.numel())
        if n_q > self.max_q or n_t != (n_q + 1) // 2 or max(queries.max_pos, targets.max_pos) > self.max_pos:
            raise ValueError("call shape exceeds the layer's allocation, or targets are not one per run")
        self._compress_score(cache, compress, targets, q_idx, w, self.scores[:n_t])
        dsa_topk_select(self.dims, targets, self.scores[:n_t], self.sel[:n_t], self.n_sel[:n_t],
                        workspace=self.ws_topk)
        sparse_mla_attn_mtp(self.dims, cache, queries, q, self.sel[:n_t], self.n_sel[:n_t], out, lse=lse,
                            workspace=self.ws_mtp)


@dataclass
class ProjectionWeights:
    """The layer's dense weights, bf16, output-major (rows = outputs): w_q [Hi*D, q_lora] (index query, head-major),
    w_w [Hi, hidden] (head weights), w_kg [2D, hidden] (key rows, then gate rows), w_uk_t [H, V, dn] (W_UK[h]
    transposed, prepared once at load), w_uv [H, dv, V]."""
    w_q: torch.Tensor
    w_w: torch.Tensor
    w_kg: torch.Tensor
    w_uk_t: torch.Tensor
    w_uv: torch.Tensor


class LayerProjections:
    """The projections of one layer for up to ``max_tokens`` tokens a step; the split-K workspace is sized once."""

    def __init__(self, weights: ProjectionWeights, max_tokens: int, device):
        self.wt = weights
        Hi_D, q_rank = weights.w_q.shape
        Hi, hidden = weights.w_w.shape
        D2 = weights.w_kg.shape[0]
        H, V, dn = weights.w_uk_t.shape
        dv = weights.w_uv.shape[1]
        need = 0
        # the split rule depends on the token count: take the largest need over every count up to max_tokens
        for T in range(1, max_tokens + 1):
            pre = [(1, T, Hi_D, q_rank, KP_DTYPE_BF16), (1, T, Hi, hidden, KP_DTYPE_F32),
                   (1, T, D2 // 2, hidden, KP_DTYPE_BF16), (1, T, D2 // 2, hidden, KP_DTYPE_BF16),
                   (H, T, V, dn, KP_DTYPE_BF16)]
            need = max(need, linear_shapes_workspace_size(pre),
                       linear_shapes_workspace_size([(H, T, dv, V, KP_DTYPE_BF16)]))
        self.ws = None if need == 0 else torch.empty(need, dtype=torch.uint8, device=device)
        self.max_tokens = max_tokens

    def pre_attention(self, x, cq, q_nope, q_idx, w, keys, gates, q) -> None:
        """q_idx [T, Hi, D], w [T, Hi] (float32), keys / gates [T, D] and q[:, :, :V] [T, H, L] from the hidden
        state x [T, hidden], the compressed query cq [T, q_lora] and q_nope [T, H, dn]: one grouped launch."""
        if x.shape[0] > self.max_tokens:
            raise ValueError("more tokens than the projections were sized for")
        wt = self.wt
        linear_group(indexer_products(x, cq, wt.w_q, wt.w_w, wt.w_kg, q_idx, w, keys, gates)
                     + [absorb_product(q_nope, wt.w_uk_t, q)], workspace=self.ws)

    def post_attention(self, o_lat, o) -> None:
        """o [T, H, dv] from the latent attention output o_lat [T, H, V]."""
        if o_lat.shape[0] > self.max_tokens:
            raise ValueError("more tokens than the projections were sized for")
        mla_unabsorb_o(o_lat, self.wt.w_uv, o, workspace=self.ws)
