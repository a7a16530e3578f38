"""One KPool-DSA layer step over the C ABI: compress -> score -> select -> attend.

``KPoolDSALayer`` sizes and owns the intermediate buffers (scores, selection, workspaces) once, at
construction, for a maximum batch shape; ``step`` then only enqueues the four library calls on the current
stream -- no allocation, no host synchronisation.  Caches, queries and outputs belong to the caller.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (Cache, Dims, Queries, dsa_indexer_score, dsa_topk_select, dsa_topk_workspace_size, kpool_compress,
               sparse_mla_attn, sparse_mla_attn_fp8, sparse_mla_workspace_size)


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
    def __init__(self, dims: Dims, device, max_q: int, max_pos: int):
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
        self.max_q, self.max_pos = max_q, max_pos

    def _ws(self, nbytes: int):
        if nbytes == 0:
            return None
        return torch.empty(((nbytes + 15) // 16 * 4,), dtype=torch.float32, device=self.device)

    def step(self, cache: Cache, queries: Queries, q_idx, w, q, out, lse=None,
             compress: Optional[CompressInput] = None) -> None:
        n_q = int(queries.seq.numel())
        if n_q > self.max_q or queries.max_pos > self.max_pos:
            raise ValueError("call shape exceeds the layer's allocation")
        if compress is not None and compress.pool_seq.numel() > 0:
            kpool_compress(self.dims, cache, compress.keys, compress.gates, compress.ape, compress.pool_seq,
                           compress.pool_id, src=compress.src)
        scores = self.scores[:n_q]
        dsa_indexer_score(self.dims, cache, queries, q_idx, w, scores)
        dsa_topk_select(self.dims, queries, scores, self.sel[:n_q], self.n_sel[:n_q], workspace=self.ws_topk)
        if cache.latent.dtype == torch.uint8:   # an fp8 (E4M3) latent cache
            sparse_mla_attn_fp8(self.dims, cache, queries, q, self.sel[:n_q], self.n_sel[:n_q], cache.latent_scale,
                                out, lse=lse, workspace=self.ws_attn)
        else:
            sparse_mla_attn(self.dims, cache, queries, q, self.sel[:n_q], self.n_sel[:n_q], out, lse=lse,
                            workspace=self.ws_attn)
