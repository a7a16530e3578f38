"""sparse_mla_attn_noalloc -- the attention entry point that allocates nothing (its split-KV partials live in the
library's static per-device scratch) -- against sparse_mla_attn with a caller workspace, through the C ABI.

Two calls in a row, the second with fewer queries (more splits per query, a different scratch layout): both must
equal sparse_mla_attn on the same inputs bit for bit (same kernels, same split count), lse included."""
import sys

import numpy as np
import pytest
import torch

import kpool_synth as ks
import sparse_attention_kpool_amd as K
from harness import DeviceRun, Guarded

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _with_workspace(run, n):
    queries = K.Queries(seq=run.queries.seq[:n], pos=run.queries.pos[:n], max_pos=run.queries.max_pos, group=1)
    need = K.sparse_mla_workspace_size(run.dims, queries)
    ws = torch.empty(max((need + 15) // 16 * 4, 4), dtype=torch.float32, device="cuda") if need else None
    out = torch.empty((n, run.wl.H, run.wl.V), dtype=run.out.dtype, device="cuda")
    lse = torch.empty((n, run.wl.H), dtype=torch.float32, device="cuda")
    K.sparse_mla_attn(run.dims, run.cache, queries, run.q[:n], run.layer.sel[:n], run.layer.n_sel[:n], out,
                      lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return queries, out, lse, need


def test_noalloc_matches_workspace_call_twice():
    base = ks.workloads()["batch64"]
    ctx = [int(3000 + 97 * s) for s in range(64)]
    wl = ks.scaled(base, name="noalloc", ctx=ctx, new_from=[t - 1 for t in ctx], q_seq=np.arange(64, dtype=np.int32),
                   q_pos=np.array([t - 1 for t in ctx], np.int32), k=512, page_perm_seed=12)
    _say("[case noalloc] 64 queries, then 3")
    run = DeviceRun(wl).run()
    for n in (64, 3):                      # the second call is smaller: more splits per query, other offsets
        queries, ref_out, ref_lse, need = _with_workspace(run, n)
        assert 0 < need <= K.NOALLOC_SCRATCH_BYTES
        out = Guarded((n, wl.H, wl.V), run.out.dtype, "cuda")
        lse = Guarded((n, wl.H), torch.float32, "cuda")
        K.sparse_mla_attn_noalloc(run.dims, run.cache, queries, run.q[:n], run.layer.sel[:n], run.layer.n_sel[:n],
                                  out.t, lse=lse.t)
        torch.cuda.synchronize()
        assert out.intact() and lse.intact(), "noalloc wrote outside its outputs"
        assert torch.equal(out.t, ref_out), f"{n} queries: output differs from sparse_mla_attn"
        assert torch.equal(lse.t, ref_lse), f"{n} queries: lse differs from sparse_mla_attn"
        _say(f"  {n} queries: {need} bytes of scratch, bit-identical to the workspace call")
    # the full step's own output (64 queries) once more, after the smaller call reused the scratch
    out = torch.empty_like(run.out)
    K.sparse_mla_attn_noalloc(run.dims, run.cache, run.queries, run.q, run.layer.sel, run.layer.n_sel, out)
    torch.cuda.synchronize()
    assert torch.equal(out, run.out)
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
