"""GPU parity of kp_linear (the dense projections beside the path) against the oracle, through the C ABI.

Shapes are the layer's (GLM-5.3-Flash model card: hidden 4096, q_lora 1536, 32 index heads x 128, 64 MLA heads,
kv_lora 512, qk_nope = v_head = 256) at a decode step of 64 tokens, ragged token counts (several tiles plus a
tail) and a 4096-token prefill chunk checked on sampled rows.
Bar: integer-valued operands ('int') make every fp32 sum exact, so fp32 outputs are bit-exact and bf16 outputs
equal the oracle's nearest-even rounding of the exact value.  Normal operands: |gpu - ref| <= 2^-8 |ref| +
2^-14 sum_k |a_k w_k| for bf16 outputs (one rounding plus fp32 accumulation), 2^-14 sum_k |a_k w_k| for fp32.
"""
import sys

import numpy as np
import pytest
import torch

import kpool_synth as ks
import oracle as O
import sparse_attention_kpool_amd as K

pytestmark = pytest.mark.gpu

HIDDEN, Q_RANK, HI, D, H, V, DN, DV, L = 4096, 1536, 32, 128, 64, 512, 256, 256, 576
SEED = 21


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda", dtype)


def _check(got, ref, abs_sum, out_bf16: bool, exact: bool, what: str):
    got = np.asarray(got, dtype=np.float64)
    if exact:
        want = O.bf16_round(ref) if out_bf16 else ref
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs " \
                              f"{want[tuple(bad[0])]}"
        return
    tol = 2.0 ** -14 * abs_sum + (2.0 ** -8 * np.abs(ref) if out_bf16 else 0.0)
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"{what}: error {err[worst]:.3g} > tol {tol[worst]:.3g} at {worst}"


def _workspace(batch, M, N, K_):
    """Split-K workspace for a shape, filled with a non-zero pattern: its contents must not matter."""
    n = K.linear_workspace_size(batch, M, N, K_)
    return torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda") if n else None


def _plain(T, N, K_, kind, out_dtype, tag, ldc=None, scale_a=1.0, scale_w=2.0 ** -6, split=True):
    """One unbatched product A [T, K] x W [N, K]^T -> C [T, N] (row stride ldc); split: pass the split-K
    workspace the shape asks for (decode shapes split K over several blocks)."""
    ws = _workspace(1, T, N, K_) if split else None
    _say(f"linear {tag}: T={T} N={N} K={K_} kind={kind} out={out_dtype} split-K={ws is not None}")
    a = ks.host_matrix(SEED, f"{tag}:a", (T, K_), kind, 1.0 if kind == "int" else scale_a)
    w = ks.host_matrix(SEED, f"{tag}:w", (N, K_), kind, 1.0 if kind == "int" else scale_w)
    ldc = ldc or N
    c_full = torch.full((T, ldc), 3.0, dtype=out_dtype, device="cuda")
    c = c_full[:, :N]
    K.linear(_dev(a), _dev(w), c, alpha=1.0, workspace=ws)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy()
    ref = O.linear(a, w)
    abs_sum = O.linear(np.abs(a), np.abs(w))
    _check(got, ref, abs_sum, out_dtype == torch.bfloat16, kind == "int", tag)
    if ldc > N:  # the padding columns are never written
        assert torch.all(c_full[:, N:] == 3.0).item(), f"{tag}: wrote past column N"


@pytest.mark.parametrize("kind,split", [("int", True), ("normal", True), ("int", False), ("normal", False)])
def test_index_query_projection_decode(kind, split):
    _plain(64, HI * D, Q_RANK, kind, torch.bfloat16, f"qidx-{kind}", split=split)


@pytest.mark.parametrize("kind,split", [("int", True), ("normal", True), ("normal", False)])
def test_head_weight_projection_fp32_out(kind, split):
    _plain(64, HI, HIDDEN, kind, torch.float32, f"w-{kind}", split=split)


def test_split_k_workspace_reuse_across_shapes():
    """One workspace (sized for the largest shape) serves consecutive calls of different shapes, whatever the
    previous call left in it."""
    _say("split-K workspace reuse")
    shapes = [(64, HI * D, Q_RANK), (64, 2 * D, HIDDEN), (64, HI, HIDDEN), (48, HI * D, Q_RANK)]
    n = max(K.linear_workspace_size(1, *s) for s in shapes)
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for i, (T, N, K_) in enumerate(shapes):
            a = ks.host_matrix(SEED, f"re{i}:a", (T, K_), "int")
            w = ks.host_matrix(SEED, f"re{i}:w", (N, K_), "int")
            c = torch.empty((T, N), dtype=torch.float32, device="cuda")
            K.linear(_dev(a), _dev(w), c, workspace=ws)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(c.cpu().numpy(), O.linear(a, w), err_msg=f"rep {rep} shape {i}")


def test_ragged_rows_and_columns():
    """Token counts that leave a partial tile (77 in one 128-row tile; 300 over three) and a column count that
    leaves a partial 4-column group (198, row stride 200)."""
    _plain(77, 198, 512, "int", torch.bfloat16, "ragged77", ldc=200)
    _plain(300, 198, 256, "int", torch.float32, "ragged300", ldc=200)
    _plain(5, 70, 128, "normal", torch.bfloat16, "ragged5", ldc=72)
    _plain(1, 64, 64, "int", torch.float32, "single")


def test_indexer_projections_key_then_gate():
    T = 64
    _say(f"indexer_project: T={T}")
    x = ks.host_matrix(SEED, "ip:x", (T, HIDDEN), "int")
    cq = ks.host_matrix(SEED, "ip:cq", (T, Q_RANK), "int")
    w_q = ks.host_matrix(SEED, "ip:wq", (HI * D, Q_RANK), "int")
    w_w = ks.host_matrix(SEED, "ip:ww", (HI, HIDDEN), "int")
    w_kg = ks.host_matrix(SEED, "ip:wkg", (2 * D, HIDDEN), "int")
    q_idx = torch.empty((T, HI, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    keys = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    n = max(K.linear_workspace_size(1, T, HI * D, Q_RANK), K.linear_workspace_size(1, T, HI, HIDDEN),
            K.linear_workspace_size(1, T, D, HIDDEN))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    K.indexer_project(_dev(x), _dev(cq), _dev(w_q), _dev(w_w), _dev(w_kg), q_idx, w, keys, gates, workspace=ws)
    torch.cuda.synchronize()
    r_q, r_w, r_k, r_g = O.indexer_project(x, cq, w_q, w_w, w_kg, HI, D)
    np.testing.assert_array_equal(q_idx.float().cpu().numpy(), O.bf16_round(r_q))
    np.testing.assert_array_equal(w.cpu().numpy(), r_w)
    np.testing.assert_array_equal(keys.float().cpu().numpy(), O.bf16_round(r_k))
    np.testing.assert_array_equal(gates.float().cpu().numpy(), O.bf16_round(r_g))


@pytest.mark.parametrize("T,kind", [(64, "int"), (64, "normal"), (300, "normal")])
def test_mla_absorb_query(T, kind):
    """q[t, h, :V] = W_UK[h]^T q_nope[t, h] for all 64 heads (one batch entry per head); the rotary columns of q
    keep what they held."""
    _say(f"mla_absorb_q: T={T} kind={kind}")
    q_nope = ks.host_matrix(SEED, f"ab{T}:q", (T, H, DN), kind)
    w_uk = ks.host_matrix(SEED, f"ab{T}:w", (H, DN, V), kind, 1.0 if kind == "int" else 2.0 ** -4)
    q = torch.full((T, H, L), 5.0, dtype=torch.bfloat16, device="cuda")
    w_uk_t = _dev(np.ascontiguousarray(np.transpose(w_uk, (0, 2, 1))))  # [H, V, dn], prepared once per layer
    K.mla_absorb_q(_dev(q_nope), w_uk_t, q)
    torch.cuda.synchronize()
    got = q.float().cpu().numpy()
    ref = O.mla_absorb_q(q_nope, w_uk)
    abs_sum = O.mla_absorb_q(np.abs(q_nope), np.abs(w_uk))
    _check(got[:, :, :V], ref, abs_sum, True, kind == "int", "absorb")
    assert np.all(got[:, :, V:] == 5.0), "absorb wrote into the rotary columns"


@pytest.mark.parametrize("T,kind", [(64, "int"), (64, "normal"), (77, "normal")])
def test_mla_unabsorb_output(T, kind):
    _say(f"mla_unabsorb_o: T={T} kind={kind}")
    o_lat = ks.host_matrix(SEED, f"un{T}:o", (T, H, V), kind)
    w_uv = ks.host_matrix(SEED, f"un{T}:w", (H, DV, V), kind, 1.0 if kind == "int" else 2.0 ** -4)
    o = torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda")
    K.mla_unabsorb_o(_dev(o_lat), _dev(w_uv), o, workspace=_workspace(H, T, DV, V))
    torch.cuda.synchronize()
    ref = O.mla_unabsorb_o(o_lat, w_uv)
    abs_sum = O.mla_unabsorb_o(np.abs(o_lat), np.abs(w_uv))
    _check(o.float().cpu().numpy(), ref, abs_sum, True, kind == "int", "unabsorb")


@pytest.mark.parametrize("T,kind", [(512, "int"), (1000, "int"), (1000, "normal")])
def test_absorb_weight_stationary(T, kind):
    """The absorb at prefill token counts (the weight-stationary kernel: one block per head and token range, the
    head's weight in registers, 32-token slabs; T = 1000 ends in a partial slab): every row of every head against
    the oracle, and the rotary columns of q untouched."""
    _say(f"mla_absorb_q (weight-stationary): T={T} kind={kind}")
    q_nope = ks.host_matrix(SEED, f"ws{T}:q", (T, H, DN), kind)
    w_uk = ks.host_matrix(SEED, f"ws{T}:w", (H, DN, V), kind, 1.0 if kind == "int" else 2.0 ** -4)
    q = torch.full((T, H, L), 5.0, dtype=torch.bfloat16, device="cuda")
    K.mla_absorb_q(_dev(q_nope), _dev(np.ascontiguousarray(np.transpose(w_uk, (0, 2, 1)))), q)
    torch.cuda.synchronize()
    got = q.float().cpu().numpy()
    _check(got[:, :, :V], O.mla_absorb_q(q_nope, w_uk), O.mla_absorb_q(np.abs(q_nope), np.abs(w_uk)), True,
           kind == "int", "absorb")
    assert np.all(got[:, :, V:] == 5.0), "absorb wrote into the rotary columns"


@pytest.mark.parametrize("T,kind,out", [(777, "int", torch.float32), (1000, "normal", torch.bfloat16),
                                        (1000, "normal", torch.float32)])
def test_unabsorb_weight_stationary(T, kind, out):
    """The un-absorb at prefill token counts (weight-stationary kernel, bf16 and fp32 outputs): every output."""
    _say(f"mla_unabsorb_o (weight-stationary): T={T} kind={kind} out={out}")
    o_lat = ks.host_matrix(SEED, f"wsu{T}:o", (T, H, V), kind)
    w_uv = ks.host_matrix(SEED, f"wsu{T}:w", (H, DV, V), kind, 1.0 if kind == "int" else 2.0 ** -4)
    o = torch.full((T, H, DV), 7.0, dtype=out, device="cuda")
    K.mla_unabsorb_o(_dev(o_lat), _dev(w_uv), o)
    torch.cuda.synchronize()
    _check(o.float().cpu().numpy(), O.mla_unabsorb_o(o_lat, w_uv), O.mla_unabsorb_o(np.abs(o_lat), np.abs(w_uv)),
           out == torch.bfloat16, kind == "int", "unabsorb")


def test_weight_stationary_batch8_alpha_and_padded_rows():
    """A plain batch of 8 entries of each weight-stationary shape through kp_linear, with alpha and output rows
    padded past N (the padding is never written), integer operands (exact)."""
    for N_, K_, M in ((512, 256, 600), (256, 512, 513)):
        _say(f"linear (weight-stationary): batch 8 M={M} N={N_} K={K_}")
        a = ks.host_matrix(SEED, f"ws8:a{N_}", (8, M, K_), "int")
        w = ks.host_matrix(SEED, f"ws8:w{N_}", (8, N_, K_), "int")
        c_full = torch.full((8, M, N_ + 8), 3.0, dtype=torch.bfloat16, device="cuda")
        K.linear(_dev(a), _dev(w), c_full[:, :, :N_], alpha=0.5)
        torch.cuda.synchronize()
        got = c_full[:, :, :N_].float().cpu().numpy()
        ref = np.stack([0.5 * O.linear(a[i], w[i]) for i in range(8)])
        np.testing.assert_array_equal(got, O.bf16_round(ref), err_msg=f"N={N_}")
        assert torch.all(c_full[:, :, N_:] == 3.0).item(), "wrote past column N"


def test_prefill_index_query_sampled_rows():
    """The 4096-token prefill chunk through the 128 x 128 tile path; 256 sampled rows, every column."""
    T = 4096
    _say(f"linear prefill: T={T} N={HI * D} K={Q_RANK}")
    a = ks.host_matrix(SEED, "pf:a", (T, Q_RANK), "normal")
    w = ks.host_matrix(SEED, "pf:w", (HI * D, Q_RANK), "normal", 2.0 ** -6)
    c = torch.empty((T, HI * D), dtype=torch.bfloat16, device="cuda")
    K.linear(_dev(a), _dev(w), c)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(T, 256, replace=False))
    rows[0], rows[-1] = 0, T - 1
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref = O.linear(a[rows], w)
    _check(got, ref, O.linear(np.abs(a[rows]), np.abs(w)), True, False, "prefill qidx")


def test_linear_alpha_and_shared_weight_batch():
    """alpha scales once before the rounding; a 2-D weight is shared by every batch entry (stride 0)."""
    _say("linear alpha / shared weight")
    a = ks.host_matrix(SEED, "al:a", (3, 40, 256), "int")
    w = ks.host_matrix(SEED, "al:w", (96, 256), "int")
    c = torch.empty((3, 40, 96), dtype=torch.float32, device="cuda")
    K.linear(_dev(a), _dev(w), c, alpha=0.25)
    torch.cuda.synchronize()
    ref = np.stack([O.linear(a[b], w, alpha=0.25) for b in range(3)])
    np.testing.assert_array_equal(c.cpu().numpy(), ref)


def test_group_mixed_products_and_short_workspace():
    """One grouped launch of products with different shapes, output dtypes, splits and row counts (the group takes
    the 128-row tile of its largest M); then the same group with a workspace that fits only the first product's
    split, so the rest run unsplit.  Integer operands: every output is exact either way."""
    _say("linear_group: mixed products")
    shapes = [(64, 32, 4096, torch.float32), (200, 130, 256, torch.bfloat16), (64, HI * D, Q_RANK, torch.bfloat16),
              (3, 8, 512, torch.float32)]
    ops, refs = [], []
    for i, (T, N, K_, dt) in enumerate(shapes):
        a = ks.host_matrix(SEED, f"gr{i}:a", (T, K_), "int")
        w = ks.host_matrix(SEED, f"gr{i}:w", (N, K_), "int")
        ldc = -(-N // 4) * 4  # output rows padded to a multiple of 4 elements
        ops.append((_dev(a), _dev(w), torch.empty((T, ldc), dtype=dt, device="cuda")[:, :N], 0.5))
        refs.append(O.linear(a, w, alpha=0.5))
    n = K.linear_group_workspace_size(ops)
    for ws_bytes in (n, 16 * 1024):
        ws = torch.full((max(ws_bytes, 16),), 0x55, dtype=torch.uint8, device="cuda") if ws_bytes else None
        for _, _, c, _ in ops:
            c.fill_(7.0)
        K.linear_group(ops, workspace=ws)
        torch.cuda.synchronize()
        for (_, _, c, _), ref in zip(ops, refs):
            want = O.bf16_round(ref) if c.dtype == torch.bfloat16 else ref
            np.testing.assert_array_equal(c.float().cpu().numpy(), want, err_msg=f"workspace {ws_bytes}")


def test_group_decode_step_products():
    """The five products that precede attention in a decode step (index query, head weights, key, gate, query
    absorb) in one grouped launch, normal operands, against the oracle."""
    T = 64
    _say(f"linear_group: decode-step products T={T}")
    x = ks.host_matrix(SEED, "ds:x", (T, HIDDEN), "normal")
    cq = ks.host_matrix(SEED, "ds:cq", (T, Q_RANK), "normal")
    w_q = ks.host_matrix(SEED, "ds:wq", (HI * D, Q_RANK), "normal", 2.0 ** -6)
    w_w = ks.host_matrix(SEED, "ds:ww", (HI, HIDDEN), "normal", 2.0 ** -6)
    w_kg = ks.host_matrix(SEED, "ds:wkg", (2 * D, HIDDEN), "normal", 2.0 ** -6)
    q_nope = ks.host_matrix(SEED, "ds:qn", (T, H, DN), "normal")
    w_uk = ks.host_matrix(SEED, "ds:wuk", (H, DN, V), "normal", 2.0 ** -4)
    q_idx = torch.empty((T, HI, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    keys = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((T, H, L), dtype=torch.bfloat16, device="cuda")
    w_uk_t = _dev(np.ascontiguousarray(np.transpose(w_uk, (0, 2, 1))))
    prods = K.indexer_products(_dev(x), _dev(cq), _dev(w_q), _dev(w_w), _dev(w_kg), q_idx, w, keys, gates)
    prods.append(K.absorb_product(_dev(q_nope), w_uk_t, q))
    ws = torch.empty(max(K.linear_group_workspace_size(prods), 16), dtype=torch.uint8, device="cuda")
    K.linear_group(prods, workspace=ws)
    torch.cuda.synchronize()
    r_q, r_w, r_k, r_g = O.indexer_project(x, cq, w_q, w_w, w_kg, HI, D)
    a_q, a_w, a_k, a_g = O.indexer_project(np.abs(x), np.abs(cq), np.abs(w_q), np.abs(w_w), np.abs(w_kg), HI, D)
    _check(q_idx.float().cpu().numpy(), r_q, a_q, True, False, "group q_idx")
    _check(w.cpu().numpy(), r_w, a_w, False, False, "group w")
    _check(keys.float().cpu().numpy(), r_k, a_k, True, False, "group keys")
    _check(gates.float().cpu().numpy(), r_g, a_g, True, False, "group gates")
    _check(q.float().cpu().numpy()[:, :, :V], O.mla_absorb_q(q_nope, w_uk),
           O.mla_absorb_q(np.abs(q_nope), np.abs(w_uk)), True, False, "group absorb")
    assert np.all(q.float().cpu().numpy()[:, :, V:] == 0.0)


@pytest.mark.parametrize("T", [64, 70])
def test_layer_projections_object(T):
    """LayerProjections (workspace sized once for up to 96 tokens): pre_attention's grouped launch and
    post_attention's un-absorb against the oracle, integer operands (exact)."""
    from sparse_attention_kpool_amd.layer import LayerProjections, ProjectionWeights
    _say(f"LayerProjections: T={T}")
    x = ks.host_matrix(SEED, f"lp{T}:x", (T, HIDDEN), "int")
    cq = ks.host_matrix(SEED, f"lp{T}:cq", (T, Q_RANK), "int")
    q_nope = ks.host_matrix(SEED, f"lp{T}:qn", (T, H, DN), "int")
    o_lat = ks.host_matrix(SEED, f"lp{T}:ol", (T, H, V), "int")
    w_q = ks.host_matrix(SEED, "lpw:q", (HI * D, Q_RANK), "int")
    w_w = ks.host_matrix(SEED, "lpw:w", (HI, HIDDEN), "int")
    w_kg = ks.host_matrix(SEED, "lpw:kg", (2 * D, HIDDEN), "int")
    w_uk = ks.host_matrix(SEED, "lpw:uk", (H, DN, V), "int")
    w_uv = ks.host_matrix(SEED, "lpw:uv", (H, DV, V), "int")
    wt = ProjectionWeights(w_q=_dev(w_q), w_w=_dev(w_w), w_kg=_dev(w_kg),
                           w_uk_t=_dev(np.ascontiguousarray(np.transpose(w_uk, (0, 2, 1)))), w_uv=_dev(w_uv))
    proj = LayerProjections(wt, max_tokens=96, device="cuda")
    q_idx = torch.empty((T, HI, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    keys = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((T, H, L), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda")
    proj.pre_attention(_dev(x), _dev(cq), _dev(q_nope), q_idx, w, keys, gates, q)
    proj.post_attention(_dev(o_lat), o)
    torch.cuda.synchronize()
    r_q, r_w, r_k, r_g = O.indexer_project(x, cq, w_q, w_w, w_kg, HI, D)
    np.testing.assert_array_equal(q_idx.float().cpu().numpy(), O.bf16_round(r_q))
    np.testing.assert_array_equal(w.cpu().numpy(), r_w)
    np.testing.assert_array_equal(keys.float().cpu().numpy(), O.bf16_round(r_k))
    np.testing.assert_array_equal(gates.float().cpu().numpy(), O.bf16_round(r_g))
    np.testing.assert_array_equal(q.float().cpu().numpy()[:, :, :V], O.bf16_round(O.mla_absorb_q(q_nope, w_uk)))
    np.testing.assert_array_equal(o.float().cpu().numpy(), O.bf16_round(O.mla_unabsorb_o(o_lat, w_uv)))


def test_group_prefill_chunk_sampled_rows():
    """The bench's prefill launch: the five pre-attention products of a 4096-token chunk in one grouped launch
    (128 x 128 tiles, 9312 blocks) and the un-absorb; 96 sampled token rows of every output against the oracle."""
    T = 4096
    _say(f"linear_group: prefill chunk T={T}")
    x = ks.host_matrix(SEED, "pc:x", (T, HIDDEN), "normal")
    cq = ks.host_matrix(SEED, "pc:cq", (T, Q_RANK), "normal")
    q_nope = ks.host_matrix(SEED, "pc:qn", (T, H, DN), "normal")
    o_lat = ks.host_matrix(SEED, "pc:ol", (T, H, V), "normal")
    w_q = ks.host_matrix(SEED, "pc:wq", (HI * D, Q_RANK), "normal", 2.0 ** -6)
    w_w = ks.host_matrix(SEED, "pc:ww", (HI, HIDDEN), "normal", 2.0 ** -6)
    w_kg = ks.host_matrix(SEED, "pc:wkg", (2 * D, HIDDEN), "normal", 2.0 ** -6)
    w_uk = ks.host_matrix(SEED, "pc:wuk", (H, DN, V), "normal", 2.0 ** -4)
    w_uv = ks.host_matrix(SEED, "pc:wuv", (H, DV, V), "normal", 2.0 ** -4)
    q_idx = torch.empty((T, HI, D), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    keys = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    gates = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((T, H, L), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda")
    prods = K.indexer_products(_dev(x), _dev(cq), _dev(w_q), _dev(w_w), _dev(w_kg), q_idx, w, keys, gates)
    prods.append(K.absorb_product(_dev(q_nope), _dev(np.ascontiguousarray(np.transpose(w_uk, (0, 2, 1)))), q))
    n = K.linear_group_workspace_size(prods)
    K.linear_group(prods, workspace=torch.empty(max(n, 16), dtype=torch.uint8, device="cuda"))
    K.mla_unabsorb_o(_dev(o_lat), _dev(w_uv), o)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(9).choice(T, 96, replace=False))
    rows[0], rows[-1] = 0, T - 1
    r = torch.from_numpy(rows).cuda()
    r_q, r_w, r_k, r_g = O.indexer_project(x[rows], cq[rows], w_q, w_w, w_kg, HI, D)
    a_q, a_w, a_k, a_g = O.indexer_project(np.abs(x[rows]), np.abs(cq[rows]), np.abs(w_q), np.abs(w_w),
                                           np.abs(w_kg), HI, D)
    _check(q_idx[r].float().cpu().numpy(), r_q, a_q, True, False, "prefill q_idx")
    _check(w[r].cpu().numpy(), r_w, a_w, False, False, "prefill w")
    _check(keys[r].float().cpu().numpy(), r_k, a_k, True, False, "prefill keys")
    _check(gates[r].float().cpu().numpy(), r_g, a_g, True, False, "prefill gates")
    _check(q[r].float().cpu().numpy()[:, :, :V], O.mla_absorb_q(q_nope[rows], w_uk),
           O.mla_absorb_q(np.abs(q_nope[rows]), np.abs(w_uk)), True, False, "prefill absorb")
    _check(o[r].float().cpu().numpy(), O.mla_unabsorb_o(o_lat[rows], w_uv),
           O.mla_unabsorb_o(np.abs(o_lat[rows]), np.abs(w_uv)), True, False, "prefill unabsorb")


def test_layer_chain_with_projections():
    """The documented decode chain: LayerProjections.pre_attention -> KPoolDSALayer.step -> post_attention, on
    real paged caches (three sequences of 29, 4096 and 7001 tokens).  Selector weights (identities) make the
    projections return the seeded inputs exactly, so the layer's output must equal, bit for bit, that of the same
    step fed those inputs directly."""
    from harness import DeviceRun
    from sparse_attention_kpool_amd.layer import LayerProjections, ProjectionWeights
    _say("layer chain with projections")
    base = ks.workloads()["batch64"]
    ctx = [29, 4096, 7001]
    wl = ks.scaled(base, name="chain", ctx=ctx, new_from=[t - 1 for t in ctx], q_seq=np.arange(3, dtype=np.int32),
                   q_pos=np.array([t - 1 for t in ctx], np.int32), k=256, page_perm_seed=5)
    run = DeviceRun(wl, device="cuda").run()
    torch.cuda.synchronize()
    T, hid = wl.n_q, 64
    bf = dict(dtype=torch.bfloat16, device="cuda")
    eye = lambda n: torch.eye(n, **bf)  # noqa: E731
    x = torch.zeros((T, hid), **bf)
    x[:, :HI] = run.w.to(torch.bfloat16)  # head weights lie on a 2^-8 grid below 1: exact in bf16
    wt = ProjectionWeights(w_q=eye(HI * D), w_w=eye(hid)[:HI].contiguous(), w_kg=torch.zeros((2 * D, hid), **bf),
                           w_uk_t=eye(V).expand(H, V, V).contiguous(), w_uv=eye(V).expand(H, V, V).contiguous())
    proj = LayerProjections(wt, max_tokens=T, device="cuda")
    q_idx = torch.empty((T, HI, D), **bf)
    w = torch.empty((T, HI), dtype=torch.float32, device="cuda")
    keys, gates = torch.empty((T, D), **bf), torch.empty((T, D), **bf)
    q = torch.zeros((T, H, L), **bf)
    proj.pre_attention(x, run.q_idx.reshape(T, HI * D), run.q[:, :, :V].contiguous(), q_idx, w, keys, gates, q)
    out = torch.empty_like(run.out)
    lse = torch.empty_like(run.lse)
    run.layer.step(run.cache, run.queries, q_idx, w, q, out, lse=lse, compress=run.compress)
    o = torch.empty((T, H, V), **bf)
    proj.post_attention(out, o)
    torch.cuda.synchronize()
    assert torch.equal(q_idx, run.q_idx) and torch.equal(w, run.w) and torch.equal(q, run.q)
    assert torch.equal(out, run.out) and torch.equal(lse, run.lse)
    assert torch.equal(o, out)
