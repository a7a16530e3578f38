"""Pins of the CPU oracle to things other than itself: hand-worked fixtures, closed forms, limits, brute force,
invariants and library routines.  CPU only.

Each test names what it pins; together they are meant to fail on a plausible slip anywhere in the oracle
(a dropped term, a wrong sign or index, a transposed operand, an off-by-one in the pool geometry)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------------------------------------
def test_bf16_round_matches_torch_rne():
    """bf16 rounding against torch's float32 -> bfloat16 conversion (round to nearest even)."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-6, 6, 20000),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 255.5, 256.5, 3.0])]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_hand_cases():
    # spacing of bf16 at 1 is 2^-7: 1 + 2^-8 ties to 1 (even); 1 + 3*2^-8 ties to 1 + 2^-6
    assert O.bf16_round(1 + 2 ** -8) == 1.0
    assert O.bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert O.bf16_round(-4.0) == -4.0 and O.bf16_round(0.0) == 0.0
    assert O.store_round(1 + 2 ** -30, "f32") == 1.0


# ----------------------------------------------------------------------------------------------------------
# pooling
# ----------------------------------------------------------------------------------------------------------
def test_pool_hand_worked_fixture():
    d = _gold("pool_closed_form.json")
    for c in d["cases"]:
        gate = np.log(np.array(c["gate_w"], dtype=np.float64))
        ape = np.log(np.array(c["ape_w"], dtype=np.float64))
        keys = np.array(c["keys"], dtype=np.float64)
        got = O.pool_compress(keys[None, :, None], gate[None, :, None], ape[:, None])
        assert abs(got[0, 0] - c["pooled"]) < 1e-12, c


def test_pool_constant_key_returns_key():
    """Specification invariant: pooling a constant key returns that key (exactly, once stored)."""
    rng = np.random.default_rng(1)
    n, P, D = 50, 4, 32
    key = rng.integers(-4, 5, size=(n, 1, D)).astype(np.float64)
    keys = np.repeat(key, P, axis=1)
    gates = rng.standard_normal((n, P, D)) * 3
    ape = rng.standard_normal((P, D))
    got = O.pool_compress(keys, gates, ape)
    np.testing.assert_allclose(got, key[:, 0], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(O.store_round(got, "bf16"), key[:, 0])


def test_pool_zero_gate_is_mean():
    """gate = ape = 0 reduces to the plain mean (the non-compressing pooling variant)."""
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((7, 4, 16))
    got = O.pool_compress(keys, np.zeros_like(keys), np.zeros((4, 16)))
    np.testing.assert_allclose(got, keys.mean(axis=1), rtol=1e-14, atol=1e-14)


def test_pool_mean_worked_example():
    """Plain-mean pooling on a hand-computed pool: tokens (1, 10), (2, 20), (4, 40), (9, -30) -> (4, 10)."""
    keys = np.array([[[1.0, 10.0], [2.0, 20.0], [4.0, 40.0], [9.0, -30.0]]])
    np.testing.assert_array_equal(O.pool_mean(keys), [[4.0, 10.0]])
    # P = 16 pools (the other pool size): sixteen tokens 0 .. 15 average to 7.5
    np.testing.assert_array_equal(O.pool_mean(np.arange(16.0).reshape(1, 16, 1)), [[7.5]])


def test_pool_mean_is_zero_gate_compress():
    """The plain mean is the learned pooling with gate = ape = 0 (uniform softmax weights)."""
    rng = np.random.default_rng(12)
    keys = rng.standard_normal((9, 4, 8))
    np.testing.assert_allclose(O.pool_mean(keys), O.pool_compress(keys, np.zeros_like(keys), np.zeros((4, 8))),
                               rtol=1e-14, atol=1e-14)


def test_pool_dominant_gate_limit():
    """One gate logit 60 above the rest: the pooled key is that token's key (weights of the rest < e^-50)."""
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((5, 4, 8))
    gates = rng.standard_normal((5, 4, 8))
    hot = rng.integers(0, 4, size=(5, 8))
    for p in range(5):
        for c in range(8):
            gates[p, hot[p, c], c] += 60.0
    got = O.pool_compress(keys, gates, np.zeros((4, 8)))
    want = np.take_along_axis(keys, hot[:, None, :], axis=1)[:, 0]
    np.testing.assert_allclose(got, want, atol=1e-18 + 1e-12)


def test_pool_ape_only_and_order_of_operands():
    """ape affects token j only through z_j: with the ape of token 1 raised by ln 3, token 1 gets weight 3/6.
    Catches ape transposed to [D, P] or added to the keys instead of the logits."""
    P, D = 4, 6
    keys = np.arange(P * D, dtype=np.float64).reshape(1, P, D)
    ape = np.zeros((P, D))
    ape[1, :] = math.log(3.0)
    got = O.pool_compress(keys, np.zeros((1, P, D)), ape)[0]
    want = (keys[0, 0] + 3 * keys[0, 1] + keys[0, 2] + keys[0, 3]) / 6.0
    np.testing.assert_allclose(got, want, rtol=1e-14)


def test_pool_bruteforce_python():
    """Tiny random pools against a pure-Python loop with math.exp."""
    rng = np.random.default_rng(4)
    n, P, D = 3, 4, 5
    keys = rng.standard_normal((n, P, D))
    gates = rng.standard_normal((n, P, D))
    ape = rng.standard_normal((P, D))
    got = O.pool_compress(keys, gates, ape)
    for p in range(n):
        for c in range(D):
            z = [float(gates[p, j, c] + ape[j, c]) for j in range(P)]
            e = [math.exp(v) for v in z]
            want = sum(e[j] * float(keys[p, j, c]) for j in range(P)) / sum(e)
            assert abs(got[p, c] - want) < 1e-13


def test_pool_shift_invariance():
    """Adding a per-(pool, channel) constant to every gate of the pool leaves the pooled key unchanged."""
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((6, 4, 8))
    gates = rng.standard_normal((6, 4, 8))
    ape = rng.standard_normal((4, 8))
    shift = rng.standard_normal((6, 1, 8)) * 50
    np.testing.assert_allclose(O.pool_compress(keys, gates + shift, ape), O.pool_compress(keys, gates, ape),
                               rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------------------------------
# pool geometry
# ----------------------------------------------------------------------------------------------------------
def test_pool_geometry_bruteforce():
    """n_c, r, tau against counting tokens one by one."""
    for P in (1, 2, 4, 16):
        for i in range(0, 70):
            n_c = sum(1 for p in range(100) if p * P + P - 1 <= i)
            tail_tokens = [t for t in range(0, i + 1) if t // P >= n_c]
            tau = i // P
            assert O.pool_geometry(i, P) == (n_c, len(tail_tokens), tau)
            assert all(t // P == tau for t in tail_tokens)


# ----------------------------------------------------------------------------------------------------------
# scoring
# ----------------------------------------------------------------------------------------------------------
def test_scores_exact_fractions():
    """Integer q and keys, w on the 2^-8 grid: exact values from Python Fractions."""
    rng = np.random.default_rng(6)
    Hi, D, n = 4, 16, 12
    q = rng.integers(-4, 5, size=(Hi, D))
    k = rng.integers(-4, 5, size=(n, D))
    wj = rng.integers(0, 256, size=Hi)
    w = wj / 256.0
    got = O.indexer_scores(q, w, k, n)
    for p in range(n):
        exact = Fraction(0)
        for h in range(Hi):
            dot = sum(int(q[h, c]) * int(k[p, c]) for c in range(D))
            exact += Fraction(int(wj[h]), 256) * max(dot, 0)
        assert Fraction(got[p]) == exact


def test_scores_single_head_is_relu_dot():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 8))
    k = rng.standard_normal((20, 8))
    got = O.indexer_scores(q, np.ones(1), k, 20)
    np.testing.assert_allclose(got, np.maximum(k @ q[0], 0), rtol=1e-14)


def test_scores_causal_prefix_and_linearity():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((20, 8))
    w = rng.standard_normal(3)
    s = O.indexer_scores(q, w, k, 20)
    assert len(O.indexer_scores(q, w, k, 7)) == 7
    np.testing.assert_allclose(O.indexer_scores(q, w, k, 7), s[:7])
    np.testing.assert_allclose(O.indexer_scores(q, 2.5 * w, k, 20), 2.5 * s, rtol=1e-13)   # linear in w
    np.testing.assert_allclose(O.indexer_scores(3 * q, w, k, 20), 3 * s, rtol=1e-13)        # homogeneous in q
    # negating one head's query swaps which pools that head contributes to (ReLU is not odd)
    q2 = q.copy()
    q2[0] *= -1
    s2 = O.indexer_scores(q2, w, k, 20)
    want = s + w[0] * (np.maximum(-(k @ q[0]), 0) - np.maximum(k @ q[0], 0))
    np.testing.assert_allclose(s2, want, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------------------------------------
def test_selection_hand_worked_fixture():
    d = _gold("selection_hand.json")
    for c in d["cases"]:
        sel = O.select_pools(np.array(c["scores"], dtype=np.float64), c["i"], c["P"], c["k"])
        assert sel.tolist() == c["sel"], c
        assert O.attended_tokens(sel, c["i"], c["P"]).tolist() == c["tokens"], c


def _select_by_counting(s, i, P, k):
    """Brute force, independent of any sort: a complete pool p is kept iff fewer than k' pools beat it under
    (score desc, index asc)."""
    n_c = (i + 1) // P
    r = (i + 1) % P
    kp = k - (1 if r else 0)
    out = []
    for p in range(n_c):
        beats = sum(1 for q in range(n_c) if s[q] > s[p] or (s[q] == s[p] and q < p))
        if beats < kp:
            out.append(p)
    if r:
        out.append(i // P)
    return sorted(out)


@pytest.mark.parametrize("seed", range(40))
def test_selection_bruteforce_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    P = int(rng.choice([1, 2, 4]))
    i = int(rng.integers(0, 60))
    k = int(rng.integers(1, 12))
    n_c = (i + 1) // P
    s = rng.integers(-3, 4, size=n_c).astype(np.float64)     # heavy ties
    s[s == 0] = rng.choice([0.0, -0.0], size=int((s == 0).sum()))
    sel = O.select_pools(s, i, P, k)
    assert sel.tolist() == _select_by_counting(s, i, P, k)


@pytest.mark.parametrize("seed", range(20))
def test_selection_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    P = 4
    i = int(rng.integers(0, 200))
    n_c, r, tau = O.pool_geometry(i, P)
    s = rng.standard_normal(n_c)
    prev = None
    for k in range(1, n_c + 3):
        sel = O.select_pools(s, i, P, k)
        assert len(sel) == min(k - (1 if r else 0), n_c) + (1 if r else 0)
        assert (np.diff(sel) > 0).all()
        if r:
            assert tau in sel.tolist()                          # the incomplete tail is always kept
        assert all(p < n_c or (r and p == tau) for p in sel)    # causal
        if prev is not None:
            assert set(prev.tolist()) <= set(sel.tolist())      # nested in k
        prev = sel
    # k at least the number of visible pools: every visible pool
    assert O.select_pools(s, i, P, n_c + 1).tolist() == list(range(n_c + (1 if r else 0)))


def test_shared_selection_hand_cases():
    """MTP draft reusing a target's selection (hand-worked, P = 4): the draft sees every token <= its position of
    the target's pools, plus its own incomplete trailing pool, which is never a top-k pick but always visible."""
    P = 4
    # target at 22 selected pools 0 and 5 (5 = its incomplete tail, tokens 20..22)
    # draft at 23 completes pool 5: tokens 0..3 and 20..23, nothing added
    assert O.shared_attended_tokens([0, 5], 23, P).tolist() == [0, 1, 2, 3, 20, 21, 22, 23]
    # draft at 24 starts pool 6, which the target could not select: tokens of 0 and 5, then token 24 itself
    assert O.shared_attended_tokens([0, 5], 24, P).tolist() == [0, 1, 2, 3, 20, 21, 22, 23, 24]
    # draft at 26 (pool 6 holds 24..26): all three pending tokens
    assert O.shared_attended_tokens([2, 5], 26, P).tolist() == [8, 9, 10, 11, 20, 21, 22, 23, 24, 25, 26]
    # a row that already holds the draft's pool adds nothing; its pool is cut at the draft
    assert O.shared_attended_tokens([1, 6], 25, P).tolist() == [4, 5, 6, 7, 24, 25]
    # an empty row: only the pending tokens
    assert O.shared_attended_tokens([], 9, P).tolist() == [8, 9]


@pytest.mark.parametrize("seed", range(10))
def test_shared_selection_invariants(seed):
    """A query reading its own selection attends exactly what attended_tokens gives; a draft reading an earlier
    target's selection always attends itself, attends no token after itself, and every target token it sees was
    selected by the target or is one of its own pending tokens."""
    rng = np.random.default_rng(300 + seed)
    P = 4
    i_t = int(rng.integers(0, 300))
    n_c, r, tau = O.pool_geometry(i_t, P)
    s = rng.standard_normal(n_c)
    for k in (1, 2, 5, 50):
        sel = O.select_pools(s, i_t, P, k)
        assert O.shared_attended_tokens(sel, i_t, P).tolist() == O.attended_tokens(sel, i_t, P).tolist()
        for d in (1, 2, 3):
            i = i_t + d
            toks = O.shared_attended_tokens(sel, i, P).tolist()
            assert i in toks                                    # the draft always sees itself
            assert max(toks) == i and len(set(toks)) == len(toks)
            own_pool = i // P
            for t in toks:
                assert t // P in sel.tolist() or t // P == own_pool


# ----------------------------------------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------------------------------------
def _masked_dense(q, c, scale, V, mask):
    """Textbook dense attention with -inf outside the mask (the 'scatter' form)."""
    logits = scale * (q @ c.T)
    logits = np.where(mask[None, :], logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return (e @ c[:, :V]) / e.sum(axis=1, keepdims=True), (m + np.log(e.sum(axis=1, keepdims=True)))[:, 0]


def test_attention_gather_equals_masked_dense():
    rng = np.random.default_rng(9)
    H, L, V, T = 4, 20, 16, 40
    q = rng.standard_normal((H, L))
    c = rng.standard_normal((T, L))
    toks = np.sort(rng.choice(T, size=13, replace=False))
    mask = np.zeros(T, bool)
    mask[toks] = True
    o, lse = O.sparse_mla(q, c[toks], 0.3, V)
    o2, lse2 = _masked_dense(q, c, 0.3, V, mask)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12)


def test_attention_against_torch_sdpa():
    """Library pin: torch CPU scaled_dot_product_attention (float64) with a boolean mask, values = first V cols."""
    rng = np.random.default_rng(10)
    H, L, V, T = 3, 24, 16, 30
    q = rng.standard_normal((H, L))
    c = rng.standard_normal((T, L))
    toks = np.sort(rng.choice(T, size=9, replace=False))
    mask = torch.zeros(T, dtype=torch.bool)
    mask[torch.from_numpy(toks)] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(c)[None, None].expand(1, H, T, L),
        torch.from_numpy(c[:, :V])[None, None].expand(1, H, T, V), attn_mask=mask[None, None, None, :],
        scale=0.25)[0, :, 0, :].numpy()
    o, _ = O.sparse_mla(q, c[toks], 0.25, V)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(11)
    H, L, V = 2, 6, 4
    c = rng.standard_normal((5, L))
    # one token: the output is that token's value row, lse its logit
    q = rng.standard_normal((H, L))
    o, lse = O.sparse_mla(q, c[2:3], 0.5, V)
    np.testing.assert_allclose(o, np.repeat(c[2:3, :V], H, axis=0), rtol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * (q @ c[2]), rtol=1e-14)
    # zero query: uniform weights -> mean of the value rows, lse = log n
    o, lse = O.sparse_mla(np.zeros((H, L)), c, 0.5, V)
    np.testing.assert_allclose(o, np.repeat(c[:, :V].mean(0, keepdims=True), H, axis=0), rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(5.0))
    # two tokens with logits 0 and ln 3: weights 1/4, 3/4; the value uses only columns < V
    q = np.zeros((1, L))
    q[0, 5] = 1.0
    cc = np.zeros((2, L))
    cc[1, 5] = math.log(3.0)
    cc[0, :V] = [4, 8, 0, -4]
    cc[1, :V] = [0, 4, 8, 4]
    o, lse = O.sparse_mla(q, cc, 1.0, V)
    np.testing.assert_allclose(o[0], [1.0, 5.0, 6.0, 2.0], rtol=1e-13)
    np.testing.assert_allclose(lse, [math.log(4.0)], rtol=1e-13)


def test_attention_permutation_invariant():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 10))
    c = rng.standard_normal((17, 10))
    perm = rng.permutation(17)
    o1, l1 = O.sparse_mla(q, c, 0.7, 8)
    o2, l2 = O.sparse_mla(q, c[perm], 0.7, 8)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


# ----------------------------------------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------------------------------------
def _tiny_layer(rng, T=37, P=4, D=8, Hi=3, H=2, L=12, V=8):
    keys = rng.integers(-4, 5, size=(T, D)).astype(np.float64)
    gates = rng.standard_normal((T, D))
    ape = rng.standard_normal((P, D))
    lat = rng.standard_normal((T, L))
    lat[:, V:] = 0
    n_pools = T // P
    pooled = O.store_round(O.pool_compress(keys[:n_pools * P].reshape(n_pools, P, D),
                                           gates[:n_pools * P].reshape(n_pools, P, D), ape), "f32")
    return keys, gates, ape, lat, pooled


def test_layer_k_covers_everything_is_dense_causal_mla():
    """With k >= number of visible pools the layer is dense causal MLA over tokens 0..i (torch SDPA pin)."""
    rng = np.random.default_rng(13)
    P, T, H, L, V = 4, 37, 2, 12, 8
    _, _, _, lat, pooled = _tiny_layer(rng, T=T, P=P, H=H, L=L, V=V)
    lo = O.LayerOracle(P=P, k=64, scale=0.4, V=V)
    for i in range(T):
        q = rng.standard_normal((H, L))
        q[:, V:] = 0
        res = lo.query(i, rng.integers(-4, 5, (3, 8)), rng.random(3), pooled, q, lambda t: lat[t])
        assert res["tokens"].tolist() == list(range(i + 1))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], torch.from_numpy(lat[:i + 1])[None, None].expand(1, H, i + 1, L),
            torch.from_numpy(lat[:i + 1, :V])[None, None].expand(1, H, i + 1, V), scale=0.4)[0, :, 0, :].numpy()
        np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_layer_causality():
    """Changing anything at tokens > i leaves query i's selection and output unchanged."""
    rng = np.random.default_rng(14)
    P, T = 4, 40
    keys, gates, ape, lat, pooled = _tiny_layer(rng, T=T, P=P)
    lo = O.LayerOracle(P=P, k=3, scale=0.4, V=8)
    qi, w = rng.integers(-4, 5, (3, 8)), rng.random(3)
    q = rng.standard_normal((2, 12))
    for i in (5, 18, 23, 30):
        a = lo.query(i, qi, w, pooled, q, lambda t: lat[t])
        lat2 = lat.copy()
        lat2[i + 1:] = rng.standard_normal(lat2[i + 1:].shape)
        pooled2 = pooled.copy()
        pooled2[(i + 1) // P:] = rng.integers(-4, 5, pooled2[(i + 1) // P:].shape)
        b = lo.query(i, qi, w, pooled2, q, lambda t: lat2[t])
        assert a["sel"].tolist() == b["sel"].tolist()
        np.testing.assert_array_equal(a["out"], b["out"])
        assert max(a["tokens"]) <= i
        if (i + 1) % P:
            assert max(a["tokens"]) == i                        # the incomplete tail reaches the query itself

# ----------------------------------------------------------------------------------------------------------
# fp8 latent codes (OCP E4M3)
# ----------------------------------------------------------------------------------------------------------
def test_fp8_e4m3_published_values():
    """Landmarks of the E4M3 format: 1.0, 1.5, 2.0, 3.75, the largest finite value 448, the smallest normal 2^-6,
    the smallest subnormal 2^-9, the signed zero and NaN."""
    d = O.fp8_e4m3_decode
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0x40) == 2.0 and d(0x47) == 3.75
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x07) == 7 * 2.0 ** -9 and d(0x01) == 2.0 ** -9
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and np.signbit(d(0x80)) and d(0xB8) == -1.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))


def test_fp8_e4m3_order_and_count():
    """Codes 0x00..0x7E decode strictly increasing (the magnitude order of the encoding), the negative half
    mirrors them, and there are 253 distinct finite values (+0 and -0 equal)."""
    pos = O.fp8_e4m3_decode(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()
    np.testing.assert_array_equal(O.fp8_e4m3_decode(np.arange(0x80, 0xFF)), -pos)
    vals = O.fp8_e4m3_decode(np.arange(256))
    assert len(np.unique(vals[~np.isnan(vals)])) == 253


# ---- dense projections (oracle/projections.py) ----

def test_linear_bruteforce_python():
    """alpha * a @ w^T against a pure-Python triple loop on a tiny case (brute force; catches a transposed w)."""
    rng = np.random.default_rng(11)
    a = rng.integers(-5, 6, size=(3, 7)).astype(float)
    w = rng.integers(-5, 6, size=(4, 7)).astype(float)
    got = O.linear(a, w, alpha=0.5)
    for m in range(3):
        for n in range(4):
            acc = 0.0
            for kk in range(7):
                acc += a[m][kk] * w[n][kk]
            assert got[m, n] == 0.5 * acc


def test_absorbed_query_scores_equal_explicit_keys():
    """Absorption: (W_UK[h]^T q) . c == q . (W_UK[h] c) for every head and latent row (associativity).  A
    transposed W_UK or a wrong head index breaks the equality."""
    rng = np.random.default_rng(12)
    T, H, dn, V, n = 3, 4, 6, 10, 5
    q_nope = rng.standard_normal((T, H, dn))
    w_uk = rng.standard_normal((H, dn, V))
    c = rng.standard_normal((n, V))
    q_lat = O.mla_absorb_q(q_nope, w_uk)
    for h in range(H):
        k_nope = c @ w_uk[h].T  # [n, dn]: the explicit keys of head h
        np.testing.assert_allclose(q_lat[:, h, :] @ c.T, q_nope[:, h, :] @ k_nope.T, rtol=1e-12, atol=1e-12)


def test_unabsorbed_output_equals_explicit_values():
    """Un-absorption: W_UV[h] (sum_t p_t c_t) == sum_t p_t (W_UV[h] c_t) for probability weights p."""
    rng = np.random.default_rng(13)
    T, H, dv, V, n = 2, 3, 5, 9, 7
    w_uv = rng.standard_normal((H, dv, V))
    c = rng.standard_normal((n, V))
    p = rng.random((T, H, n))
    p /= p.sum(axis=2, keepdims=True)
    o_lat = np.einsum("thn,nv->thv", p, c)
    got = O.mla_unabsorb_o(o_lat, w_uv)
    for t in range(T):
        for h in range(H):
            vals = c @ w_uv[h].T  # [n, dv]: the explicit values of head h
            np.testing.assert_allclose(got[t, h], p[t, h] @ vals, rtol=1e-12, atol=1e-12)


def test_indexer_project_key_then_gate_and_head_major():
    """Key | gate order of the shared projection (llama.cpp PR, "What I implemented new") and the head-major
    layout of the index query, on selector weights whose outputs are known in closed form."""
    rng = np.random.default_rng(14)
    T, hidden, q_rank, Hi, D = 3, 16, 12, 2, 4
    x = rng.integers(-8, 9, size=(T, hidden)).astype(float)
    cq = rng.integers(-8, 9, size=(T, q_rank)).astype(float)
    w_kg = np.zeros((2 * D, hidden))
    for d in range(D):
        w_kg[d, d] = 1.0          # key channel d = x[:, d]
        w_kg[D + d, D + d] = -2.0  # gate channel d = -2 x[:, D + d]
    w_q = np.zeros((Hi * D, q_rank))
    for h in range(Hi):
        for d in range(D):
            w_q[h * D + d, (3 * h + d) % q_rank] = 1.0
    w_w = np.zeros((Hi, hidden))
    w_w[0, hidden - 1] = 1.0
    w_w[1, 0] = 3.0
    q_idx, w, keys, gates = O.indexer_project(x, cq, w_q, w_w, w_kg, Hi, D)
    assert q_idx.shape == (T, Hi, D) and w.shape == (T, Hi) and keys.shape == (T, D) and gates.shape == (T, D)
    np.testing.assert_array_equal(keys, x[:, :D])
    np.testing.assert_array_equal(gates, -2.0 * x[:, D:2 * D])
    for h in range(Hi):
        for d in range(D):
            np.testing.assert_array_equal(q_idx[:, h, d], cq[:, (3 * h + d) % q_rank])
    np.testing.assert_array_equal(w[:, 0], x[:, hidden - 1])
    np.testing.assert_array_equal(w[:, 1], 3.0 * x[:, 0])
