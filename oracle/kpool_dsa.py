"""Plain float64 definitions of the four stages of the KPool-DSA layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Sources, cited by page title and section:

* [MAX ``max.pipelines.architectures.glm5_next`` API page] -- config fields ``index_kpool`` (tokens per scoring
  pool), ``index_kpool_always_select_tail`` (the incomplete trailing pool is always visible),
  ``index_kpool_compress`` (pooled key = learned weighted average over the pool's tokens: gate logits plus a
  learned intra-pool position embedding), ``mla_use_nope`` (no rotary embedding in the text decoder),
  ``build_layers()`` (576-wide latent carrying 64 rotary columns that are all zero), ``mla_head_dim``.
* [llama.cpp pull request "add GLM-5.3-Flash (GLM5-Next) support", section "What I implemented new"] -- the
  indexer scores pools of 4 consecutive tokens and always keeps the incomplete tail; the indexer cache stores
  key and gate per token; attention layers are nope-only MLA.  [same page, soft_max crash report] -- the pooling
  softmax runs on a [4, 128, n_pool] tensor, i.e. over a pool's 4 tokens, per channel, per pool, with
  n_pool = n_kv / kpool (integer division: complete pools only).
* [GLM-5.3-Flash model card, "Raw config fields"] -- index_head_dim 128, index_n_heads 32, index_kpool 4,
  index_topk 2048, kv_lora_rank 512, num_attention_heads 64, qk_head_dim 256, qk_rope_head_dim 0.

Where the pages give no formula, the layer's specification fixes it: pooling is a softmax over (gate logit +
position term) within each pool followed by a weighted sum of the keys; a pool's score is the head-weighted sum
of ReLU(q_h . k_pool); ties break toward the lower pool index.

Readings taken here (each one lives in exactly one function):
  R1  one gate logit per (token, channel); the softmax runs over the pool's P tokens independently per channel.
  R2  the position term ``ape`` has shape [P, D] and is added to the gate logits before the softmax.
  R3  one D-wide index key per token and per pool, shared by all index heads.
  R4  only complete pools (P*p + P-1 <= i) are pooled and scored.
  R5  the tail pool is forced only when it is incomplete, i.e. when (i+1) mod P != 0.
  R6  the forced tail uses one of the k slots.
  R7  inside the tail pool only tokens <= i are attended.
  R24 a query reusing another query's selection row (an MTP draft) keeps its own incomplete tail visible.
  R8  ranking order is (score descending, pool index ascending).
  R9  the selection is reported as ascending pool ids.
  R14 attention keys are the full latent rows; values are their first V columns.
  R16 lse is the natural log of the sum of exp(scaled logits).
  R17 stored values are rounded once, to nearest-even, to the storage dtype.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------------------------------------
# storage rounding (R17)
# ----------------------------------------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64 ``x``, returned as float64.

    Written from the format's definition: x = m * 2^e with m in [0.5, 1); keep round_half_even(m * 2^8) / 2^8.
    Values here are far inside bf16's exponent range, so subnormals and overflow do not arise.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def store_round(x, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage dtype ('bf16' or 'f32')."""
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 ("e4m3fn") codes as float64: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN; there are no infinities.
    The fp8 latent cache stores these codes; a row's values are the decoded codes times the cache's scale.
    Written from the format's definition.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


# ----------------------------------------------------------------------------------------------------------
# stage 1: pool compression (R1, R2, R4)
# ----------------------------------------------------------------------------------------------------------
def pool_compress(keys, gates, ape) -> np.ndarray:
    """Pooled keys of complete pools.

    keys, gates: [n_pools, P, D] (token j of pool p at [p, j]); ape: [P, D].
    For each pool and channel c: z_j = gate[j, c] + ape[j, c]; a = softmax_j(z); pooled[c] = sum_j a_j key[j, c].
    Returned unrounded in float64; the cache stores ``store_round`` of it.
    """
    keys = np.asarray(keys, dtype=np.float64)
    z = np.asarray(gates, dtype=np.float64) + np.asarray(ape, dtype=np.float64)[None, :, :]
    z = z - z.max(axis=1, keepdims=True)
    a = np.exp(z)
    a = a / a.sum(axis=1, keepdims=True)
    return (a * keys).sum(axis=1)


def pool_mean(keys) -> np.ndarray:
    """Pooled keys of complete pools without the learned weighting.

    [MAX ``glm5_next`` API page, ``index_kpool_compress``]: with the flag off, a pool's key is the plain mean of its
    tokens' keys.  keys: [n_pools, P, D] -> [n_pools, D], unrounded float64.
    """
    keys = np.asarray(keys, dtype=np.float64)
    return keys.sum(axis=1) / keys.shape[1]


# ----------------------------------------------------------------------------------------------------------
# positions (R4, R5)
# ----------------------------------------------------------------------------------------------------------
def pool_geometry(i: int, P: int):
    """For a query at absolute position i (0-based): (n_c, r, tau).

    n_c: number of complete pools visible to it (pools p with P*p + P - 1 <= i);
    r:   tokens in its incomplete trailing pool (0 when the last visible pool is complete);
    tau: index of the pool holding token i.
    """
    n_c = (i + 1) // P
    r = (i + 1) % P
    tau = i // P
    return n_c, r, tau


# ----------------------------------------------------------------------------------------------------------
# stage 2: pool scoring (R3, R4)
# ----------------------------------------------------------------------------------------------------------
def indexer_scores(q_idx, w, pooled, n_c: int) -> np.ndarray:
    """s[p] = sum_h w[h] * max(0, q_idx[h] . pooled[p]) for the complete pools p < n_c.

    q_idx: [Hi, D]; w: [Hi]; pooled: [>= n_c, D] (one key per pool, shared by every head).
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(pooled, dtype=np.float64)[:n_c]
    dots = k @ q_idx.T                       # [n_c, Hi]
    return (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)


# ----------------------------------------------------------------------------------------------------------
# stage 3: causal top-k with the forced incomplete tail (R5, R6, R8, R9)
# ----------------------------------------------------------------------------------------------------------
def select_pools(scores, i: int, P: int, k: int) -> np.ndarray:
    """Selected pool ids (ascending, int64) for the query at position i.

    The incomplete tail pool tau (present when r != 0) is always selected and takes one of the k slots; the
    remaining min(k - [r != 0], n_c) slots go to complete pools in the order (score desc, pool index asc).
    """
    n_c, r, tau = pool_geometry(i, P)
    s = np.asarray(scores, dtype=np.float64)[:n_c]
    budget = min(k - (1 if r else 0), n_c)
    # a stable sort of -s keeps equal scores in ascending pool order; -0.0 and 0.0 compare equal
    order = np.argsort(-s, kind="stable")
    chosen = list(order[:max(budget, 0)])
    if r:
        chosen.append(tau)
    return np.sort(np.asarray(chosen, dtype=np.int64))


# ----------------------------------------------------------------------------------------------------------
# stage 4: nope-only absorbed sparse MLA (R7, R14, R16)
# ----------------------------------------------------------------------------------------------------------
def attended_tokens(sel, i: int, P: int) -> np.ndarray:
    """Token ids a query at position i attends: every token of each selected pool, cut at i (causal)."""
    toks = []
    for p in np.asarray(sel, dtype=np.int64):
        for j in range(P):
            t = int(p) * P + j
            if t <= i:
                toks.append(t)
    return np.asarray(toks, dtype=np.int64)


def shared_attended_tokens(sel, i: int, P: int) -> np.ndarray:
    """Token ids a query at position i attends when it reuses another query's selection row ``sel``.

    [MAX ``glm5_next`` API page, ``index_share_for_mtp_iteration``]: an MTP draft reuses its target's top-k
    selection.  [same page, ``index_kpool_always_select_tail``]: the incomplete trailing pool is always visible.
    The shared item is the target's top-k pick; the draft's own incomplete tail is not a pick, so it stays visible:
    the draft attends every token <= i of the row's pools, plus tokens P*tau .. i of its own pool tau = i // P
    when (i+1) mod P != 0 and the row does not already hold tau.  A query reading its own selection gets exactly
    ``attended_tokens`` (its selection already holds its incomplete tail).
    """
    n_c, r, tau = pool_geometry(i, P)
    pools = [int(p) for p in np.asarray(sel, dtype=np.int64)]
    if r and tau not in pools:
        pools.append(tau)
    return attended_tokens(np.sort(np.asarray(pools, dtype=np.int64)), i, P)


def sparse_mla(q, rows, scale: float, V: int):
    """Attention of one query over gathered latent rows.

    q: [H, L]; rows: [n, L] (latent rows of the attended tokens).  Logits l = scale * q . row over all L
    columns; a = softmax over the n tokens; O = sum_t a_t row_t[:V]; lse = log sum_t exp(l_t).
    Returns (O [H, V], lse [H]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    c = np.asarray(rows, dtype=np.float64)
    logits = scale * (q @ c.T)               # [H, n]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    ssum = e.sum(axis=1, keepdims=True)
    out = (e @ c[:, :V]) / ssum
    lse = (m + np.log(ssum))[:, 0]
    return out, lse


# ----------------------------------------------------------------------------------------------------------
# the layer over logical (unpaged) per-sequence arrays
# ----------------------------------------------------------------------------------------------------------
class LayerOracle:
    """Runs the four stages for queries of one sequence, from logical arrays.

    pooled:  [>= n_c, D] pooled keys of the sequence (already in storage precision);
    latent:  callable(tokens) -> [len(tokens), L] latent rows (storage precision), so huge caches need not
             be materialised on the host.
    """

    def __init__(self, P: int, k: int, scale: float, V: int):
        self.P, self.k, self.scale, self.V = P, k, scale, V

    def query(self, i: int, q_idx, w, pooled, q, latent):
        n_c, _, _ = pool_geometry(i, self.P)
        s = indexer_scores(q_idx, w, pooled, n_c)
        sel = select_pools(s, i, self.P, self.k)
        toks = attended_tokens(sel, i, self.P)
        out, lse = sparse_mla(q, latent(toks), self.scale, self.V)
        return dict(scores=s, sel=sel, tokens=toks, out=out, lse=lse)
