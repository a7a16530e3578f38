"""Plain float64 definitions of the dense projections on either side of the KPool-DSA path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Sources, cited by page title and section:

* [llama.cpp pull request "add GLM-5.3-Flash (GLM5-Next) support", section "What I implemented new"] -- the
  indexer cache holds a key and a gate for every token, so one projection of the hidden state yields both;
  the indexer and the MLA low-rank paths stay unquantized.
* [MAX ``max.pipelines.architectures.glm5_next`` API page, ``compute_dtype``] -- the indexer and ``kv_b_proj``
  run in the compute dtype (bf16), not in the fp8 of the quantized attention projections.
* [GLM-5.3-Flash model card, "Raw config fields"] -- hidden_size 4096, q_lora_rank 1536, index_n_heads 32,
  index_head_dim 128, num_attention_heads 64, kv_lora_rank 512, qk_nope_head_dim 256, v_head_dim 256.

Absorbed MLA (the layer's specification): the key of token t for head h would be W_UK[h] c_t and its value
W_UV[h] c_t, with c_t the token's latent row.  Because q . (W_UK[h] c) = (W_UK[h]^T q) . c, the query is moved
into latent space once ("absorb") and attention runs on the latent rows; because the output is linear in the
values, sum_t p_t W_UV[h] c_t = W_UV[h] (sum_t p_t c_t), so the latent output is mapped back once ("un-absorb").

Readings taken here:
  R26 the key-and-gate projection puts the key in its first D output columns and the gate in the next D
      (the page lists them in that order: key | gate).
  R27 index head h's query is channels h*D .. h*D+D-1 of the index query projection (head-major rows).
  R28 W_UK[h] is [qk_nope_head_dim, kv_lora_rank] and W_UV[h] is [v_head_dim, kv_lora_rank] (each maps a
      latent row to one head's key or value, as kv_b_proj's two halves do).
"""
from __future__ import annotations

import numpy as np


def linear(a, w, alpha: float = 1.0) -> np.ndarray:
    """alpha * a @ w^T in float64: a [..., K], w [N, K] (a weight stored output-major) -> [..., N]."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return alpha * (a @ w.T)


def indexer_project(x, cq, w_q, w_w, w_kg, Hi: int, D: int):
    """The indexer's three projections (R26, R27).

    x [T, hidden] hidden state, cq [T, q_lora] compressed query; w_q [Hi*D, q_lora], w_w [Hi, hidden],
    w_kg [2D, hidden].  Returns q_idx [T, Hi, D], w [T, Hi], keys [T, D], gates [T, D].
    """
    T = np.asarray(x).shape[0]
    q_idx = linear(cq, w_q).reshape(T, Hi, D)
    w = linear(x, w_w)
    kg = linear(x, w_kg)
    return q_idx, w, kg[:, :D], kg[:, D:2 * D]


def mla_absorb_q(q_nope, w_uk) -> np.ndarray:
    """Query in latent space: q_lat[t, h] = W_UK[h]^T q_nope[t, h] (R28).

    q_nope [T, H, dn], w_uk [H, dn, V] -> [T, H, V].
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    T, H, dn = q_nope.shape
    out = np.empty((T, H, w_uk.shape[2]))
    for h in range(H):
        out[:, h, :] = q_nope[:, h, :] @ w_uk[h]
    return out


def mla_unabsorb_o(o_lat, w_uv) -> np.ndarray:
    """Head output from the latent output: o[t, h] = W_UV[h] o_lat[t, h] (R28).

    o_lat [T, H, V], w_uv [H, dv, V] -> [T, H, dv].
    """
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    T, H, V = o_lat.shape
    out = np.empty((T, H, w_uv.shape[1]))
    for h in range(H):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[h].T
    return out
