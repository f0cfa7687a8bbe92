"""fp64 reference for the dense products around the attention (test infrastructure only).

What the pages fix:

* The hidden state h_t is compressed into a query latent c_t^Q and a key/value
  latent c_t^KV, and the decoupled rotary key k_t^R is produced beside them
  ([LKVC] "Operation Flow", step 1; [LRKV] "Empirical Gains", the paragraph on
  what MLA caches): c = W^D h for each down-projection W^D.
* The query parts come from the query latent: q^C_i = W^UQ_i c^Q per head and
  the rotary query q^R_i from its own projection ([LKVC] "Operation Flow",
  step 2).
* At inference W^UK can be folded into the query weights and W^UV into the
  output projection W^O ([LRKV] "Empirical Gains", the paragraph on absorption;
  FAQ "How does MLA optimize computation during inference?"):
    q~_i = W^UK_i^T q^C_i = (W^UK_i^T W^UQ_i) c^Q,
    y    = W^O [o_1; ...; o_H] = sum_i (W^O_i W^UV_i) o~_i,
  with o~_i = sum_t p_t c_t the latent output of head i and W^O_i the columns
  of W^O that multiply head i's d_v outputs.

Every function here is that linear algebra written out with numpy products
(a library primitive); the pins are in tests/test_oracle_projections.py.
"""

import numpy as np


def down_project(h, w):
    """c = W h for every row of h: h [T, d_model], w [d_out, d_model] -> [T, d_out]."""
    return np.asarray(h, np.float64) @ np.asarray(w, np.float64).T


def up_project_query(c_q, w_uq, w_qr):
    """Per-head content and rotary queries from the query latent.

    c_q [T, d_cq], w_uq [H, d_nope, d_cq], w_qr [H, d_rope, d_cq] ->
    (q_nope [T, H, d_nope], q_rope [T, H, d_rope]); q_rope is not rotated.
    """
    c_q = np.asarray(c_q, np.float64)
    q_nope = np.einsum("hnq,tq->thn", np.asarray(w_uq, np.float64), c_q)
    q_rope = np.einsum("hrq,tq->thr", np.asarray(w_qr, np.float64), c_q)
    return q_nope, q_rope


def absorb_query_weights(w_uq, w_uk):
    """W~_i = W^UK_i^T W^UQ_i per head: w_uq [H, d_nope, d_cq], w_uk [H, d_nope, d_c]
    -> [H, d_c, d_cq], so that q~_i = W~_i c^Q."""
    w_uq = np.asarray(w_uq, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    return np.stack([w_uk[i].T @ w_uq[i] for i in range(w_uq.shape[0])])


def absorb_output_weights(w_o, w_uv):
    """W~^O = [W^O_1 W^UV_1, ..., W^O_H W^UV_H]: w_o [d_model, H d_v],
    w_uv [H, d_v, d_c] -> [d_model, H d_c], so that y = W~^O [o~_1; ...; o~_H]."""
    w_o = np.asarray(w_o, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    H, d_v, _ = w_uv.shape
    return np.concatenate([w_o[:, i * d_v:(i + 1) * d_v] @ w_uv[i] for i in range(H)], axis=1)


def output_project(o, w_o):
    """y = W^O o for every row: o [T, K], w_o [d_model, K] -> [T, d_model]."""
    return np.asarray(o, np.float64) @ np.asarray(w_o, np.float64).T
