"""The two modes of MLA attention (oracle; test infrastructure only).

Source: GLM5.3 sparse-attention page, MLA-modes paragraph: MLA runs either in an MHA mode
(fewer FLOPs, far more memory read) or in an MQA mode (less memory, 3.4 times the FLOPs); DSA
uses the MQA mode, and below some sequence length the MHA mode is the faster one.  The page
names the modes and their costs, not their equations.  Reading (the usual latent attention):
every token t stores a latent c_t (d_c values) and one rotary key r_t (r values) shared by all
heads; head h has up-projections W_UK[h] (d_nope x d_c) and W_UV[h] (d_v x d_c), and its query
is q_nope[h] (d_nope values) followed by q_rope[h] (r values).

MHA mode: per-head keys and values are materialised and each head attends to its own:
    k[t, h] = [W_UK[h] c_t ; r_t]              (d_nope + r values)
    v[t, h] = W_UV[h] c_t                      (d_v values)
    o[h]    = sum_t softmax_t(scale * q[h] . k[t, h]) v[t, h]
MQA mode: W_UK is absorbed into the query and W_UV into the output, so every head reads the one
latent row [c_t ; r_t] (d_c + r values), whose first d_c values act as the value:
    q'[h] = [W_UK[h]^T q_nope[h] ; q_rope[h]]
    o'[h] = sum_t softmax_t(scale * q'[h] . [c_t ; r_t]) c_t
    o[h]  = W_UV[h] o'[h]
The two give the same o, since q'[h] . [c_t ; r_t] = q[h] . k[t, h] and W_UV is linear.  Per
token and head, the MHA mode multiplies d_nope + r + d_v pairs and the MQA mode d_c + r + d_c;
per token, the MHA mode reads H (d_nope + r + d_v) values and the MQA mode d_c + r.
"""
from __future__ import annotations

import numpy as np


def mha_kv(c: np.ndarray, r: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray):
    """Per-head keys [n, H, d_nope + r] and values [n, H, d_v] from latents c [n, d_c], rotary
    keys r [n, r] and up-projections w_uk [H, d_nope, d_c], w_uv [H, d_v, d_c]."""
    c = np.asarray(c, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    n, H = c.shape[0], w_uk.shape[0]
    k_nope = np.einsum("hec,nc->nhe", np.asarray(w_uk, dtype=np.float64), c)
    k = np.concatenate([k_nope, np.broadcast_to(r[:, None, :], (n, H, r.shape[1]))], axis=2)
    v = np.einsum("hvc,nc->nhv", np.asarray(w_uv, dtype=np.float64), c)
    return k, v


def absorb_query(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """MQA-mode queries [H, d_c + r] from q_nope [H, d_nope], q_rope [H, r]."""
    qa = np.einsum("hec,he->hc", np.asarray(w_uk, dtype=np.float64), np.asarray(q_nope, dtype=np.float64))
    return np.concatenate([qa, np.asarray(q_rope, dtype=np.float64)], axis=1)


def unabsorb_output(o_latent: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Per-head outputs [H, d_v] from MQA-mode outputs over the latent [H, d_c]."""
    return np.einsum("hvc,hc->hv", np.asarray(w_uv, dtype=np.float64), np.asarray(o_latent, dtype=np.float64))


def mode_costs(H: int, d_c: int, r: int, d_nope: int, d_v: int) -> dict:
    """Multiply-adds and values read per cached token, for each mode (one query token)."""
    return {
        "mha_macs": H * (d_nope + r + d_v),
        "mqa_macs": H * (d_c + r + d_c),
        "mha_values": H * (d_nope + r + d_v),
        "mqa_values": d_c + r,
    }
