"""Scaled dot-product attention over the selected tokens (oracle; test infrastructure only).

Source: GLM5.3 sparse-attention page: sparse attention runs SDPA only over the
top-k tokens the indexer selected (opening paragraph); the selection is shared
by every attention head (lightning-indexer paragraph); DSA runs MLA in MQA mode,
where all query heads read one latent key whose leading dims are the values
(MLA-modes paragraph).

For query head h of one request, with KV head g(h):

    logits_j = scale * q[h] . K[t_j, g(h)]        over the selected t_j
    p        = exp(logits - max logits) / sum(...)
    o[h]     = sum_j p_j V[t_j, g(h)]

Readings where the pages are silent: grouped heads are consecutive,
g(h) = floor(h / (Hq / Hkv)); the scale is passed in (the workloads use
1/sqrt(d_k)); q and K are taken after any rotary embedding.  Everything is
float64 from exactly-decoded bf16 inputs.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """One request: q [Hq, dk], k_sel [n, Hkv, dk], v_sel [n, Hkv, dv] -> o [Hq, dv] float64."""
    q = np.asarray(q, dtype=np.float64)
    k_sel = np.asarray(k_sel, dtype=np.float64)
    v_sel = np.asarray(v_sel, dtype=np.float64)
    hq = q.shape[0]
    n, hkv = k_sel.shape[0], k_sel.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    grp = hq // hkv
    out = np.zeros((hq, v_sel.shape[2]), dtype=np.float64)
    if n == 0:
        return out
    for h in range(hq):
        g = h // grp
        logits = scale * (k_sel[:, g, :] @ q[h])
        p = np.exp(logits - logits.max())
        p /= p.sum()
        out[h] = p @ v_sel[:, g, :]
    return out


def normwise_rel_err(o: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||o - ref||_inf / ||ref||_inf (rows = last axis)."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(o - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0
