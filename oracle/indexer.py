"""Lightning-indexer scores (oracle; test infrastructure only).

Source: GLM5.3 sparse-attention page ("Cơ chế chú ý thưa (Sparse Attention)
trên GLM5.3 ảnh hưởng thế nào đến bộ nhớ HBM?"), lightning-indexer paragraph.
The indexer query has several heads, the indexer key one head; each head's
query-key dot product goes through a ReLU, and the token's score is the sum of
those over heads, each weighted by the head's weight.  No values, no softmax.

    score[t] = sum_h  w[h] * max(0, sum_d q[h, d] * k[t, d])

The projections that produce q and k need trained weights and are not part of
this reference: q, k and w are inputs.  When every input is integer-valued the
score is computed exactly in int64 (that is what makes the fp32 result of a
GPU exactly comparable); otherwise in float64.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64


def _as_int_if_exact(x: np.ndarray):
    xi = np.rint(x)
    if np.array_equal(xi, x) and np.all(np.abs(xi) < 2 ** 31):
        return xi.astype(np.int64)
    return None


def scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Scores of every key row against one request's indexer query.

    q: [heads, dim] float values; w: [heads]; keys: [tokens, dim].
    Returns int64 [tokens] when all inputs are integers, else float64.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    qi, wi, ki = _as_int_if_exact(q), _as_int_if_exact(w), _as_int_if_exact(keys)
    if qi is not None and wi is not None and ki is not None:
        q, w, keys = qi, wi, ki
    logits = keys @ q.T                     # [tokens, heads]: one dot product per head
    relu = np.maximum(logits, 0)            # ReLU per head
    return relu @ w                         # weighted sum over heads


def scores_bf16(q_bits: np.ndarray, w: np.ndarray, key_bits: np.ndarray) -> np.ndarray:
    """``scores`` on bf16 bit patterns (decoded exactly to float64 first)."""
    return scores(to_f64(q_bits), np.asarray(w, dtype=np.float64), to_f64(key_bits))
