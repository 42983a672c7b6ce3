"""Top-k token selection (oracle; test infrastructure only).

Source: GLM5.3 sparse-attention page, lightning-indexer paragraph: the indexer
score picks the top K tokens; a query that attends to fewer than K tokens stays
dense (all its tokens are kept), otherwise the top K are kept.  The MLA-modes
paragraph restates it: below 2K tokens (top K = 2048) attention is dense.

The pages do not say how equal scores are ordered.  Reading: among equal
scores the lower position wins.  The result is returned as ascending
positions, so two correct selections compare equal element by element.

Method: a full sort by (score descending, position ascending) and the first k
entries, i.e. the definition itself.  Scores compare as floats: -0 equals +0
(a tie, decided by position), and numpy's sort puts a NaN after every number,
so a NaN ranks last (NaNs among themselves by position).  Indexer scores have
neither; the reading matters only for scores a caller passes in.
"""
from __future__ import annotations

import numpy as np


def select(scores: np.ndarray, k: int) -> np.ndarray:
    """Ascending positions of the kept tokens of one request (int64)."""
    s = np.asarray(scores)
    n = s.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    pos = np.arange(n)
    order = np.lexsort((pos, -s))          # last key is primary: score desc, then position asc
    return np.sort(order[:k]).astype(np.int64)


def select_padded(scores: np.ndarray, k: int) -> np.ndarray:
    """``select`` padded with -1 to length k (int32), the library's output layout."""
    sel = select(scores, k)
    out = np.full(k, -1, dtype=np.int32)
    out[:sel.shape[0]] = sel
    return out
