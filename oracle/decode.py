"""One decode step of one request: score, select, attend (oracle; test infrastructure only).

Chains ``indexer.scores``, ``topk.select`` and ``sdpa.attend`` in the order the
GLM5.3 sparse-attention page describes (lightning indexer picks the top K,
sparse attention runs over them).  The cache is given in logical order, i.e.
already read through the page table; reading through the table is checked
separately by ``paging.build_page_tables`` parity and by permuting the pool.
"""
from __future__ import annotations

import numpy as np

from . import indexer, topk, sdpa
from .bf16 import to_f64


def request_step(q_bits, qidx_bits, w_idx, kidx_bits, k_bits, v_bits, top_k: int, scale: float,
                 v_from_k_dims: int = 0):
    """Returns (scores, selected positions, output [Hq, dv] float64).

    ``v_bits`` may be None with ``v_from_k_dims`` > 0: the values are the first
    ``v_from_k_dims`` dims of each key row (MQA mode of MLA).
    """
    s = indexer.scores_bf16(qidx_bits, w_idx, kidx_bits)
    sel = topk.select(s, top_k)
    k_sel = to_f64(k_bits[sel])
    v_sel = k_sel[:, :, :v_from_k_dims] if v_bits is None else to_f64(v_bits[sel])
    o = sdpa.attend(to_f64(q_bits), k_sel, v_sel, scale)
    return s, sel, o


def attend_positions(q_bits, k_bits, v_bits, sel, scale: float, v_from_k_dims: int = 0):
    """SDPA over caller-given positions (no indexer): the tiered workload's path."""
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[sel >= 0]
    k_sel = to_f64(k_bits[sel])
    v_sel = k_sel[:, :, :v_from_k_dims] if v_bits is None else to_f64(v_bits[sel])
    return sdpa.attend(to_f64(q_bits), k_sel, v_sel, scale)
