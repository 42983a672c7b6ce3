"""Pins of the oracle's indexer score and top-k selection.

Indexer: GLM5.3 sparse-attention page, lightning-indexer paragraph (per-head dot
product, ReLU, weighted sum over heads).  The pages print no numeric example, so
the pins are closed forms on constructed inputs, chosen so that a dropped ReLU,
a wrong sign, a wrong weight or a transposed operand each change the result.

Top-k: same paragraph (top K, dense when the context has at most K tokens); the
tie rule (lower position first) is the stated reading.  Pinned by closed forms
and by an independent threshold-count construction.
"""
import numpy as np
import pytest

import synth
from oracle import indexer, topk


def test_scores_single_head_closed_form():
    D = 32
    c = np.array([-3, -1, 0, 1, 2, 5])
    keys = np.repeat(c[:, None], D, axis=1)
    s = indexer.scores(np.ones((1, D)), [1], keys)
    assert s.dtype == np.int64
    assert s.tolist() == [0, 0, 0, D, 2 * D, 5 * D]           # max(0, D c)


def test_scores_two_heads_weighted_relu():
    D = 16
    c = np.array([-4, -1, 0, 2, 3])
    keys = np.repeat(c[:, None], D, axis=1)
    q = np.stack([np.ones(D), -np.ones(D)])
    s = indexer.scores(q, [2, 3], keys)
    expect = D * (2 * np.maximum(c, 0) + 3 * np.maximum(-c, 0))
    assert s.tolist() == expect.tolist()


def test_scores_rectangular_one_hot():
    """q [3 heads x 5 dims] with distinct entries; key t is a * e_(t mod 5)."""
    H, D = 3, 5
    q = np.arange(H * D).reshape(H, D) - 7              # entries -7..7, rows differ
    w = np.array([1, -2, 5])
    T = 20
    a = np.arange(T) % 4 - 1                             # -1, 0, 1, 2
    keys = np.zeros((T, D), dtype=np.int64)
    keys[np.arange(T), np.arange(T) % D] = a
    s = indexer.scores(q, w, keys)
    for t in range(T):
        d = t % D
        expect = sum(int(w[h]) * max(0, int(q[h, d]) * int(a[t])) for h in range(H))
        assert s[t] == expect


def test_scores_exact_at_workload_extremes():
    """Largest magnitude a workload can produce stays exact (integer path)."""
    w = synth.get("gqa_b32_8k")
    D, r = w.index_dim, w.index_range
    keys = np.full((3, D), r)
    keys[1] = -r
    s = indexer.scores(np.full((1, D), r), [1], keys)
    assert s.tolist() == [D * r * r, 0, D * r * r] and D * r * r < 2 ** 24


def test_scores_exact_at_multihead_extremes():
    """The 64-head workload: every head at the largest logit and the largest weight, and the
    signed case where the negative-weight heads alone fire.  The magnitude stays below 2^24, so
    an fp32 accumulation of these integers is exact in any order."""
    w = synth.get("mla_b64_32k_ih64")
    H, D, r = w.index_heads, w.index_dim, w.index_range
    q = np.full((H, D), r)
    q[1::2] = -r                                         # odd heads see the negated key
    wt = np.where(np.arange(H) % 2 == 0, 3, -2)
    keys = np.stack([np.full(D, r), np.full(D, -r)])
    s = indexer.scores(q, wt, keys)
    top = D * r * r
    assert s.tolist() == [3 * (H // 2) * top, -2 * (H // 2) * top]
    assert 3 * H * top < 2 ** 24


def test_bf16_decode_of_small_integers():
    """bf16 bit patterns of the integer range the workloads draw decode to those integers."""
    from oracle.bf16 import to_f64
    ints = np.arange(-8, 9, dtype=np.float32)
    assert np.array_equal(to_f64(synth.f32_to_bf16_bits(ints)), ints)
    # and a few non-integers whose bf16 value is known: 1.5, -0.375, 2**-10
    vals = np.array([1.5, -0.375, 2.0 ** -10], dtype=np.float32)
    assert np.array_equal(to_f64(synth.f32_to_bf16_bits(vals)), vals)


def test_scores_float_path():
    q = np.array([[0.5, -0.25]])
    keys = np.array([[1.0, 1.0], [-1.0, 0.0], [0.1, 0.3]])
    s = indexer.scores(q, [2.0], keys)
    assert s.dtype == np.float64
    np.testing.assert_allclose(s, [0.5, 0.0, 0.0], atol=0)


# ---------------------------------------------------------------- top-k

def _threshold_select(s, k):
    """Independent construction: find the k-th largest value v, keep every position
    scoring above v, then the lowest positions scoring exactly v until k are kept."""
    n = len(s)
    if n <= k:
        return list(range(n))
    v = sorted(s, reverse=True)[k - 1]
    above = [i for i in range(n) if s[i] > v]
    need = k - len(above)
    eq = [i for i in range(n) if s[i] == v][:need]
    return sorted(above + eq)


def test_dense_when_short():
    assert topk.select(np.array([5, 1, 9]), 3).tolist() == [0, 1, 2]
    assert topk.select(np.array([5, 1, 9]), 64).tolist() == [0, 1, 2]
    assert topk.select(np.array([]), 4).tolist() == []


def test_all_equal_takes_first_positions():
    assert topk.select(np.zeros(100), 7).tolist() == list(range(7))


def test_distinct_permutation():
    rng = np.random.default_rng(1)
    n, k = 1000, 37
    s = rng.permutation(n)
    assert topk.select(s, k).tolist() == np.flatnonzero(s >= n - k).tolist()


def test_descending_and_ascending():
    n, k = 50, 10
    assert topk.select(np.arange(n)[::-1], k).tolist() == list(range(k))
    assert topk.select(np.arange(n), k).tolist() == list(range(n - k, n))


@pytest.mark.parametrize("seed", range(12))
def test_ties_against_threshold_count(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    k = int(rng.integers(1, 120))
    m = int(rng.integers(1, 9))                     # few distinct values: many ties
    s = rng.integers(0, m, size=n)
    assert topk.select(s, k).tolist() == _threshold_select(s.tolist(), k)


def test_relu_zero_class_fills_by_position():
    """Tiny request 2 (96 tokens > k = 64) has fewer than 64 positive scores, so the rest of
    the selection is the lowest positions among the tokens whose ReLU clamped to 0."""
    w = synth.get("tiny_b5")
    qb = synth.index_queries(w, 0)
    kb, _, _ = synth.request_tokens(w, 0, 1, 96)
    s = indexer.scores_bf16(qb[1], synth.index_weights(w), kb)
    sel = topk.select(s, 64)
    pos = np.flatnonzero(s > 0)
    assert 0 < len(pos) < 64
    zeros = np.flatnonzero(s == 0)[: 64 - len(pos)]
    assert sel.tolist() == sorted(pos.tolist() + zeros.tolist())


def test_padded_layout():
    out = topk.select_padded(np.array([3, 1, 2]), 5)
    assert out.dtype == np.int32 and out.tolist() == [0, 1, 2, -1, -1]


def test_signed_zeros_tie_and_nan_ranks_last():
    """Worked by hand.  Scores by position: NaN, 1, -0, +0, NaN, -0, 2, NaN, -1.  Descending:
    2 (pos 6), 1 (pos 1), then the three zeros of either sign as one tie class by position
    (2, 3, 5), then -1 (pos 8), then the NaNs by position (0, 4, 7)."""
    s = np.array([np.nan, 1.0, -0.0, 0.0, np.nan, -0.0, 2.0, np.nan, -1.0], dtype=np.float32)
    assert topk.select(s, 3).tolist() == [1, 2, 6]          # 2, 1 and the first zero (pos 2)
    assert topk.select(s, 5).tolist() == [1, 2, 3, 5, 6]
    assert topk.select(s, 6).tolist() == [1, 2, 3, 5, 6, 8]
    assert topk.select(s, 7).tolist() == [0, 1, 2, 3, 5, 6, 8]
    assert topk.select(s, 8).tolist() == [0, 1, 2, 3, 4, 5, 6, 8]
