"""The benchmark's algorithmic byte and FLOP counts, against figures worked out by hand.

The roofline fractions the benchmark reports divide these counts by measured kernel times, so a
wrong term here (a dropped index write, V counted for a latent head whose values are the key
prefix, the wrong element size) would misstate every fraction.  The expected values below are
written out from the workloads' shapes: the indexer reads one bf16 key of D_I dims per cached token
and writes one fp32 score; the attention reads min(len, k) selected rows, the bf16 queries and the
int32 indices, and writes the fp32 outputs (GLM5.3 sparse-attention page, opening and
lightning-indexer paragraphs for what each step touches).
"""
import numpy as np

import bench
import synth


def test_latent_64x32k_counts():
    w = synth.get("mla_b64_32k")
    lens = synth.lens(w, 0)
    assert lens.tolist() == [32768] * 64
    ib, iflop, ab, aflop = bench.algorithmic_counts(w, lens)
    # 64 x 32,768 tokens x (128 dims x 2 B + 4 B score)
    assert ib == 64 * 32768 * 260 == 545_259_520
    assert iflop == 2 * 128 * 64 * 32768
    # 2,048 rows of 576 bf16 (values are the first 512 dims of the same row: no separate V),
    # 64 heads x 576 bf16 queries, 64 heads x 512 fp32 outputs, 2,048 int32 indices, per request
    rows = 64 * 2048 * 576 * 2
    assert rows == 150_994_944
    assert ab == rows + 64 * 64 * 576 * 2 + 64 * 64 * 512 * 4 + 64 * 2048 * 4 == 164_626_432
    # QK^T over 576 dims and PV over 512, 64 heads, per selected row
    assert aflop == 2 * 64 * 2048 * 64 * (576 + 512) == 18_253_611_008


def test_grouped_query_counts():
    w = synth.get("gqa_b32_8k")
    lens = synth.lens(w, 0)
    assert lens.min() > 512               # every request selects exactly k = 512 rows
    ib, _, ab, aflop = bench.algorithmic_counts(w, lens)
    assert ib == int(lens.sum()) * (64 * 2 + 4)
    # K and V stored apart: 4 KV heads x 128 dims x 2 B each, per selected row
    assert ab == 32 * 512 * (4 * 128 * 2 * 2) + 32 * 32 * 128 * 2 + 32 * 32 * 128 * 4 + 32 * 512 * 4
    assert aflop == 2 * 32 * 512 * 32 * (128 + 128)


def test_tiny_counts_with_dense_request():
    w = synth.get("tiny_b5")
    lens = synth.lens(w, 0)
    assert lens.tolist() == [403, 96, 241, 30, 176]
    ib, _, ab, _ = bench.algorithmic_counts(w, lens)
    # 946 tokens x (32 dims x 2 B + 4 B)
    assert ib == 946 * 68
    # the 30-token request attends to all 30 of its tokens (len <= k), the others to k = 64;
    # the index array is k wide for every request
    n_sel = 64 + 64 + 64 + 30 + 64
    assert ab == n_sel * (64 * 2 + 64 * 2) + 5 * 8 * 64 * 2 + 5 * 8 * 64 * 4 + 5 * 64 * 4 == 89_856


def test_counts_scale_with_length():
    w = synth.get("mla_b64_32k")
    a = bench.algorithmic_counts(w, np.array([4096, 100]))
    b = bench.algorithmic_counts(w, np.array([4096, 100, 0]))
    # an empty request adds its queries, outputs and index row but no keys or selected rows
    assert b[0] == a[0]
    assert b[2] - a[2] == 64 * 576 * 2 + 64 * 512 * 4 + 2048 * 4
