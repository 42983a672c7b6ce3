"""The seeded input generators: deterministic, sliceable, and shaped as each workload states."""
import numpy as np

import synth


def test_bf16_rounding_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -2.5], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert b.tolist() == [0x3F80, 0x3F82, 0x3F80, 0xC020]


def test_deterministic_and_sliceable():
    w = synth.get("gqa_b32_8k")
    L = int(synth.lens(w)[3])
    a = synth.request_tokens(w, 0, 3, L)
    b = synth.request_tokens(w, 0, 3, L, start=100, stop=700)
    for full, part in zip(a, b):
        assert np.array_equal(full[100:700], part)
    c = synth.request_tokens(w, 1, 3, L)
    assert not np.array_equal(a[1], c[1])


def test_shapes_and_ranges():
    for name in ["tiny_b5", "gqa_b32_8k", "prefix_b128_16k"]:
        w = synth.get(name)
        lens = synth.lens(w)
        assert lens.shape == (w.batch,)
        kidx, k, v = synth.request_tokens(w, 0, 0, int(lens[0]), start=0, stop=50)
        assert kidx.shape == (50, w.index_dim) and k.shape == (50, w.num_kv_heads, w.head_dim_k)
        assert v.shape == (50, w.num_kv_heads, w.head_dim_v)
        qi = synth.index_queries(w)
        assert qi.shape == (w.batch, w.index_heads, w.index_dim)
    w = synth.get("gqa_b32_8k")
    assert synth.lens(w).min() >= 2048 and synth.lens(w).max() <= 8192
    assert sorted(synth.free_order(w).tolist()) == list(range(w.pool_pages))
    assert synth.free_order(synth.get("tiny_b5")).tolist() == list(range(66))


def test_prefix_is_shared():
    w = synth.get("prefix_b128_16k")
    lens = synth.lens(w)
    assert (lens >= 16384 + 1024).all() and (lens <= 16384 + 4096).all()
    a = synth.request_tokens(w, 0, 0, int(lens[0]), start=16000, stop=16500)
    b = synth.request_tokens(w, 0, 7, int(lens[7]), start=16000, stop=16500)
    for x, y in zip(a, b):
        assert np.array_equal(x[:384], y[:384])          # positions below 16384 are shared
        assert not np.array_equal(x[384:], y[384:])      # the suffixes differ


def test_tier_positions_are_distinct_sorted():
    w = synth.get("tiered_b256_64k")
    pos, centres = synth.tier_positions(w, 0, 0, 0, 0)
    assert pos.shape == (2048,) and (np.diff(pos) > 0).all()
    assert pos.min() >= 0 and pos.max() < 65536
    pos2, _ = synth.tier_positions(w, 0, 1, 0, 0, centres)
    assert not np.array_equal(pos, pos2)


def test_multihead_indexer_inputs():
    w = synth.get("mla_b64_32k_ih64")
    q, wt = synth.index_queries(w), synth.index_weights(w)
    assert q.shape == (64, 64, 128) and wt.shape == (64,)
    assert set(np.unique(wt).tolist()) <= set(range(-2, 4))
    assert (wt < 0).any() and (wt > 0).any()            # signed weights
    q2, w2 = synth.index_inputs(w, 0, 64, 8)            # the workload's own heads: a slice
    assert np.array_equal(q2, q[:8]) and np.array_equal(w2, wt)
    q3, w3 = synth.index_inputs(synth.get("gqa_b32_8k"), 0, 17, 40)
    assert q3.shape == (40, 17, 64) and w3.shape == (17,)
    assert np.array_equal(synth.index_weights(synth.get("gqa_b32_8k")), [1.0])


def test_queries_of_a_larger_batch_extend_the_default_draw():
    """Staging more requests than a workload lists draws more query rows; the first rows stay."""
    w = synth.get("gqa_b32_8k")
    q = synth.queries(w, 0)
    q2 = synth.queries(w, 0, 3 * w.batch)
    assert q2.shape == (3 * w.batch, w.num_q_heads, w.head_dim_k)
    assert np.array_equal(q2[:w.batch], q)
    assert np.array_equal(synth.queries(w, 0, 5), q[:5])
