"""Pins of the oracle's sparse SDPA, its decode chain, the LRU model and the roofline formula.

SDPA: pinned against torch's own scaled_dot_product_attention (a library routine,
CPU, float64) in the dense case the GLM5.3 sparse-attention page names (context of
at most K tokens), including its grouped-query mode, and against special cases
with exact answers.  LRU: the state-snapshot page's sequential-scan cliff and the
uniform-access hit rate.  Roofline: the GLM5.3 page's printed intensities.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import decode, lru, roofline, sdpa
from oracle.bf16 import to_f64


def _torch_sdpa(q, k, v, scale):
    """q [Hq, dk], k [n, Hkv, dk], v [n, Hkv, dv] -> [Hq, dv] via torch (CPU fp64)."""
    tq = torch.from_numpy(q)[None, :, None, :]                 # [1, Hq, 1, dk]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]   # [1, Hkv, n, dk]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, enable_gqa=q.shape[0] != k.shape[1])
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,n,dk,dv", [(8, 1, 30, 64, 64), (32, 4, 50, 128, 128),
                                           (4, 4, 17, 16, 8), (64, 1, 40, 576, 512)])
def test_dense_matches_torch_sdpa(hq, hkv, n, dk, dv):
    rng = np.random.default_rng(hq * 1000 + n)
    q = rng.standard_normal((hq, dk))
    k = rng.standard_normal((n, hkv, dk))
    v = rng.standard_normal((n, hkv, dv))
    scale = 1 / math.sqrt(dk)
    np.testing.assert_allclose(sdpa.attend(q, k, v, scale), _torch_sdpa(q, k, v, scale),
                               rtol=1e-12, atol=1e-12)


def test_single_token_returns_value_row():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((8, 64))
    k = rng.standard_normal((1, 2, 64))
    v = rng.standard_normal((1, 2, 32))
    o = sdpa.attend(q, k, v, 0.125)
    assert np.array_equal(o[:4], np.repeat(v[0, 0][None], 4, 0))
    assert np.array_equal(o[4:], np.repeat(v[0, 1][None], 4, 0))


def test_equal_logits_give_mean():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((9, 1, 16))
    v = rng.standard_normal((9, 1, 8))
    o = sdpa.attend(np.zeros((3, 16)), k, v, 1.0)
    np.testing.assert_allclose(o, np.repeat(v[:, 0].mean(0)[None], 3, 0), rtol=1e-14)


def test_weights_are_convex():
    """Outputs lie inside the hull of the value rows: with one-hot value rows the output
    row is the softmax itself (non-negative, sums to one, ordered like the logits)."""
    n = 6
    v = np.eye(n)[:, None, :]
    k = np.arange(n, dtype=float)[:, None, None] * np.ones((n, 1, 3))
    o = sdpa.attend(np.ones((1, 3)), k, v, 0.5)[0]
    assert abs(o.sum() - 1) < 1e-14 and (np.diff(o) > 0).all()
    np.testing.assert_allclose(o, np.exp(1.5 * np.arange(n)) / np.exp(1.5 * np.arange(n)).sum())


def test_empty_selection():
    assert not sdpa.attend(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 3)), 1.0).any()


def test_normwise_error_metric():
    ref = np.array([[1.0, -4.0, 0.0], [0.0, 0.0, 0.0]])
    o = ref + np.array([[0.0, 0.004, 0.0], [0.0, 0.0, 0.0]])
    assert sdpa.normwise_rel_err(o, ref) == pytest.approx(0.001)


def test_tiny_dense_request_matches_torch():
    """Tiny request 4 has 30 tokens <= k = 64: the sparse step is plain dense SDPA."""
    w = synth.get("tiny_b5")
    L = int(synth.lens(w)[3])
    assert L == 30
    kb, kk, vv = synth.request_tokens(w, 0, 3, L)
    qb = synth.queries(w, 0)[3]
    s, sel, o = decode.request_step(qb, synth.index_queries(w, 0)[3], synth.index_weights(w),
                                    kb, kk, vv, w.top_k, w.sm_scale)
    assert sel.tolist() == list(range(30))
    ref = _torch_sdpa(to_f64(qb), to_f64(kk), to_f64(vv), w.sm_scale)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_mqa_values_are_key_prefix():
    """MLA in MQA mode: values are the first 512 dims of the 576-dim latent key row."""
    w = synth.get("mla_b64_32k")
    rng = np.random.default_rng(5)
    kbits = synth.f32_to_bf16_bits(rng.standard_normal((40, 1, 576)).astype(np.float32))
    qbits = synth.f32_to_bf16_bits(rng.standard_normal((64, 576)).astype(np.float32))
    sel = np.arange(0, 40, 3)
    o = decode.attend_positions(qbits, kbits, None, sel, w.sm_scale, v_from_k_dims=512)
    kf = to_f64(kbits[sel])
    ref = _torch_sdpa(to_f64(qbits), kf, np.ascontiguousarray(kf[:, :, :512]), w.sm_scale)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- LRU

def test_lru_sequential_scan_is_a_cliff():
    """256 slots, 500 items sent twice in the same order: strict LRU reuses nothing."""
    c = lru.LRUCache(256)
    for i in range(500):
        c.touch(i)
    c.hits = c.misses = 0
    for i in range(500):
        c.touch(i)
    assert c.hits == 0 and c.misses == 500


def test_lru_uniform_access_hit_rate():
    """Independent uniform access over N items with C slots hits C/N of the time: 256/500
    = 51.2%, the page's "about 51%" for random order."""
    rng = np.random.default_rng(0)
    c = lru.LRUCache(256)
    for i in rng.integers(0, 500, size=5000):
        c.touch(int(i))
    c.hits = c.misses = 0
    for i in rng.integers(0, 500, size=200000):
        c.touch(int(i))
    assert abs(c.hit_rate - 0.512) < 0.006


def test_lru_fits_means_cold_misses_only():
    rng = np.random.default_rng(2)
    c = lru.LRUCache(100)
    keys = rng.integers(0, 100, size=3000)
    for x in keys:
        c.touch(int(x))
    assert c.misses == len(set(keys.tolist())) and c.hits + c.misses == 3000
    assert c.evictions == 0


def test_lru_eviction_order_and_pins():
    c = lru.LRUCache(3)
    for x in "abc":
        c.touch(x)
    c.touch("a")                 # order now b, c, a
    c.touch("d")                 # evicts b
    assert set(c.slots) == {"c", "a", "d"} and c.evictions == 1
    c.touch("c", tag=1)          # pin c
    c.touch("e")                 # c is least recent but pinned: a goes
    assert set(c.slots) == {"c", "d", "e"}
    c.touch("d", tag=1)
    c.touch("e", tag=1)
    with pytest.raises(MemoryError):
        c.touch("f")
    c.release(1)
    c.touch("f")
    assert "f" in c.slots


def test_lru_slot_reuse():
    c = lru.LRUCache(2)
    s0, _ = c.touch("x")
    s1, _ = c.touch("y")
    s2, _ = c.touch("z")         # evicts x, takes its slot
    assert (s0, s1, s2) == (0, 1, 0)


def test_pages_of_positions():
    assert lru.pages_of_positions([0, 63, 64, 130, -1, 5], 64) == [0, 1, 2]


# ---------------------------------------------------------------- roofline

def test_mla_intensity_printed_values():
    """GLM-5 shape (d=512, r=64, b=2, H=64) gives 120.8 FLOP/B (printed truncated);
    258.2 FLOP/B solved for H gives roughly 128 heads."""
    ai = roofline.mqa_intensity(512, 64, 64, 2)
    assert math.floor(ai * 10) / 10 == 120.8
    assert roofline.mqa_flops(1000, 512, 64, 64) / roofline.mqa_bytes(1000, 512, 64, 2) == pytest.approx(ai)
    h = roofline.heads_for_intensity(258.2, 512, 64, 2)
    assert 120 < h < 140
    assert roofline.mqa_intensity(512, 64, 128, 2) == pytest.approx(2 * ai)
