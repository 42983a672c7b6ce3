"""Hand-worked pin of the tiered cache's per-layer plan (oracle.lru.plan_layer) and the same
sequence through the library's tier (bookkeeping only, no GPU).

GLM5.3 sparse-attention page, HiSparse paragraph: the HBM part of the KV cache is an LRU cache,
a selection that misses loads the page from host memory and evicts the least recently used one,
and layer N's loads overlap layer N-1's compute (so two layers' pages are in flight).  The plan
policy is the library's reading (the page fixes no order): requests ascending, each request's
distinct pages ascending, key = (layer * num_req + req) * pages_per_req + page, free slots taken
lowest first, pages of unreleased plans pinned.

The case, worked by hand: 2 layers x 2 requests x 3 pages of 4 tokens, 5 cache slots, plans
tagged 0..3 with each tag released after the next plan (the flow of a decode step).

  plan 0 (layer 0): req 0 positions 1, 5   -> pages 0, 1 -> keys 0, 1 -> miss, miss: slots 0, 1
                    req 1 position 9       -> page 2     -> key 5     -> miss: slot 2
  plan 1 (layer 1): req 0 positions 0, 11  -> pages 0, 2 -> keys 6, 8 -> miss, miss: slots 3, 4
                    req 1 (nothing)
  release 0         (keys 0, 1, 5 become evictable)
  plan 2 (layer 0): req 0 positions 2, 10  -> pages 0, 2 -> key 0 hit (slot 0); key 2 misses
                    with no free slot: least recent unpinned of 1, 5 (0 is pinned by plan 2
                    now, 6 and 8 by plan 1) is key 1 -> slot 1, one eviction
                    req 1 position 8       -> page 2     -> key 5 hit (slot 2)
  release 1         (keys 6, 8 become evictable)
  plan 3 (layer 1): req 0 (nothing)
                    req 1 positions 1, 5   -> pages 0, 1 -> keys 9, 10 -> misses; unpinned in
                    recency order are 6 then 8 -> slots 3, 4, two evictions

  totals: 2 hits, 8 misses, 3 evictions.
"""
import numpy as np
import pytest

from oracle import lru

P, NUM_LAYERS, NUM_REQ, PPR, CAPACITY = 4, 2, 2, 3, 5

PLANS = [   # (layer, positions per request; -1 pads)
    (0, [[1, 5], [9, -1]]),
    (1, [[0, 11], [-1, -1]]),
    (0, [[2, 10], [8, -1]]),
    (1, [[-1, -1], [1, 5]]),
]
TABLES = [
    [[0, 1, -1], [-1, -1, 2]],
    [[3, -1, 4], [-1, -1, -1]],
    [[0, -1, 1], [-1, -1, 2]],
    [[-1, -1, -1], [3, 4, -1]],
]
HITS, MISSES, EVICTIONS = 2, 8, 3


def test_plan_layer_by_hand():
    cache = lru.LRUCache(CAPACITY)
    for tag, (layer, pos) in enumerate(PLANS):
        table = lru.plan_layer(cache, layer, NUM_REQ, PPR, np.array(pos), P, tag)
        assert table.tolist() == TABLES[tag], f"plan {tag}"
        if tag > 0:
            cache.release(tag - 1)
    assert (cache.hits, cache.misses, cache.evictions) == (HITS, MISSES, EVICTIONS)


def test_plan_layer_keys_by_hand():
    """The keys each plan pins, and the recency order (least recent first) after the last."""
    cache = lru.LRUCache(CAPACITY)
    pinned = []
    for tag, (layer, pos) in enumerate(PLANS):
        lru.plan_layer(cache, layer, NUM_REQ, PPR, np.array(pos), P, tag)
        pinned.append(sorted(cache.pins[tag]))
        if tag > 0:
            cache.release(tag - 1)
    assert pinned == [[0, 1, 5], [6, 8], [0, 2, 5], [9, 10]]
    assert list(cache.slots) == [0, 2, 5, 9, 10]


def test_library_tier_plan_by_hand():
    """The library's tier (host bookkeeping through the C ABI) on the same sequence."""
    tsa = pytest.importorskip("top_sparse_attention_amd")
    from top_sparse_attention_amd import _lib
    try:
        _lib.load()
    except ImportError:
        pytest.skip("libtsa.so not built")
    cache = tsa.KvPool(CAPACITY, P, 1, 8, 8, allocate=False)
    tier = tsa.LruTier(cache, NUM_LAYERS, NUM_REQ, PPR)
    for tag, (layer, pos) in enumerate(PLANS):
        table, _ = tier.plan(layer, tag, np.array(pos, dtype=np.int32))
        assert table.tolist() == TABLES[tag], f"plan {tag}"
        if tag > 0:
            tier.release(tag - 1)
    st = tier.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (HITS, MISSES, EVICTIONS)
