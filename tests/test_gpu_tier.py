"""GPU tests of the tiered KV cache (HBM cache with LRU eviction over pinned host memory), with
whole pages and with single token rows as the unit.

GLM5.3 sparse-attention page, HiSparse paragraph: the KV cache lives in host memory, HBM holds an
LRU cache of it, selections that miss are loaded from host memory, and the loads for layer N
overlap the computation of layer N-1.

Two shapes, each run layer by layer for two decode steps (plan on the host, fetch on a side
stream, attention on the main stream after the fetch, the layer before released with the event
recorded after its attention):
  * a scaled tiered workload (4 requests x 4,096 tokens x 8 layers, page 64, 16 query / 2 KV heads,
    d = 128, top-256 seeded locality-biased positions, cache = a quarter of all pages' bytes);
  * the tiered configuration's own per-request shape (65,536 tokens x 8 layers x top-2,048,
    page 64, cache = a quarter of the pages) at 8 requests: 4 GiB of pinned host copy per cache
    unit, which keeps the test within a couple of minutes; the benchmark runs all 256 requests.
Checked, for each unit:
  * slot tables, hits, misses and evictions equal the oracle's LRU under the same sequence;
  * attention through the cache is bit-identical to attention over a pool holding every page
    (tier on vs off);
  * sampled (layer, request) outputs match the float64 oracle within 2e-3 normwise.
And the ordering the library provides: with the main stream or the side stream held up by a long
matrix product, every output still equals the tier-off one (a copy never overwrites a slot an
attention has yet to read, and an attention never reads a slot whose copy is in flight).
"""
import numpy as np
import pytest

import synth
from oracle import decode, lru, sdpa

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL_REL = 2e-3


@pytest.fixture(scope="module")
def tsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_sparse_attention_amd as m
    m.load()
    return m


def _slow(stream):
    """About 20 ms of matrix products on `stream` (holds back what is queued after it)."""
    with torch.cuda.stream(stream):
        a = torch.randn((4096, 4096), device="cuda")
        for _ in range(24):
            a = torch.mm(a, a) * 1e-3
    return a


def _run_tier(tsa, st, steps, prefetch=False, slow_main=None, slow_side=None):
    """Plan / fetch / attend / release over `steps` x layers; returns per-layer outputs, slot
    tables (host tables from the plan, or None with `prefetch`) and positions.  slow_main /
    slow_side: layer-step indices before whose attention / fetch a long matrix product is
    queued on that stream."""
    NL, R = st.w.num_layers, st.num_req
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    table_dev = [torch.empty((R, st.pages_per_req), dtype=torch.int32, device="cuda") for _ in range(2)]
    fetched = [torch.cuda.Event() for _ in range(2)]
    done = {}
    keep = []
    outs, tables, positions = [], [], []
    centres = {}
    g = 0
    for step in range(steps):
        for layer in range(NL):
            pos = st.positions(step, layer, centres)
            if g == slow_side:
                keep.append(_slow(side))
            if prefetch:
                st.tier.prefetch(layer, g, pos, table_dev[g & 1], stream=side, fetched=fetched[g & 1])
                table = None
            else:
                table, _ = st.tier.plan(layer, g, pos)
                st.tier.fetch(table_dev[g & 1], stream=side)
                fetched[g & 1].record(side)
            main.wait_event(fetched[g & 1])
            if g == slow_main:
                keep.append(_slow(main))
            topk = torch.from_numpy(pos).cuda()
            out = torch.empty((R, st.w.num_q_heads, st.w.head_dim_v), dtype=torch.float32, device="cuda")
            st.attend(table_dev[g & 1], topk, out)
            ev = torch.cuda.Event()
            ev.record(main)
            done[g] = ev
            if g > 0:
                # tag g-1's slots become evictable now; later copies wait for its attention
                st.tier.release_layer(g - 1, done[g - 1])
            outs.append(out)
            tables.append(table)
            positions.append(pos)
            g += 1
    torch.cuda.synchronize()
    return outs, tables, positions


def _bookkeeping(st, tables, positions, table_dev_reads=None):
    """Replays the plans on the oracle's LRU; compares slot tables (host tables, or the touched
    entries of the device tables read back after each layer) and the counters."""
    oc = lru.LRUCache(st.cache.desc.num_pages)
    for g, pos in enumerate(positions):
        layer = g % st.w.num_layers
        ref = lru.plan_layer(oc, layer, st.num_req, st.pages_per_req, pos, st.cache.desc.page_size, g)
        if tables[g] is not None:
            assert np.array_equal(tables[g], ref), g
        if table_dev_reads is not None:
            got = table_dev_reads[g]
            touched = ref >= 0
            assert np.array_equal(got[touched], ref[touched]), g
        if g > 0:
            oc.release(g - 1)
    s = st.tier.stats()
    assert (s["hits"], s["misses"], s["evictions"]) == (oc.hits, oc.misses, oc.evictions)
    page_bytes = st.cache.desc.page_size * st.w.num_kv_heads * st.w.head_dim_k * 2
    assert s["h2d_bytes"] == 2 * page_bytes * s["misses"]
    return s


def _tier_off(tsa, st, outs, positions):
    """Attention over a pool that holds every page equals attention through the cache."""
    w = st.w
    keys = w.num_layers * st.num_req * st.pages_per_req
    full = tsa.KvPool(keys, st.cache.desc.page_size, w.num_kv_heads, w.head_dim_k, w.head_dim_v)
    full.k.copy_(st.host_k.view(-1).cuda())
    full.v.copy_(st.host_v.view(-1).cuda())
    ws = torch.empty(max(tsa.workspace_bytes(full, st.params), 256), dtype=torch.uint8, device="cuda")
    for g, pos in enumerate(positions):
        layer = g % w.num_layers
        ftab = (np.arange(st.num_req, dtype=np.int64)[:, None] + layer * st.num_req) * st.pages_per_req \
            + np.arange(st.pages_per_req, dtype=np.int64)[None, :]
        out = torch.empty_like(outs[g])
        tsa.sparse_attn_gather(full, 0, st.params, st.q, torch.from_numpy(pos).cuda(),
                               torch.from_numpy(ftab.astype(np.int32)).cuda(), st.lens_dev, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, outs[g]), f"layer step {g}"
    del full


def _oracle_sampled(st, outs, positions, picks):
    w = st.w
    q = synth.queries(w, st.seed)
    worst = 0.0
    for g, r in picks:
        layer = g % w.num_layers
        _, kk, vv = synth.request_tokens(w, st.seed, r, st.length, layer=layer)
        ref = decode.attend_positions(q[r], kk, vv, positions[g][r], w.sm_scale)
        err = sdpa.normwise_rel_err(outs[g][r].double().cpu().numpy(), ref)
        assert err < ATOL_REL, (g, r, err)
        worst = max(worst, err)
    return worst


# ------------------------------------------------------------------ scaled tiered workload

@pytest.fixture(scope="module", params=["page", "token"])
def tier_run(tsa, request):
    from top_sparse_attention_amd import workload
    w = synth.get("tiered_b256_64k")
    # token unit: a cache of 48 pages' bytes (3,072 token slots) so that 2 steps x 8 layers x
    # 1,024 touched tokens also evict
    cache_pages = 48 if request.param == "token" else None
    st = workload.stage_tier(w, seed=0, num_req=4, length=4096, num_layers=8, top_k=256,
                             cache_pages=cache_pages, unit=request.param)
    outs, tables, positions = _run_tier(tsa, st, steps=2)
    return st, outs, tables, positions


def test_tier_bookkeeping_matches_oracle(tier_run):
    st, outs, tables, positions = tier_run
    s = _bookkeeping(st, tables, positions)
    assert s["misses"] > 0 and s["evictions"] > 0
    print(f"tier: hits {s['hits']} misses {s['misses']} evictions {s['evictions']} "
          f"hit rate {s['hits'] / (s['hits'] + s['misses']):.3f}")


def test_tier_on_equals_tier_off(tsa, tier_run):
    st, outs, tables, positions = tier_run
    _tier_off(tsa, st, outs, positions)


def test_tier_outputs_match_oracle(tier_run):
    st, outs, tables, positions = tier_run
    worst = _oracle_sampled(st, outs, positions, [(0, 0), (5, 3), (8, 1), (15, 2)])
    print(f"tier: max normwise error {worst:.2e}")


@pytest.fixture(scope="module", params=["page", "token"])
def tier_merge_run(tsa, request):
    """32 requests x 2 KV heads: 64 (request, KV head) pairs, so the attention through the cache
    runs the grouped-query kernel with the four splits of each pair merged in one workgroup."""
    from top_sparse_attention_amd import workload
    w = synth.get("tiered_b256_64k")
    # whole pages: a layer's plan pins nearly every page of these short contexts, so the cache
    # holds all of them; token rows: the default quarter, with evictions
    cache_pages = 2 * 32 * (2048 // w.page_size) if request.param == "page" else None
    st = workload.stage_tier(w, seed=1, num_req=32, length=2048, num_layers=2, top_k=256,
                             cache_pages=cache_pages, unit=request.param)
    outs, tables, positions = _run_tier(tsa, st, steps=2)
    return st, outs, tables, positions


def test_tier_with_merged_splits(tsa, tier_merge_run):
    """Bookkeeping equal to the oracle's LRU, outputs through the cache bit-identical to a pool
    holding every page, and sampled outputs within the bar of the fp64 oracle."""
    st, outs, tables, positions = tier_merge_run
    _bookkeeping(st, tables, positions)
    _tier_off(tsa, st, outs, positions)
    worst = _oracle_sampled(st, outs, positions, [(0, 0), (1, 31), (2, 17), (3, 5)])
    print(f"tier, 32 requests: max normwise error {worst:.2e}")


def test_tier_prefetch_equals_plan_and_fetch(tsa, tier_run):
    """tsa_lru_prefetch (plan + ordered fetch + fetched event in one call) gives the same outputs
    and counters as separate plan and fetch calls on a fresh tier over the same host copy."""
    from top_sparse_attention_amd import KvPool, LruTier
    st, outs, tables, positions = tier_run
    d = st.cache.desc
    cache = KvPool(d.num_pages, d.page_size, d.num_kv_heads, d.head_dim_k, d.head_dim_v)
    st2 = type(st)(**{**st.__dict__, "cache": cache,
                      "tier": LruTier(cache, st.w.num_layers, st.num_req, st.pages_per_req,
                                      st.host_k, st.host_v)})
    outs2, _, positions2 = _run_tier(tsa, st2, steps=2, prefetch=True)
    for g in range(len(outs)):
        assert np.array_equal(positions[g], positions2[g])
        assert torch.equal(outs[g], outs2[g]), g
    assert st2.tier.stats() == st.tier.stats()


def test_tier_ordering_under_held_streams(tsa):
    """The library orders the two streams itself: with the main stream held up before one
    layer's attention (so that later copies would overwrite its slots first) and the side stream
    held up before another layer's fetch (so that its attention would read slots still being
    copied), every output equals the tier-off output.  The cache holds a little over two
    layers' pages, so each plan evicts the slots of the layer released before it."""
    from top_sparse_attention_amd import workload
    w = synth.get("tiered_b256_64k")
    st = workload.stage_tier(w, seed=3, num_req=4, length=4096, num_layers=8, top_k=256,
                             cache_pages=600, unit="page")
    outs, tables, positions = _run_tier(tsa, st, steps=2, slow_main=5, slow_side=9)
    # the plan two layers after the held attention reused slots that attention read
    reused = set(tables[5][tables[5] >= 0].tolist()) & set(tables[7][tables[7] >= 0].tolist())
    assert reused, "the case does not reuse the held layer's slots"
    _bookkeeping(st, tables, positions)
    _tier_off(tsa, st, outs, positions)


# ------------------------------------------------------------------ the configuration's request shape

@pytest.fixture(scope="module", params=["page", "token"])
def tier_c5(tsa, request):
    """8 requests of the tiered configuration's shape: 65,536 tokens, 8 layers, top-2,048, cache
    of a quarter of the pages; two decode steps through tsa_lru_prefetch, device tables read back
    after every layer."""
    from top_sparse_attention_amd import workload
    w = synth.get("tiered_b256_64k")
    print(f"[tier c5] staging 8 x 65536 x 8 layers, unit {request.param}", flush=True)
    st = workload.stage_tier(w, seed=0, num_req=8, unit=request.param)
    assert st.length == 65536 and st.w.num_layers == 8 and st.w.top_k == 2048
    NL, R = st.w.num_layers, st.num_req
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    table_dev = [torch.full((R, st.pages_per_req), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    fetched = [torch.cuda.Event() for _ in range(2)]
    done = {}
    outs, reads, positions = [], [], []
    centres = {}
    g = 0
    for step in range(2):
        for layer in range(NL):
            pos = st.positions(step, layer, centres)
            st.tier.prefetch(layer, g, pos, table_dev[g & 1], stream=side, fetched=fetched[g & 1])
            main.wait_event(fetched[g & 1])
            out = torch.empty((R, st.w.num_q_heads, st.w.head_dim_v), dtype=torch.float32, device="cuda")
            st.attend(table_dev[g & 1], torch.from_numpy(pos).cuda(), out)
            reads.append(table_dev[g & 1].cpu().numpy())     # synchronizes main (after the fetch)
            ev = torch.cuda.Event()
            ev.record(main)
            done[g] = ev
            if g > 0:
                st.tier.release_layer(g - 1, done[g - 1])
            outs.append(out)
            positions.append(pos)
            g += 1
    torch.cuda.synchronize()
    print(f"[tier c5] ran, stats {st.tier.stats()}", flush=True)
    return st, outs, reads, positions


def test_tier_c5_bookkeeping_matches_oracle(tier_c5):
    st, outs, reads, positions = tier_c5
    s = _bookkeeping(st, [None] * len(positions), positions, table_dev_reads=reads)
    assert s["misses"] > 0
    print(f"tier c5: hits {s['hits']} misses {s['misses']} evictions {s['evictions']} "
          f"hit rate {s['hits'] / (s['hits'] + s['misses']):.3f}")


def test_tier_c5_on_equals_tier_off(tsa, tier_c5):
    st, outs, reads, positions = tier_c5
    _tier_off(tsa, st, outs, positions)


def test_tier_c5_outputs_match_oracle(tier_c5):
    st, outs, reads, positions = tier_c5
    worst = _oracle_sampled(st, outs, positions, [(0, 0), (3, 7), (7, 2), (8, 5), (12, 1), (15, 6)])
    print(f"tier c5: max normwise error {worst:.2e}")
