"""GPU tests of the tiered KV cache (HBM cache with LRU eviction over pinned host memory), with
whole pages and with single token rows as the unit.

A scaled tiered workload (4 requests x 4096 tokens x 8 layers, page 64, 16 query / 2 KV heads,
d = 128, top-256 seeded locality-biased positions, cache = a quarter of all pages' bytes) runs
two decode steps layer by layer: plan on the host, fetch on a side stream, attention on the
main stream after the fetch, release of the layer before.  Checked, for each unit:
  * slot tables, hits, misses and evictions equal the oracle's LRU under the same sequence;
  * attention through the cache is bit-identical to attention over a pool holding every page
    (tier on vs off);
  * sampled (layer, request) outputs match the float64 oracle within 2e-3 normwise.
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


def _run_tier(tsa, st, steps):
    """Plan / fetch / attend / release over `steps` x layers; returns per-layer outputs, slot
    tables and positions."""
    NL, R = st.w.num_layers, st.num_req
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    table_dev = [torch.empty((R, st.pages_per_req), dtype=torch.int32, device="cuda") for _ in range(2)]
    fetched = [torch.cuda.Event() for _ in range(2)]
    done = {}
    outs, tables, positions = [], [], []
    centres = {}
    g = 0
    for step in range(steps):
        for layer in range(NL):
            pos = st.positions(step, layer, centres)
            table, _ = st.tier.plan(layer, g, pos)
            # eviction may reuse slots of layers released so far: their attention must be done
            if g - 2 in done:
                side.wait_event(done[g - 2])
            st.tier.fetch(table_dev[g & 1], stream=side)
            fetched[g & 1].record(side)
            main.wait_event(fetched[g & 1])
            topk = torch.from_numpy(pos).cuda()
            out = torch.empty((R, st.w.num_q_heads, st.w.head_dim_v), dtype=torch.float32, device="cuda")
            st.attend(table_dev[g & 1], topk, out)
            ev = torch.cuda.Event()
            ev.record(main)
            done[g] = ev
            if g > 0:
                st.tier.release(g - 1)
            outs.append(out)
            tables.append(table)
            positions.append(pos)
            g += 1
    torch.cuda.synchronize()
    return outs, tables, positions


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
    oc = lru.LRUCache(st.cache.desc.num_pages)
    for g, pos in enumerate(positions):
        layer = g % st.w.num_layers
        ref = lru.plan_layer(oc, layer, st.num_req, st.pages_per_req, pos, st.cache.desc.page_size, g)
        assert np.array_equal(tables[g], ref), g
        if g > 0:
            oc.release(g - 1)
    s = st.tier.stats()
    assert (s["hits"], s["misses"], s["evictions"]) == (oc.hits, oc.misses, oc.evictions)
    assert s["misses"] > 0 and s["evictions"] > 0
    page_bytes = st.cache.desc.page_size * st.w.num_kv_heads * st.w.head_dim_k * 2
    assert s["h2d_bytes"] == 2 * page_bytes * s["misses"]
    print(f"tier: hits {s['hits']} misses {s['misses']} evictions {s['evictions']} "
          f"hit rate {s['hits'] / (s['hits'] + s['misses']):.3f}")


def test_tier_on_equals_tier_off(tsa, tier_run):
    """Attention through the cache equals attention over a pool that holds every page."""
    st, outs, tables, positions = tier_run
    w = st.w
    keys = w.num_layers * st.num_req * st.pages_per_req
    full = tsa.KvPool(keys, st.cache.desc.page_size, w.num_kv_heads, w.head_dim_k, w.head_dim_v)
    full.k.copy_(st.host_k.view(-1).cuda())
    full.v.copy_(st.host_v.view(-1).cuda())
    ws = torch.empty(max(tsa.workspace_bytes(full, st.params), 256), dtype=torch.uint8, device="cuda")
    for g, pos in enumerate(positions):
        layer = g % w.num_layers
        ftab = np.array([[st.key(layer, r, p) for p in range(st.pages_per_req)] for r in range(st.num_req)],
                        dtype=np.int32)
        out = torch.empty_like(outs[g])
        tsa.sparse_attn_gather(full, 0, st.params, st.q, torch.from_numpy(pos).cuda(),
                               torch.from_numpy(ftab).cuda(), st.lens_dev, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, outs[g]), f"layer step {g}"


def test_tier_outputs_match_oracle(tier_run):
    st, outs, tables, positions = tier_run
    w = st.w
    q = synth.queries(w, st.seed)
    worst = 0.0
    for g, r in [(0, 0), (5, 3), (8, 1), (15, 2)]:
        layer = g % w.num_layers
        _, kk, vv = synth.request_tokens(w, st.seed, r, st.length, layer=layer)
        ref = decode.attend_positions(q[r], kk, vv, positions[g][r], w.sm_scale)
        err = sdpa.normwise_rel_err(outs[g][r].double().cpu().numpy(), ref)
        assert err < ATOL_REL, (g, r, err)
        worst = max(worst, err)
    print(f"tier: max normwise error {worst:.2e}")
