"""libtsa host-side tests (no GPU): exported symbols, page tables against the oracle, refcounts,
error codes.  The pool here is metadata-only (no device memory), so nothing is launched."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth
from oracle import paging

tsa = pytest.importorskip("top_sparse_attention_amd")
from top_sparse_attention_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _have_lib():
    try:
        _lib.load()
        return True
    except ImportError:
        return False


pytestmark = pytest.mark.skipif(not _have_lib(), reason="libtsa.so not built")


def _declared():
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(tsa_\w+)\s*\(", text, re.M))
    return names


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 18, names
    lib = C.CDLL(_lib.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing
    assert set(_lib.SIGNATURES) >= names


def _declared_arity():
    """Parameter count of every tsa_* function declared in include/*.h."""
    out = {}
    for h in os.listdir(os.path.join(ROOT, "include")):
        if not h.endswith(".h"):
            continue
        text = re.sub(r"/\*.*?\*/", " ", open(os.path.join(ROOT, "include", h)).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\**\s+\**(tsa_\w+)\s*\(([^)]*)\)\s*;", text, re.M):
            params = " ".join(m.group(2).split())
            out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_bindings_match_declared_arity():
    """Every ctypes signature in the binding has as many arguments as the C declaration."""
    arity = _declared_arity()
    assert arity, "no declarations parsed"
    for name, (_, args) in _lib.SIGNATURES.items():
        assert name in arity, f"{name} has a binding but no declaration"
        assert len(args) == arity[name], f"{name}: binding takes {len(args)} arguments, header {arity[name]}"


def test_abi_version():
    assert tsa.abi_version() == 1


def _pool(n, P, **kw):
    return tsa.KvPool(n, P, kw.pop("kv_heads", 1), kw.pop("dk", 64), kw.pop("dv", 64),
                      allocate=False, **kw)


def test_worked_example_tables_match_oracle():
    lens = [403, 96, 241, 30, 176]
    pool = _pool(66, 16)
    table, num, saved = pool.build_tables(lens, 26)
    ref = paging.build_page_tables(lens, 16, np.arange(66), max_pages=26)
    assert np.array_equal(table, ref["table"]) and np.array_equal(num, ref["num_pages"])
    assert num.sum() == 61 and saved == 0
    assert pool.usage() == (5, 61)


@pytest.mark.parametrize("name", ["tiny_b5", "gqa_b32_8k", "mla_b64_32k", "prefix_b128_16k"])
def test_workload_tables_match_oracle(name):
    w = synth.get(name)
    lens = synth.lens(w, 0)
    fo = synth.free_order(w, 0)
    grp, plen = synth.prefix_groups(w)
    maxp = -(-int(lens.max()) // w.page_size)
    pool = tsa.KvPool(w.pool_pages, w.page_size, w.num_kv_heads, w.head_dim_k, w.head_dim_v,
                      v_from_k=w.v_from_k, index_dim=w.index_dim, free_order=fo, allocate=False)
    table, num, saved = pool.build_tables(lens, maxp, grp, plen)
    ref = paging.build_page_tables(lens, w.page_size, fo, grp, plen, max_pages=maxp)
    assert np.array_equal(table, ref["table"])
    assert np.array_equal(num, ref["num_pages"])
    assert saved == ref["saved"]
    if name == "prefix_b128_16k":
        assert saved == 127 * (16384 // 64) == 32512
    for p in np.unique(table[table >= 0])[:50]:
        assert pool.refcount(int(p)) == ref["refcount"][p]


def test_sharing_worked_example_and_boundaries():
    lens = [403, 96, 241, 30, 176]
    grp = [0, 0, 0, -1, -1]
    for prefix, used in [(64, 53), (15, 61), (16, 59)]:
        pool = _pool(70, 16)
        table, num, saved = pool.build_tables(lens, 26, grp, [prefix])
        ref = paging.build_page_tables(lens, 16, np.arange(70), grp, [prefix], max_pages=26)
        assert np.array_equal(table, ref["table"])
        assert pool.usage()[1] == used == ref["pages_in_use"]
        assert saved == paging.prefix_pages_saved(3, prefix, 16)


def test_out_of_pages_is_all_or_nothing():
    pool = _pool(60, 16)
    with pytest.raises(tsa.TsaError) as e:
        pool.build_tables([403, 96, 241, 30, 176], 26)
    assert e.value.status == _lib.TSA_ERR_OUT_OF_PAGES
    assert pool.usage() == (60, 0)


def test_grow_and_release_match_oracle():
    perm = np.random.default_rng(4).permutation(40).astype(np.int32)
    pool = _pool(40, 16, free_order=perm)
    lens = [16, 17, 5]
    table, num, _ = pool.build_tables(lens, 4)
    ref = paging.build_page_tables(lens, 16, perm, max_pages=4)
    new = [33, 17, 40]
    pool.grow_tables(table, num, new)
    g = paging.grow_page_tables(ref["table"], ref["num_pages"], new, 16, ref["free"])
    assert np.array_equal(table, g["table"]) and np.array_equal(num, g["num_pages"])
    with pytest.raises(tsa.TsaError) as e:
        pool.grow_tables(table, num, [10, 17, 40])          # shrink
    assert e.value.status == _lib.TSA_ERR_INVALID
    with pytest.raises(tsa.TsaError) as e:
        pool.grow_tables(table, num, [65, 65, 65])          # more than max_pages (4 x 16)
    assert e.value.status == _lib.TSA_ERR_INVALID
    free0, used0 = pool.usage()
    pool.release_tables(table, num)
    assert pool.usage() == (40, 0) and used0 == int(num.sum())
    with pytest.raises(tsa.TsaError):
        pool.release_tables(table, num)                     # double release


def test_shared_release_keeps_pages_until_last():
    pool = _pool(20, 16)
    table, num, _ = pool.build_tables([40, 40], 3, [0, 0], [32])
    assert pool.refcount(int(table[0, 0])) == 2
    pool.release_tables(table[:1].copy(), num[:1].copy())
    assert pool.refcount(int(table[0, 0])) == 1
    pool.release_tables(table[1:].copy(), num[1:].copy())
    assert pool.usage() == (20, 0)


def test_append_check():
    pool = _pool(20, 16)
    table, num, _ = pool.build_tables([40, 40], 3, [0, 0], [32])
    pool.append_check([0, 1], [39, 32], table, num)         # third page is private
    with pytest.raises(tsa.TsaError) as e:
        pool.append_check([1], [31], table, num)            # second page is shared
    assert e.value.status == _lib.TSA_ERR_SHARED_PAGE_WRITE
    with pytest.raises(tsa.TsaError) as e:
        pool.append_check([0], [48], table, num)            # beyond the allocated pages
    assert e.value.status == _lib.TSA_ERR_INVALID
    with pytest.raises(tsa.TsaError) as e:
        pool.append_check([2], [0], table, num)
    assert e.value.status == _lib.TSA_ERR_INVALID


def test_invalid_arguments():
    with pytest.raises(tsa.TsaError):
        _pool(0, 16)
    with pytest.raises(tsa.TsaError):
        tsa.KvPool(10, 16, 1, 60, 64, allocate=False)        # head dim not a multiple of 8
    with pytest.raises(tsa.TsaError):
        tsa.KvPool(10, 16, 1, 64, 128, v_from_k=True, allocate=False)
    with pytest.raises(ValueError):
        _pool(10, 16, free_order=np.arange(9))
    with pytest.raises(tsa.TsaError):
        _pool(3, 16, free_order=np.array([0, 0, 1]))
    pool = _pool(10, 16)
    with pytest.raises(tsa.TsaError):
        pool.build_tables([10, 20], 2, [0, 0], [16])         # shorter than its prefix
    with pytest.raises(tsa.TsaError):
        pool.build_tables([-1], 2)


def test_pool_bytes_exact():
    pool = tsa.KvPool(32832, 64, 1, 576, 512, v_from_k=True, index_dim=128, allocate=False)
    k, v, i = pool.bytes
    assert k == 32832 * 64 * 576 * 2 and v == 0 and i == 32832 * 64 * 128 * 2


def test_device_calls_refuse_metadata_pool():
    pool = _pool(10, 16, index_dim=32)
    p = tsa.decode_params(1, 8, 4, 16, 0.125)
    n = tsa.workspace_bytes(pool, p)
    assert n > 0
    with pytest.raises(tsa.TsaError) as e:
        tsa.sparse_decode_attn(pool, 0, p, None, None, None, _FakeDev(1), None, None, None,
                               stream=0)
    assert e.value.status == _lib.TSA_ERR_INVALID


def test_step_graph_refuses_before_capture():
    """Argument errors of the captured step are reported before anything touches the GPU."""
    import ctypes as C
    pool = _pool(10, 16, index_dim=32)
    p = tsa.decode_params(1, 8, 4, 16, 0.125)
    lib = _lib.load()
    h = C.c_void_p()
    st = lib.tsa_step_graph_create(pool.handle, 0, C.byref(p), None, None, None, None, None, 1, None,
                                   None, None, None, 0, C.byref(h))
    assert st == _lib.TSA_ERR_INVALID and b"device memory" in lib.tsa_last_error()
    st = lib.tsa_step_graph_create(pool.handle, 0, C.byref(p), None, None, None, None, None, 1, None,
                                   None, None, None, 0, None)
    assert st == _lib.TSA_ERR_INVALID
    assert lib.tsa_step_graph_launch(None, None) == _lib.TSA_ERR_INVALID
    assert lib.tsa_step_graph_destroy(None) == _lib.TSA_OK


class _FakeDev:
    """Stands in for a device tensor in argument-validation tests (never dereferenced)."""
    def __init__(self, max_pages):
        self.shape = (1, max_pages)

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0


# ---------------------------------------------------------------- tiered cache bookkeeping

def _tier_positions(rng, n_req, k, length, hot):
    """Locality-biased positions (a few hot spots plus uniform picks), distinct per request."""
    out = np.empty((n_req, k), dtype=np.int32)
    for r in range(n_req):
        centres = rng.integers(0, length, size=hot)
        loc = np.clip(centres[rng.integers(0, hot, size=2 * k)] + rng.normal(0, 200, size=2 * k), 0,
                      length - 1).astype(np.int64)
        pool = np.unique(np.concatenate([loc, rng.integers(0, length, size=k)]))
        out[r] = np.sort(rng.choice(pool, size=k, replace=False))
    return out


@pytest.mark.parametrize("capacity,K", [(256, 96), (160, 24), (4096, 96)])
def test_lru_tier_matches_oracle(capacity, K):
    """Slot tables, hits, misses and evictions of the library's tier equal the oracle's under
    the same plan / release sequence (two layers in flight), with a preloaded start."""
    from oracle import lru
    P, L, R, NPR = 64, 3, 4, 32
    cache = _pool(capacity, P, kv_heads=2, dk=128, dv=128)
    tier = tsa.LruTier(cache, L, R, NPR)
    oc = lru.LRUCache(capacity)
    pre = np.array([(l * R + r) * NPR + p for l in range(L) for r in range(R) for p in range(NPR - 3, NPR)
                    if ((l * R + r) * 3 + p) % 2 == 0][:capacity // 2], dtype=np.int64)
    tier.preload(pre)
    oc.preload(pre.tolist())
    rng = np.random.default_rng(capacity)
    g = touches = 0
    for step in range(4):
        for layer in range(L):
            pos = _tier_positions(rng, R, K, NPR * P, hot=3)
            touches += sum(len(lru.pages_of_positions(p, P)) for p in pos)
            table, _ = tier.plan(layer, g, pos)
            ref = lru.plan_layer(oc, layer, R, NPR, pos, P, g)
            assert np.array_equal(table, ref), (step, layer)
            if g > 0:
                tier.release(g - 1)
                oc.release(g - 1)
            g += 1
    st = tier.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (oc.hits, oc.misses, oc.evictions)
    assert st["hits"] + st["misses"] == touches
    if capacity >= L * R * NPR:
        assert st["evictions"] == 0
    elif K == 24:
        assert st["hits"] > 0 and st["evictions"] > 0      # a cache that both hits and evicts


@pytest.mark.parametrize("capacity", [400, 700])
def test_lru_token_tier_matches_oracle(capacity):
    """Token-granular tier (a cache pool with one-token pages): slot tables and counters equal
    the oracle's LRU over token keys.  Up to three tags are in flight and the middle one is
    released first, so released slots must rejoin the eviction order by touch time, not at
    the newest end; plans without the host table count the same."""
    from oracle import lru
    L, R, T, K = 2, 3, 768, 40
    cache = _pool(capacity, 1, kv_heads=2, dk=128, dv=128)
    tier = tsa.LruTier(cache, L, R, T)
    oc = lru.LRUCache(capacity)
    rng = np.random.default_rng(capacity + 7)
    held = []
    g = 0
    for step in range(6):
        for layer in range(L):
            pos = _tier_positions(rng, R, K, T, hot=2)
            want_table = g % 3 != 2
            table, pending = tier.plan(layer, g, pos, table=want_table)
            ref = lru.plan_layer(oc, layer, R, T, pos, 1, g)
            if want_table:
                assert np.array_equal(table, ref), (step, layer)
            else:
                assert table is None
            held.append(g)
            if len(held) == 3:
                # release the middle tag, then the oldest: out of plan order
                for tag in (held[1], held[0]):
                    tier.release(tag)
                    oc.release(tag)
                held = held[2:]
            g += 1
            st = tier.stats()
            assert (st["hits"], st["misses"], st["evictions"]) == (oc.hits, oc.misses, oc.evictions)
    assert oc.evictions > 0 and oc.hits > 0


def test_lru_tier_capacity_error_changes_nothing():
    P, R, NPR = 64, 2, 8
    cache = _pool(4, P, kv_heads=2, dk=128, dv=128)
    tier = tsa.LruTier(cache, 1, R, NPR)
    t0, _ = tier.plan(0, 0, np.array([[0, 64, 128], [-1, -1, 5]], dtype=np.int32))
    assert sorted(t0[t0 >= 0].tolist()) == [0, 1, 2, 3]
    before = tier.stats()
    # tag 0 still pins all four slots: a plan that needs a new page cannot fit
    with pytest.raises(tsa.TsaError) as e:
        tier.plan(0, 1, np.array([[0, 200, 300], [5, 6, 7]], dtype=np.int32))
    assert e.value.status == _lib.TSA_ERR_CAPACITY
    assert tier.stats() == before
    # hits only: fits even with everything pinned
    t1, _ = tier.plan(0, 1, np.array([[0, 65, 130], [1, 2, 3]], dtype=np.int32))
    assert np.array_equal(t1, t0)
    tier.release(0)
    tier.release(1)
    with pytest.raises(tsa.TsaError):
        tier.release(1)
    t2, _ = tier.plan(0, 2, np.array([[300, 301, 302], [-1, -1, -1]], dtype=np.int32))
    assert t2[0, 4] >= 0 and tier.stats()["evictions"] == 1


def test_lru_tier_refuses_fetch_without_device_memory():
    cache = _pool(8, 64, kv_heads=2, dk=128, dv=128)
    tier = tsa.LruTier(cache, 1, 1, 4)
    table, _ = tier.plan(0, 0, np.array([[0]], dtype=np.int32))
    with pytest.raises(tsa.TsaError):
        _lib.call("tsa_lru_fetch", tier.handle, 1, None, None, None, 0, None)


def test_latent_selection_beyond_64_splits_leaves_the_matrix_core_kernel():
    """A latent-shape selection longer than 64 row lists of 1,024 tokens would need more splits
    than the split combine merges; the plan must then take the vector-ALU kernel, whose split
    count stays <= 64.  Checked through the workspace size (no kernel runs): with 64 splits at
    most, the partials of 1 request x 64 heads x 512 value dims fit in
    (2 n + n * 512) * 4 bytes with n = 64 * 64."""
    pool = tsa.KvPool(1600, 64, 1, 576, 512, v_from_k=True, index_dim=128, allocate=False)
    L = 100_000
    p = tsa.decode_params(1, 64, L, L, 1.0 / 24.0)
    ws = tsa.workspace_bytes(pool, p)
    scores = -(-L // 64) * 64 * 4
    topk = -(-(L * 4) // 256) * 256
    n = 64 * 64
    partial = (2 * n + n * 512) * 4
    assert 0 < ws <= scores + topk + partial + 3 * 256


@pytest.mark.parametrize("seed", range(60))
def test_random_tables_build_grow_release_match_oracle(seed):
    """Seeded random batches through build, grow and release: tables, page counts, saved pages
    and refcounts equal the oracle's; a pool too small for a build or a grow is refused by both,
    with nothing changed; releasing everything returns every page."""
    rng = np.random.default_rng(seed)
    P = int(rng.choice([1, 2, 8, 16, 48, 64, 128]))
    n = int(rng.integers(1, 13))
    lens = rng.integers(0, 1500, size=n)
    grp = np.full(n, -1, dtype=np.int32)
    plen = []
    for g in range(int(rng.integers(0, 4))):
        members = rng.choice(n, size=int(rng.integers(1, n + 1)), replace=False)
        members = [m for m in members if grp[m] < 0]
        if not members:
            continue
        gi = len(plen)
        grp[members] = gi
        plen.append(int(rng.integers(0, int(lens[members].min()) + 1)))
    need = sum(-(-int(L) // P) for L in lens)
    N = max(1, need + int(rng.integers(-3, 40)))
    fo = rng.permutation(N).astype(np.int32)
    maxp = max(1, -(-2000 // P))
    pool = _pool(N, P, free_order=fo)
    args = (grp, plen) if plen else (None, None)
    try:
        ref = paging.build_page_tables(lens, P, fo, *args, max_pages=maxp) if plen else \
            paging.build_page_tables(lens, P, fo, max_pages=maxp)
    except MemoryError:
        with pytest.raises(tsa.TsaError) as e:
            pool.build_tables(lens, maxp, *args) if plen else pool.build_tables(lens, maxp)
        assert e.value.status == _lib.TSA_ERR_OUT_OF_PAGES and pool.usage() == (N, 0)
        return
    table, num, saved = pool.build_tables(lens, maxp, *args) if plen else pool.build_tables(lens, maxp)
    assert np.array_equal(table, ref["table"]) and np.array_equal(num, ref["num_pages"])
    assert saved == ref["saved"] and pool.usage()[1] == ref["pages_in_use"]
    for p in np.unique(table[table >= 0]):
        assert pool.refcount(int(p)) == ref["refcount"][p]
    # grow: requests without shared pages may lengthen (a write into a shared page is refused)
    new = np.array([L + (int(rng.integers(0, 300)) if grp[i] < 0 else 0) for i, L in enumerate(lens)])
    try:
        g = paging.grow_page_tables(ref["table"], ref["num_pages"], new, P, ref["free"])
    except MemoryError:
        before = (table.copy(), num.copy(), pool.usage())
        with pytest.raises(tsa.TsaError) as e:
            pool.grow_tables(table, num, new)
        assert e.value.status == _lib.TSA_ERR_OUT_OF_PAGES
        assert np.array_equal(table, before[0]) and np.array_equal(num, before[1]) and pool.usage() == before[2]
    else:
        pool.grow_tables(table, num, new)
        assert np.array_equal(table, g["table"]) and np.array_equal(num, g["num_pages"])
    pool.release_tables(table, num)
    assert pool.usage() == (N, 0)


@pytest.mark.parametrize("seed", range(40))
def test_random_lru_tier_matches_oracle(seed):
    """Seeded random tier runs: page or token units, 1-4 layers, 1-5 requests, capacities from
    tight to roomy, a random preload, positions with -1 padding, and tags released in random
    order while others stay in flight.  After every plan the slot table and the hit, miss and
    eviction counts equal the oracle's; a plan the oracle cannot complete (every slot it would
    need is pinned) is refused by the library with nothing changed."""
    import copy
    from oracle import lru
    rng = np.random.default_rng(900 + seed)
    P = int(rng.choice([1, 16, 64]))
    L, R = int(rng.integers(1, 5)), int(rng.integers(1, 6))
    NPR = int(rng.integers(4, 65)) if P > 1 else int(rng.integers(64, 1025))
    keys = L * R * NPR
    capacity = int(rng.integers(max(2, keys // 20), keys + 10))
    cache = _pool(capacity, P, kv_heads=1, dk=64, dv=64)
    tier = tsa.LruTier(cache, L, R, NPR)
    oc = lru.LRUCache(capacity)
    pre = rng.choice(keys, size=int(rng.integers(0, min(keys, capacity) + 1)), replace=False).astype(np.int64)
    tier.preload(pre)
    oc.preload(pre.tolist())
    held, g, refused = [], 0, 0
    for step in range(int(rng.integers(3, 8))):
        for layer in range(L):
            k = int(rng.integers(1, min(NPR * P, 300) + 1))
            pos = np.full((R, k), -1, dtype=np.int32)
            for r in range(R):
                m = int(rng.integers(0, k + 1))
                pos[r, :m] = np.sort(rng.choice(NPR * P, size=min(m, NPR * P), replace=False))[:m]
            saved = copy.deepcopy(oc)
            try:
                ref = lru.plan_layer(oc, layer, R, NPR, pos, P, g)
            except MemoryError:
                oc = saved
                before = tier.stats()
                with pytest.raises(tsa.TsaError) as e:
                    tier.plan(layer, g, pos)
                assert e.value.status == _lib.TSA_ERR_CAPACITY and tier.stats() == before
                refused += 1
                for tag in held:                          # free everything and go on
                    tier.release(tag)
                    oc.release(tag)
                held = []
            else:
                table, _ = tier.plan(layer, g, pos)
                assert np.array_equal(table, ref), (seed, step, layer)
                held.append(g)
            g += 1
            st = tier.stats()
            assert (st["hits"], st["misses"], st["evictions"]) == (oc.hits, oc.misses, oc.evictions)
            # release a random subset of the tags in flight, in random order
            if held and rng.random() < 0.7:
                chosen = [int(i) for i in rng.choice(len(held), size=int(rng.integers(1, len(held) + 1)),
                                                     replace=False)]
                for i in sorted(chosen, reverse=bool(rng.random() < 0.5)):
                    tier.release(held[i])
                    oc.release(held[i])
                held = [t for j, t in enumerate(held) if j not in chosen]
    assert refused or oc.hits + oc.misses > 0
