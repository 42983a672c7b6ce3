"""The whole decode step on seeded random shapes against the oracle.

Each seed draws one configuration: the latent layout (576-dim rows whose first 512 dims are the
values, one KV head, 8 to 128 query heads) or a grouped-query layout (head dims 64 to 256, some
with values aliasing the keys, 1 to 32 query heads per KV head), a page size from 1 to 128, an
indexer of 32 to 128 dims with 1 to 64 heads, a ragged batch of up to 9 requests (lengths from 0
to 5,000, page boundaries included) and a top-k from 1 to 2,048.  So the draws reach every
attention kernel (latent and grouped-query matrix-core kernels, the vector-ALU kernel), both
indexer kernels and both top-k paths.  Indexer scores and top-k sets must equal the oracle's bit
for bit and every request's attention must be within the 2e-3 normwise bar.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import synth
from oracle import decode, sdpa

pytestmark = pytest.mark.gpu

ATOL_REL = 2e-3


@pytest.fixture(scope="module")
def tsa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import top_sparse_attention_amd as m
    m.load()
    return m


def _draw(seed):
    """One configuration: (base workload, field replacements, stage keyword arguments)."""
    rng = np.random.default_rng(1000 + seed)
    if rng.random() < 0.4:
        base = "mla_b64_32k"
        wrep = {"num_q_heads": int(rng.choice([8, 16, 48, 64, 128]))}
    else:
        base = "gqa_b32_8k"
        dk, dv, alias = [(64, 64, False), (128, 128, False), (192, 128, False), (256, 256, False),
                         (96, 96, False), (128, 64, True)][int(rng.integers(6))]
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16, 32]))
        wrep = {"head_dim_k": dk, "head_dim_v": dv, "v_from_k": alias, "num_kv_heads": hkv,
                "num_q_heads": hkv * g}
    page = int(rng.choice([1, 8, 16, 48, 64, 128]))
    wrep["index_dim"] = int(rng.choice([32, 64, 128]))
    heads = int(rng.choice([1, 2, 4, 16, 64]))
    if page < 16:                       # the register indexer kernel takes up to 8 heads
        heads = min(heads, 8)
    wrep["top_k"] = int(rng.choice([1, 3, 64, 100, 512, 2048]))
    B = int(rng.integers(1, 10))
    lens = rng.integers(0, 5001, size=B)
    edges = [0, 1, page - 1, page, page + 1, 2 * page, wrep["top_k"], wrep["top_k"] + 1]
    for i in range(B):
        if rng.random() < 0.3:
            lens[i] = max(0, int(rng.choice(edges)))
    return base, wrep, dict(lens=lens.astype(np.int32), page_size=page, index_heads=heads)


# 48 draws by default; RANDOM_SHAPES=N runs more of the same sequence
@pytest.mark.parametrize("seed", range(int(os.environ.get("RANDOM_SHAPES", "48"))))
def test_random_shape_step_matches_oracle(tsa, seed):
    from top_sparse_attention_amd import workload
    base, wrep, kw = _draw(seed)
    print(f"[random shape {seed}] {base} {wrep} page {kw['page_size']} index heads "
          f"{kw['index_heads']} lens {kw['lens'].tolist()}", flush=True)
    w = dataclasses.replace(synth.get(base), **wrep)
    st = workload.stage(w, seed=seed, **kw)
    B = len(st.lens)
    ld = max(64, -(-st.params.max_len // 64) * 64)
    sc = torch.full((B, ld), float("nan"), dtype=torch.float32, device="cuda")
    tsa.indexer_scores(st.pool, 0, st.params, st.qidx, st.widx, st.table_dev, st.lens_dev, sc)
    st.step(append=False)
    torch.cuda.synchronize()
    scores = sc.cpu().numpy()
    topk = st.topk.cpu().numpy()
    out = st.out.double().cpu().numpy()
    for b in range(B):
        L = int(st.lens[b])
        if L == 0:                      # nothing to score or attend: no selection, zero output
            assert (topk[b] == -1).all() and not out[b].any(), f"empty request {b}"
            continue
        kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
        s_ref, sel_ref, o_ref = decode.request_step(
            st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv, w.top_k, w.sm_scale,
            v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
        assert np.array_equal(scores[b, :L].astype(np.float64), np.asarray(s_ref, np.float64)), \
            f"scores differ, request {b} (len {L})"
        exp = np.full(w.top_k, -1, dtype=np.int32)
        exp[:len(sel_ref)] = sel_ref
        assert np.array_equal(topk[b], exp), f"top-k differs, request {b} (len {L})"
        err = sdpa.normwise_rel_err(out[b], o_ref)
        assert err < ATOL_REL, f"attention error {err} on request {b} (len {L})"


@pytest.mark.parametrize("base,page", [("mla_b64_32k", 64), ("mla_b64_32k", 48), ("gqa_b32_8k", 8),
                                       ("tiny_b5", 16)])
def test_all_empty_batch_every_entry_point(tsa, base, page):
    """A batch whose requests are all empty (every length 0, so the longest is 0): each step
    entry point runs, selects nothing and writes zero outputs."""
    from top_sparse_attention_amd import workload
    lens = np.zeros(3, dtype=np.int32)
    print(f"[empty batch] {base} page {page}", flush=True)
    st = workload.stage(synth.get(base), seed=0, lens=lens, page_size=page)
    B = len(lens)
    w = st.w
    assert st.params.max_len == 0

    def fresh():
        st.out.fill_(float("nan"))
        st.topk.fill_(7)
    fresh()
    tsa.sparse_decode_attn(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                           st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    assert (st.topk.cpu() == -1).all() and not st.out.cpu().double().numpy().any()
    fresh()
    # new-token rows of the right shape (an empty request appends nothing)
    k_new = torch.zeros((B, w.num_kv_heads * w.head_dim_k), dtype=torch.int16, device="cuda")
    v_new = None if w.v_from_k else torch.zeros((B, w.num_kv_heads * w.head_dim_v), dtype=torch.int16,
                                                device="cuda")
    i_new = torch.zeros((B, w.index_dim), dtype=torch.int16, device="cuda")
    tsa.decode_step(st.pool, 0, st.params, k_new, v_new, i_new, st.q, st.qidx, st.widx,
                    st.table_dev, st.lens_dev, st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    assert (st.topk.cpu() == -1).all() and not st.out.cpu().double().numpy().any()
    fresh()
    tsa.indexer_topk(st.pool, 0, st.params, st.qidx, st.widx, st.table_dev, st.lens_dev, st.topk,
                     st.workspace)
    tsa.sparse_attn_gather(st.pool, 0, st.params, st.q, st.topk, st.table_dev, st.lens_dev, st.out,
                           st.workspace)
    torch.cuda.synchronize()
    assert (st.topk.cpu() == -1).all() and not st.out.cpu().double().numpy().any()
    assert st.out.shape[0] == B and st.topk.shape == (B, w.top_k)


@pytest.mark.parametrize("seed", range(int(os.environ.get("RANDOM_SHAPES", "48"))))
def test_random_shape_decode_step_matches_oracle(tsa, seed):
    """tsa_decode_step on the same draws, short ones made shorter so that some take the one-launch
    step: each request's newest token is written inside the step (scoring launch, separate append
    or one-launch kernel) and the result must match the oracle over all L tokens."""
    from top_sparse_attention_amd import workload
    base, wrep, kw = _draw(seed)
    if seed % 3 == 0:                   # short contexts, few rows: the one-launch step's range
        kw["lens"] = np.minimum(kw["lens"], 900).astype(np.int32)
        wrep["top_k"] = min(wrep["top_k"], 64)
    print(f"[random step {seed}] {base} {wrep} page {kw['page_size']} index heads "
          f"{kw['index_heads']} lens {kw['lens'].tolist()}", flush=True)
    w = dataclasses.replace(synth.get(base), **wrep)
    st = workload.stage(w, seed=seed, **kw)
    B = len(st.lens)
    # one new-row per request; empty requests append nothing, so theirs stay zero
    k_new = torch.zeros((B, w.num_kv_heads * w.head_dim_k), dtype=torch.int16, device="cuda")
    v_new = None if w.v_from_k else torch.zeros((B, w.num_kv_heads * w.head_dim_v), dtype=torch.int16,
                                                device="cuda")
    i_new = torch.zeros((B, w.index_dim), dtype=torch.int16, device="cuda")
    if st.new_req is not None:
        nz = st.new_req.long()
        k_new[nz] = st.new_k.view(torch.int16).reshape(len(nz), -1)
        if v_new is not None:
            v_new[nz] = st.new_v.view(torch.int16).reshape(len(nz), -1)
        i_new[nz] = st.new_idx.view(torch.int16).reshape(len(nz), -1)
    st.out.fill_(float("nan"))
    tsa.decode_step(st.pool, 0, st.params, k_new, v_new, i_new, st.q, st.qidx, st.widx,
                    st.table_dev, st.lens_dev, st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    topk = st.topk.cpu().numpy()
    out = st.out.double().cpu().numpy()
    for b in range(B):
        L = int(st.lens[b])
        if L == 0:
            assert (topk[b] == -1).all() and not out[b].any(), f"empty request {b}"
            continue
        kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
        _, sel_ref, o_ref = decode.request_step(
            st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv, w.top_k, w.sm_scale,
            v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
        exp = np.full(w.top_k, -1, dtype=np.int32)
        exp[:len(sel_ref)] = sel_ref
        assert np.array_equal(topk[b], exp), f"top-k differs, request {b} (len {L})"
        err = sdpa.normwise_rel_err(out[b], o_ref)
        assert err < ATOL_REL, f"attention error {err} on request {b} (len {L})"


@pytest.mark.parametrize("seed", range(int(os.environ.get("RANDOM_SHAPES", "48")) // 2))
def test_random_appends_land_where_the_oracle_says(tsa, seed):
    """Seeded random tsa_kv_append calls (several layers, ragged tables, page sizes 1-128, values
    aliased or separate, with or without indexer rows): every row lands in the physical slot the
    oracle's table gives, every other byte of the pool is unchanged, and each refused token
    (request or position out of range, position past the request's pages) is counted once."""
    from oracle import paging
    rng = np.random.default_rng(500 + seed)
    P = int(rng.choice([1, 8, 16, 48, 64, 128]))
    NL = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2, 4]))
    dk = int(rng.choice([64, 128, 576]))
    alias = dk == 576 or bool(rng.random() < 0.3)
    dv = 512 if dk == 576 else (dk if not alias else dk // 2)
    D = int(rng.choice([0, 32, 128]))
    n = int(rng.integers(1, 8))
    lens = rng.integers(0, 800, size=n)
    need = sum(-(-int(L) // P) for L in lens)
    N = need + int(rng.integers(1, 20))
    fo = rng.permutation(N).astype(np.int32)
    maxp = max(1, -(-900 // P))
    pool = tsa.KvPool(N, P, hkv, dk, dv, num_layers=NL, v_from_k=alias, index_dim=D, free_order=fo)
    table, num, _ = pool.build_tables(lens, maxp)
    ref = paging.build_page_tables(lens, P, fo, max_pages=maxp)
    assert np.array_equal(table, ref["table"])
    table_dev = torch.from_numpy(table).cuda()
    slots = N * P
    regions = [(pool.k, hkv * dk)] + ([] if pool.v is None else [(pool.v, hkv * dv)]) + \
              ([] if pool.idx is None else [(pool.idx, D)])
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t, _ in regions:
        t.view(torch.int16).copy_(torch.randint(-30000, 30000, t.shape, generator=g, device="cuda",
                                                dtype=torch.int16))
    expect = [t.view(torch.int16).cpu().numpy().reshape(NL * slots, width).copy() for t, width in regions]
    for layer in range(NL):
        # distinct valid tokens, plus refused ones of every kind
        valid = [(r, p) for r in range(n) for p in range(int(num[r]) * P)]
        pick = [valid[i] for i in rng.choice(len(valid), size=min(len(valid), 60), replace=False)] if valid else []
        refused = [(n + 1, 0), (-1, 0), (0, -5), (0, maxp * P + 3)]
        refused += [(r, int(num[r]) * P + int(rng.integers(0, P))) for r in range(n) if num[r] < maxp][:3]
        items = pick + refused
        order = rng.permutation(len(items))
        req = np.array([items[i][0] for i in order], dtype=np.int32)
        pos = np.array([items[i][1] for i in order], dtype=np.int32)
        M = len(req)
        rows = [rng.integers(-30000, 30000, size=(M, width)).astype(np.int16) for _, width in regions]
        bad = torch.zeros(1, dtype=torch.int32, device="cuda")
        print(f"[random append {seed}] layer {layer} P {P} hkv {hkv} dk {dk} dv {dv} alias {alias} "
              f"D {D} tokens {M} refused {len(refused)}", flush=True)
        src = [torch.from_numpy(x).cuda() for x in rows]
        k_src = src[0]
        v_src = src[1] if pool.v is not None else None
        i_src = src[-1] if pool.idx is not None else None
        pool.append(layer, torch.from_numpy(req).cuda(), torch.from_numpy(pos).cuda(), table_dev, n,
                    k_src, v_src, i_src, bad_dev=bad)
        torch.cuda.synchronize()
        for j in range(M):
            r, p = int(req[j]), int(pos[j])
            if 0 <= r < n and p >= 0 and p // P < maxp and table[r, p // P] >= 0:
                s = layer * slots + paging.physical_slot(table, r, p, P)
                for e, x in zip(expect, rows):
                    e[s] = x[j]
        assert int(bad.item()) == len(refused)
        for (t, width), e in zip(regions, expect):
            assert np.array_equal(t.view(torch.int16).cpu().numpy().reshape(NL * slots, width), e)


@pytest.mark.parametrize("seed", range(int(os.environ.get("RANDOM_SHAPES", "48")) // 3))
def test_random_tier_fetch_copies_the_host_rows(tsa, seed):
    """Seeded random tier runs on the GPU (page or token unit, random shapes and capacities,
    tags released in random order): after each plan and fetch, the device slot table equals the
    plan's, and every touched page's cache slot holds exactly that page's host K and V rows."""
    rng = np.random.default_rng(1300 + seed)
    P = int(rng.choice([1, 16, 64]))
    hkv, d = int(rng.choice([1, 2])), int(rng.choice([64, 128]))
    L, R = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    NPR = int(rng.integers(4, 41)) if P > 1 else int(rng.integers(64, 513))
    keys = L * R * NPR
    # at least one layer's pages, so that a plan fits once nothing else is pinned; below the
    # whole set, so that layers and held tags make evictions
    capacity = int(rng.integers(max(8, R * NPR), max(R * NPR, keys) + 1))
    g = torch.Generator().manual_seed(seed)
    host_k = torch.randint(-30000, 30000, (keys * P, hkv * d), generator=g, dtype=torch.int16).pin_memory()
    host_v = torch.randint(-30000, 30000, (keys * P, hkv * d), generator=g, dtype=torch.int16).pin_memory()
    cache = tsa.KvPool(capacity, P, hkv, d, d)
    tier = tsa.LruTier(cache, L, R, NPR, host_k, host_v)
    ck = cache.k.view(torch.int16).view(capacity * P, hkv * d)
    cv = cache.v.view(torch.int16).view(capacity * P, hkv * d)
    print(f"[random tier {seed}] P {P} hkv {hkv} d {d} layers {L} requests {R} pages {NPR} "
          f"capacity {capacity}", flush=True)
    held, tag, checked = [], 0, 0
    for step in range(3):
        for layer in range(L):
            k = int(rng.integers(1, min(NPR * P, 256) + 1))
            pos = np.full((R, k), -1, dtype=np.int32)
            for r in range(R):
                m = int(rng.integers(0, k + 1))
                pos[r, :m] = np.sort(rng.choice(NPR * P, size=m, replace=False))
            try:
                table, _ = tier.plan(layer, tag, pos)
            except tsa.TsaError:
                for t in held:
                    tier.release(t)
                held = []
                tag += 1
                continue
            table_dev = torch.full((R, NPR), -1, dtype=torch.int32, device="cuda")
            tier.fetch(table_dev)
            torch.cuda.synchronize()
            assert np.array_equal(table_dev.cpu().numpy(), table)
            hk, hv = ck.cpu().numpy(), cv.cpu().numpy()
            for r, page in zip(*np.nonzero(table >= 0)):
                key = (layer * R + int(r)) * NPR + int(page)
                s = int(table[r, page])
                assert np.array_equal(hk[s * P:(s + 1) * P], host_k[key * P:(key + 1) * P].numpy()), (r, page)
                assert np.array_equal(hv[s * P:(s + 1) * P], host_v[key * P:(key + 1) * P].numpy()), (r, page)
                checked += 1
            held.append(tag)
            tag += 1
            if rng.random() < 0.6:
                chosen = [int(i) for i in rng.permutation(len(held))[:int(rng.integers(1, len(held) + 1))]]
                for i in chosen:
                    tier.release(held[i])
                held = [t for j, t in enumerate(held) if j not in chosen]
    assert checked > 0
