"""Requests that alias prefix pages against the oracle and against private copies of the prefix.

When requests map the same physical pages for a common prefix (paged-KV page, page sharing), every
kernel of the step reads those pages through each request's own page table.  The step's scores
(read back from its workspace) must equal the oracle's bit for bit on every request, its top-k
sets must equal the oracle's and its attention must be within the 2e-3 bar; the same requests
staged with private copies of the prefix must give bit-identical scores, top-k and outputs.
Besides the 128-request workload, a batch of 8 whose page tables are edited after staging: some
shared pages of some requests replaced by private copies of the same rows, so that request 0
shares nothing with the others, request 3 shares its first 100 pages, request 5 all but the last
prefix page and request 7 none.
"""
import numpy as np
import pytest

import synth
from oracle import sdpa

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


def _step_scores(st):
    B = len(st.lens)
    ld = max(64, -(-st.params.max_len // 64) * 64)
    return st.workspace[:B * ld * 4].view(torch.float32).view(B, ld)


def _privatize(st, b, pages, free_ids):
    """Give request b private copies of its logical pages `pages` (same rows, new physical pages)."""
    w, P = st.w, st.w.page_size
    rows = ((st.pool.k, w.num_kv_heads * w.head_dim_k), (st.pool.v, w.num_kv_heads * w.head_dim_v),
            (st.pool.idx, w.index_dim))
    for i in pages:
        src, dst = int(st.table_dev[b, i].item()), free_ids.pop()
        for t, r in rows:
            t[dst * P * r:(dst + 1) * P * r] = t[src * P * r:(src + 1) * P * r]
        st.table_dev[b, i] = dst


@pytest.mark.parametrize("edited", [False, True])
def test_shared_prefix_pass_matches_oracle_and_copies(tsa, edited):
    from top_sparse_attention_amd import workload
    w = synth.get("prefix_b128_16k")
    kw = {"batch": 8} if edited else {}
    print(f"[prefix share] {'edited tables, 8 requests' if edited else 'workload'}", flush=True)
    shared = workload.stage(w, seed=0, extra_pages=600 if edited else 0, **kw)
    if edited:
        P = w.page_size
        n_pages = shared.pool.k.numel() // (P * w.num_kv_heads * w.head_dim_k)
        used = set(shared.table_dev.flatten().tolist())
        free_ids = sorted(set(range(n_pages)) - used)
        _privatize(shared, 0, [0], free_ids)
        _privatize(shared, 3, range(100, 256), free_ids)
        _privatize(shared, 5, [255], free_ids)
        _privatize(shared, 7, range(0, 256), free_ids)
        torch.cuda.synchronize()
    # private copies need the pages the sharing saves (the stated pool counts the prefix once)
    private = workload.stage(w, seed=0, share_prefix=False, extra_pages=int(shared.saved), **kw)
    assert shared.saved > 0 and private.saved == 0
    for st in (shared, private):
        st.step(append=False)
    torch.cuda.synchronize()
    B = len(shared.lens)
    sc_s, sc_p = _step_scores(shared), _step_scores(private)
    for b in range(B):
        L = int(shared.lens[b])
        assert torch.equal(sc_s[b, :L], sc_p[b, :L]), f"scores differ from the private copies, request {b}"
    assert torch.equal(shared.topk, private.topk)
    assert torch.equal(shared.out, private.out)
    scores = sc_s.cpu().numpy()
    got = shared.topk.cpu().numpy()
    out = shared.out.double().cpu().numpy()
    from oracle_pool import oracle_requests
    ref = oracle_requests(w, shared.seed, range(B), shared.q_np, shared.qidx_np, shared.widx_np)
    worst = 0.0
    for b in range(B):
        L = int(shared.lens[b])
        if L == 0:
            assert (got[b] == -1).all() and not np.any(out[b])
            continue
        s_ref, sel_ref, o_ref = ref[b]
        assert np.array_equal(scores[b, :L].astype(np.float64), np.asarray(s_ref, np.float64)), f"scores, request {b}"
        exp = np.full(w.top_k, -1, dtype=np.int32)
        exp[:len(sel_ref)] = sel_ref
        assert np.array_equal(got[b], exp), f"top-k, request {b}"
        err = sdpa.normwise_rel_err(out[b], o_ref)
        assert err < ATOL_REL, f"attention error {err} on request {b}"
        worst = max(worst, err)
    print(f"{B} requests, max normwise attention error {worst:.3e}")
