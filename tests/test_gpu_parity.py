"""GPU parity: every kernel of the decode step against the CPU oracle, through the C ABI.

Bar: page tables, pool placement, indexer scores and top-k index sets bit-exact; attention
output within 2e-3 normwise relative error per (request, head) row (max_{row} ||o - ref||_inf /
||ref||_inf), the bound stated for this path.  Inputs are the seeded synthetic workloads; the
oracle recomputes each checked request from the same draws.
"""
import os

import numpy as np
import pytest

import synth
from oracle import decode, indexer, paging, sdpa, topk as otopk
from oracle.bf16 import to_f64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL_REL = 2e-3


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def tsa():
    _need_gpu()
    import top_sparse_attention_amd as m
    m.load()
    return m


_STAGED = {}


def staged(name, wreplace=None, **kw):
    """Stage workload `name` (with fields replaced by `wreplace`), cached across tests."""
    import dataclasses
    from top_sparse_attention_amd import workload
    wr = tuple(sorted((wreplace or {}).items()))
    key = (name, wr, tuple((k, v.tobytes() if isinstance(v, np.ndarray) else v) for k, v in sorted(kw.items())))
    if key not in _STAGED:
        print(f"[stage] {name} {dict(wr)} {kw}", flush=True)
        _STAGED[key] = workload.stage(dataclasses.replace(synth.get(name), **dict(wr)), **kw)
    return _STAGED[key]


def _oracle_request(st, b):
    w = st.w
    L = int(st.lens[b])
    kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
    s, sel, o = decode.request_step(st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv, w.top_k,
                                    w.sm_scale, v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
    return s, sel, o


def _scores_gpu(tsa, st):
    ld = max(64, -(-st.params.max_len // 64) * 64)
    sc = torch.full((len(st.lens), ld), float("nan"), dtype=torch.float32, device="cuda")
    tsa.indexer_scores(st.pool, 0, st.params, st.qidx, st.widx, st.table_dev, st.lens_dev, sc)
    torch.cuda.synchronize()
    return sc


def _check_request(st, b, scores_gpu=None):
    s_ref, sel_ref, o_ref = _oracle_request(st, b)
    L = int(st.lens[b])
    if scores_gpu is not None:
        got = scores_gpu[b, :L].cpu().numpy()
        assert np.array_equal(got.astype(np.float64), s_ref.astype(np.float64)), f"scores differ, request {b}"
    tk = st.topk[b].cpu().numpy()
    exp = np.full(st.w.top_k, -1, dtype=np.int32)
    exp[:len(sel_ref)] = sel_ref
    assert np.array_equal(tk, exp), f"top-k differs, request {b}"
    o = st.out[b].double().cpu().numpy()
    err = sdpa.normwise_rel_err(o, o_ref)
    assert err < ATOL_REL, f"attention error {err} on request {b}"
    return err


def _check_all_requests(st, scores_gpu):
    """Every request of a staged workload against the oracle (computed in parallel worker
    processes): scores and top-k sets bit-exact, attention within the bar."""
    from oracle_pool import oracle_requests
    B = len(st.lens)
    ref = oracle_requests(st.w, st.seed, range(B), st.q_np, st.qidx_np, st.widx_np)
    sc = scores_gpu.cpu().numpy()
    tk = st.topk.cpu().numpy()
    out = st.out.double().cpu().numpy()
    errs = []
    for b in range(B):
        s_ref, sel_ref, o_ref = ref[b]
        L = int(st.lens[b])
        assert np.array_equal(sc[b, :L].astype(np.float64), s_ref), f"scores differ, request {b}"
        exp = np.full(st.w.top_k, -1, dtype=np.int32)
        exp[:len(sel_ref)] = sel_ref
        assert np.array_equal(tk[b], exp), f"top-k differs, request {b}"
        err = sdpa.normwise_rel_err(out[b], o_ref)
        assert err < ATOL_REL, f"attention error {err} on request {b}"
        errs.append(err)
    return errs


@pytest.mark.parametrize("name", ["tiny_b5", "gqa_b32_8k", "prefix_b128_16k"])
def test_step_matches_oracle(tsa, name):
    st = staged(name)
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    errs = _check_all_requests(st, sc)
    print(f"{name}: {len(errs)} requests, max normwise attention error {max(errs):.3e}")


def test_tables_match_oracle(tsa):
    for name in ["tiny_b5", "gqa_b32_8k", "prefix_b128_16k"]:
        st = staged(name)
        w = st.w
        grp, plen = synth.prefix_groups(w)
        ref = paging.build_page_tables(st.lens, w.page_size, synth.free_order(w, 0), grp, plen,
                                       max_pages=st.max_pages)
        assert np.array_equal(st.table, ref["table"]) and st.saved == ref["saved"]


@pytest.mark.parametrize("name", ["tiny_b5", "gqa_b32_8k"])
def test_pool_placement(tsa, name):
    """Each logical token sits in the physical slot the oracle's table assigns."""
    st = staged(name)
    w = st.w
    ref = paging.build_page_tables(st.lens, w.page_size, synth.free_order(w, 0), max_pages=st.max_pages)
    kpool = st.pool.k.view(torch.int16).view(-1, w.num_kv_heads, w.head_dim_k)
    ipool = st.pool.idx.view(torch.int16).view(-1, w.index_dim)
    for b in [0, len(st.lens) - 1]:
        L = int(st.lens[b])
        kidx, kk, _ = synth.request_tokens(w, 0, b, L)
        t = np.unique(np.linspace(0, L - 1, 50).astype(int))
        slots = torch.tensor([paging.physical_slot(ref["table"], b, int(x), w.page_size) for x in t],
                             device="cuda")
        assert np.array_equal(kpool[slots].cpu().numpy().view(np.uint16), kk[t])
        assert np.array_equal(ipool[slots].cpu().numpy().view(np.uint16), kidx[t])


def test_free_order_invariance(tsa):
    """Physical placement must not change any result (the slot translation is the library's)."""
    w = synth.get("gqa_b32_8k")
    a = staged("gqa_b32_8k")
    b = staged("gqa_b32_8k", free_order=np.arange(w.pool_pages, dtype=np.int32)[::-1].copy())
    for st in (a, b):
        st.step(append=False)
    torch.cuda.synchronize()
    assert not np.array_equal(a.table, b.table)
    assert torch.equal(a.topk, b.topk)
    assert torch.equal(a.out, b.out)


def test_prefix_alias_vs_copy(tsa):
    """Aliased prefix pages and private copies of the same prefix give identical results."""
    a = staged("prefix_b128_16k", batch=6)
    b = staged("prefix_b128_16k", batch=6, share_prefix=False)
    assert a.saved == 5 * 256 and b.saved == 0
    for st in (a, b):
        st.step(append=False)
    torch.cuda.synchronize()
    assert torch.equal(a.topk, b.topk)
    assert torch.equal(a.out, b.out)


@pytest.mark.parametrize("P", [48, 16])
def test_edge_lengths_and_page_sizes(tsa, P):
    lens = np.array([0, 1, 63, 512, 513, 1000, 4099, 77], dtype=np.int32)
    st = staged("gqa_b32_8k", lens=lens, page_size=P)
    sc = _scores_gpu(tsa, st)
    st.step(append=False)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        if lens[b] == 0:
            assert (st.topk[b] == -1).all() and (st.out[b] == 0).all()
            continue
        _check_request(st, b, sc)


def _check_scores(st, sc, reqs):
    for b in reqs:
        L = int(st.lens[b])
        kidx, _, _ = synth.request_tokens(st.w, st.seed, b, L)
        ref = indexer.scores_bf16(st.qidx_np[b], st.widx_np, kidx)
        got = sc[b, :L].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref.astype(np.float64)), f"scores differ, request {b}"


@pytest.mark.parametrize("heads", [2, 4, 16, 17, 33, 64])
def test_multihead_indexer(tsa, heads):
    """Indexer heads on the matrix cores (2..64, padded to blocks of 16): bit-exact scores."""
    st = staged("gqa_b32_8k", batch=4, index_heads=heads)
    assert st.params.index_heads == heads
    _check_scores(st, _scores_gpu(tsa, st), range(4))


@pytest.mark.parametrize("P,name,heads", [(48, "gqa_b32_8k", 40), (16, "tiny_b5", 64), (8, "tiny_b5", 8)])
def test_multihead_indexer_page_sizes(tsa, P, name, heads):
    """Unaligned pages (48, index_dim 64), the smallest page the streaming kernel takes (16,
    index_dim 32), and pages below it (8), where the register kernel holds up to 8 heads."""
    lens = np.array([1, 47, 48, 49, 200, 777], dtype=np.int32)
    st = staged(name, lens=lens, page_size=P, index_heads=heads)
    _check_scores(st, _scores_gpu(tsa, st), range(len(lens)))


@pytest.mark.parametrize("D,P,heads", [(256, 64, 1), (256, 64, 64), (256, 8, 4), (32, 1, 2), (128, 1, 1)])
def test_indexer_dims_and_small_pages(tsa, D, P, heads):
    """index_dim 256 on the streaming kernel (one head and 64 heads), and pages below 16 tokens,
    down to one token per page, on the register kernel; then the whole step."""
    lens = np.array([1, 100, 1000, 3001], dtype=np.int32)
    st = staged("gqa_b32_8k", wreplace={"index_dim": D}, lens=lens, page_size=P, index_heads=heads)
    sc = _scores_gpu(tsa, st)
    _check_scores(st, sc, range(len(lens)))
    st.step(append=False)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        _check_request(st, b, sc)


@pytest.mark.parametrize("wrep", [
    {"head_dim_k": 256, "head_dim_v": 256},                       # matrix cores, 256-dim heads
    {"num_kv_heads": 1},                                          # 32 q heads on one KV head: vector ALUs
    {"head_dim_k": 128, "head_dim_v": 64, "v_from_k": True},      # values alias keys: vector ALUs
    {"head_dim_k": 96, "head_dim_v": 96},                         # dims no matrix-core kernel takes
])
def test_attention_kernel_shapes(tsa, wrep):
    """Each attention kernel and shape class through the whole step on a few requests."""
    lens = np.array([5, 700, 3001], dtype=np.int32)
    st = staged("gqa_b32_8k", wreplace=wrep, lens=lens, page_size=64)
    sc = _scores_gpu(tsa, st)
    st.step(append=False)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        _check_request(st, b, sc)


def test_multihead_indexer_rejects_too_many_heads(tsa):
    st = staged("tiny_b5", lens=np.array([30, 40], dtype=np.int32), page_size=8, index_heads=8)
    p = tsa.decode_params(2, st.params.num_q_heads, st.params.top_k, st.params.max_len,
                          st.params.sm_scale, index_heads=9)
    sc = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    qidx = torch.zeros((2, 9, st.w.index_dim), dtype=torch.int16, device="cuda")
    widx = torch.ones(9, dtype=torch.float32, device="cuda")
    with pytest.raises(tsa.TsaError, match="index_heads"):
        tsa.indexer_scores(st.pool, 0, p, qidx, widx, st.table_dev, st.lens_dev, sc)
    p65 = tsa.decode_params(2, st.params.num_q_heads, st.params.top_k, st.params.max_len,
                            st.params.sm_scale, index_heads=65)
    st16 = staged("gqa_b32_8k", batch=2, index_heads=64)
    with pytest.raises(tsa.TsaError, match="index_heads"):
        tsa.indexer_scores(st16.pool, 0, p65, st16.qidx, st16.widx, st16.table_dev, st16.lens_dev, sc)


def test_multihead_step_matches_oracle(tsa):
    """The whole step with a 64-head indexer: scores, top-k sets and attention."""
    st = staged("gqa_b32_8k", batch=6, index_heads=64)
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    for b in range(6):
        _check_request(st, b, sc)


def test_topk_kernel_ties_and_lengths(tsa):
    """Top-k on crafted scores: heavy ties, every length class, up to 65536 positions."""
    rng = np.random.default_rng(11)
    lens = np.array([0, 5, 64, 65, 1000, 4096, 33000, 65536], dtype=np.int32)
    k = 64
    ld = 65536
    s = np.full((len(lens), ld), np.nan, dtype=np.float32)
    for i, L in enumerate(lens):
        s[i, :L] = rng.integers(0, 3 + i, size=L).astype(np.float32)
    s[6, :33000] = 7.0                                   # all equal: first k positions
    s[7, :100] = -1.5                                    # negatives and a distinct max
    s[7, 65535] = 1e30
    p = tsa.decode_params(len(lens), 8, k, ld, 1.0)
    out = torch.empty((len(lens), k), dtype=torch.int32, device="cuda")
    tsa.topk(p, torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i, L in enumerate(lens):
        assert np.array_equal(got[i], otopk.select_padded(s[i, :L], k)), f"row {i}"


def test_topk_random_floats(tsa):
    rng = np.random.default_rng(12)
    B, L, k = 16, 20000, 2048
    s = rng.standard_normal((B, L)).astype(np.float32)
    s[:, ::7] = np.round(s[:, ::7], 1)                   # some duplicated values
    lens = rng.integers(1, L + 1, size=B).astype(np.int32)
    p = tsa.decode_params(B, 8, k, L, 1.0)
    out = torch.empty((B, k), dtype=torch.int32, device="cuda")
    tsa.topk(p, torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b], otopk.select_padded(s[b, :lens[b]], k)), f"row {b}"


@pytest.mark.parametrize("max_len", [300, 901, 2000, 3000, 8000, 12001, 16000, 24000, 32768, 48000, 65536])
def test_topk_every_launch_shape(tsa, max_len):
    """One max length per launch shape of the top-k (512 threads with 1, 2 or 4 scores each up to
    2,048 scores, then 1,024 threads with 4 .. 64):
    rows of floats with repeated values, integer-valued rows with many ties, and a row of one
    repeated value; lengths drawn up to max_len (two odd maxima take the scalar score loads).
    Bit-exact against the oracle's selection."""
    rng = np.random.default_rng(max_len)
    B, k = 8, 512
    s = rng.standard_normal((B, max_len)).astype(np.float32)
    s[:, ::5] = np.round(s[:, ::5], 1)
    s[2:5] = np.maximum(0, np.round(rng.normal(0, 75, size=(3, max_len)))).astype(np.float32)
    s[5] = 3.0
    lens = rng.integers(1, max_len + 1, size=B).astype(np.int32)
    lens[0] = max_len
    p = tsa.decode_params(B, 8, k, max_len, 1.0)
    out = torch.empty((B, k), dtype=torch.int32, device="cuda")
    print(f"[topk] max_len {max_len}", flush=True)
    tsa.topk(p, torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b], otopk.select_padded(s[b, :lens[b]], k)), f"row {b}, len {lens[b]}"


@pytest.mark.parametrize("L", [700, 6000, 20000])
def test_topk_signed_zeros_and_nans(tsa, L):
    """Scores compared as floats, as the oracle does: -0 equals +0 (ties by position) and a NaN
    ranks below every number (NaNs by position).  Row 0 is mostly zeros of both signs with NaNs,
    row 1 needs some of its NaNs, row 2 is zeros of both signs and a few denormals of either sign
    (kept apart from the zeros: no flush to zero); these three take the register passes at every
    length.  Row 3 has fewer positive scores than k, then zeros of both signs, NaNs and negative
    scores: the k-th score is a zero, and at 20,000 scores the row takes the sampled list.  The
    lengths cover the 512-thread launch (700) and two 1,024-thread ones."""
    rng = np.random.default_rng(21 + L)
    k = 64 if L < 2048 else 512
    s = np.zeros((4, L), dtype=np.float32)
    s[0] = np.round(rng.normal(0, 0.2, size=L))            # mostly zeros: the k-th score is 0
    s[0, rng.choice(L, L // 20, replace=False)] = np.nan
    s[0, ::3] = -s[0, ::3]                                 # -0 among the zeros
    s[1] = np.nan
    s[1, rng.choice(L, L // 15, replace=False)] = -0.0
    s[1, rng.choice(L, k // 10, replace=False)] = 1.5
    s[2] = np.where(rng.random(L) < 0.5, -0.0, 0.0)
    s[2, rng.choice(L, 40, replace=False)] = np.float32(1e-40)    # denormals rank above the zeros
    s[2, rng.choice(L, 40, replace=False)] = np.float32(-1e-40)   # ... and below them
    order = rng.permutation(L)
    n_pos, n_zero, n_nan = 3 * k // 4, 4 * k, L // 100
    s[3] = rng.normal(-3, 1, size=L)
    s[3, order[:n_pos]] = rng.normal(5, 1, size=n_pos)
    s[3, order[n_pos:n_pos + n_zero]] = np.where(rng.random(n_zero) < 0.5, -0.0, 0.0)
    s[3, order[n_pos + n_zero:n_pos + n_zero + n_nan]] = np.nan
    lens = np.full(4, L, dtype=np.int32)
    p = tsa.decode_params(4, 8, k, L, 1.0)
    out = torch.empty((4, k), dtype=torch.int32, device="cuda")
    print(f"[topk] signed zeros, L {L}", flush=True)
    tsa.topk(p, torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.signbit(s[0][s[0] == 0]).any() and np.signbit(s[2]).any() and np.signbit(s[3][s[3] == 0]).any()
    for b in range(4):
        assert np.array_equal(got[b], otopk.select_padded(s[b], k)), f"row {b}"


def test_gather_given_positions(tsa):
    """Attention over caller-given positions, with invalid entries to skip."""
    st = staged("tiny_b5")
    w = st.w
    rng = np.random.default_rng(3)
    idx = np.full((5, w.top_k), -1, dtype=np.int32)
    for b in range(5):
        L = int(st.lens[b])
        n = min(L, 40)
        idx[b, :n] = rng.choice(L, size=n, replace=False)
        idx[b, n:n + 3] = [L, L + 100, -7]               # out of range: ignored
    out = torch.empty_like(st.out)
    tsa.sparse_attn_gather(st.pool, 0, st.params, st.q, torch.from_numpy(idx).cuda(), st.table_dev,
                           st.lens_dev, out, st.workspace)
    torch.cuda.synchronize()
    for b in range(5):
        L = int(st.lens[b])
        _, kk, vv = synth.request_tokens(w, 0, b, L)
        sel = idx[b][(idx[b] >= 0) & (idx[b] < L)]
        ref = decode.attend_positions(st.q_np[b], kk, vv, sel, w.sm_scale)
        assert sdpa.normwise_rel_err(out[b].double().cpu().numpy(), ref) < ATOL_REL


def test_append_skips_bad_tokens(tsa):
    st = staged("tiny_b5")
    w = st.w
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    before = st.pool.k.clone()
    req = torch.tensor([7, 0, -1, 1], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0, 5000, 0, -3], dtype=torch.int32, device="cuda")
    k = torch.zeros((4, w.num_kv_heads, w.head_dim_k), dtype=torch.int16, device="cuda")
    v = torch.zeros((4, w.num_kv_heads, w.head_dim_v), dtype=torch.int16, device="cuda")
    st.pool.append(0, req, pos, st.table_dev, 5, k, v, None, bad_dev=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 4
    # bit patterns: slots never written hold whatever the allocation held, NaNs included
    assert torch.equal(before.view(torch.int16), st.pool.k.view(torch.int16))


def test_mla_full_size_all_requests(tsa):
    """The benchmark's workload (64 requests x 32768 tokens, top-2048, one 576-dim latent head
    for 64 query heads) in the benchmark's launch configuration; every request checked whole
    against the oracle (scores and top-k sets bit-exact, attention within the bar)."""
    st = staged("mla_b64_32k")
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    errs = _check_all_requests(st, sc)
    print(f"mla_b64_32k: {len(errs)} requests, max normwise attention error {max(errs):.3e}")
    tk = st.topk.cpu().numpy()
    assert (np.diff(tk, axis=1) > 0).all() and tk.min() >= 0 and tk.max() < 32768
    assert torch.isfinite(st.out).all()


def test_mla_ih64_full_size_all_requests(tsa):
    """The 64 x 32k latent workload with a 64-head indexer on the matrix cores, in the launch
    configuration the benchmark uses for it: every request checked whole (scores bit-exact,
    top-k sets, attention)."""
    st = staged("mla_b64_32k_ih64")
    assert st.params.index_heads == 64
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    errs = _check_all_requests(st, sc)
    print(f"mla_b64_32k_ih64: {len(errs)} requests, max normwise attention error {max(errs):.3e}")
    tk = st.topk.cpu().numpy()
    assert (np.diff(tk, axis=1) > 0).all() and tk.min() >= 0 and tk.max() < 32768


@pytest.mark.parametrize("heads", [16, 32, 48, 128])
def test_mla_head_counts_match_oracle(tsa, heads):
    """The latent kernel at other query-head counts (GLM5.3 page, roofline paragraph: 64 heads
    for GLM-5, about 128 for DeepSeek V3.2): 128 heads run as two 64-head blocks, 16 / 32 / 48
    heads fill one block in part.  4 requests x 32,768 tokens, top-2048, every request checked."""
    st = staged("mla_b64_32k", {"num_q_heads": heads}, batch=4)
    assert st.params.num_q_heads == heads
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    errs = _check_all_requests(st, sc)
    print(f"latent, {heads} heads: max normwise attention error {max(errs):.3e}")


def test_mla_h128_full_size_all_requests(tsa):
    """The 64 x 32k latent workload with 128 query heads, in the benchmark's launch configuration:
    every request checked whole against the oracle."""
    st = staged("mla_b64_32k_h128")
    assert st.params.num_q_heads == 128
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    errs = _check_all_requests(st, sc)
    print(f"mla_b64_32k_h128: {len(errs)} requests, max normwise attention error {max(errs):.3e}")


def test_mla_mha_mode_matches_oracle(tsa):
    """The MHA mode of latent attention (64 heads, each with a 192-dim key and a 128-dim value of
    its own) through the whole step, on the grouped-query kernel with one query head per KV head:
    scores, top-2048 of 4096, attention."""
    st = staged("mla_mha_b64_4k", batch=4)
    assert st.pool.desc.num_kv_heads == 64 and st.pool.desc.head_dim_k == 192
    sc = _scores_gpu(tsa, st)
    st.step()
    torch.cuda.synchronize()
    errs = [_check_request(st, b, sc) for b in range(4)]
    print(f"mla_mha_b64_4k: max normwise attention error {max(errs):.3e}")


def test_mla_large_logits_take_the_rescan_path(tsa):
    """Queries scaled so that logits span far more than 2^32 between the first tile of a split
    and later tiles: the latent kernel must detect it, rescan for the true max and still match
    the oracle (softmax over float64 logits)."""
    st = staged("mla_b64_32k", batch=2)
    w = st.w
    rng = np.random.default_rng(21)
    q = synth.f32_to_bf16_bits((rng.standard_normal((2, 64, 576)) * 60).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(int(st.lens[b]), size=w.top_k, replace=False)) for b in range(2)])
    idx = idx.astype(np.int32)
    out = torch.empty((2, 64, 512), dtype=torch.float32, device="cuda")
    tsa.sparse_attn_gather(st.pool, 0, st.params, torch.from_numpy(q.view(np.int16)).cuda(),
                           torch.from_numpy(idx).cuda(), st.table_dev, st.lens_dev, out, st.workspace)
    torch.cuda.synchronize()
    for b in range(2):
        _, kk, _ = synth.request_tokens(w, 0, b, int(st.lens[b]))
        ref = decode.attend_positions(q[b], kk, None, idx[b], w.sm_scale, v_from_k_dims=512)
        err = sdpa.normwise_rel_err(out[b].double().cpu().numpy(), ref)
        assert err < ATOL_REL, f"request {b}: {err}"
