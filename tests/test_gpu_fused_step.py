"""tsa_decode_step_fused: the whole decode step of each request in one workgroup, one launch.

Bar: the pool rows it writes and the top-k sets equal the separate calls (kv_append, then the
whole step) bit for bit, and the oracle's; attention within fp32 rounding of the separate calls
and within 2e-3 of the oracle.  Cases: the tiny worked example, ragged lengths with 8-token
pages (an empty request, contexts shorter than top_k, a 1-token context, several tiles), several indexer heads,
one query head per KV head with 192/128 dims (the MHA mode of latent attention), dense and
sparse requests in one batch, the latent layout with aliased values, and a missing page.
"""
import numpy as np
import pytest

import synth
from oracle import decode, sdpa

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_sparse_attention_amd as m
    m.load()
    return m


def _stage(name, **kw):
    from top_sparse_attention_amd import workload
    print(f"[stage] {name} {kw}", flush=True)
    return workload.stage(synth.get(name), **kw)


def _new_rows(st):
    B = len(st.lens)

    def full(src):
        if src is None:
            return None
        out = torch.zeros((B,) + tuple(src.shape[1:]), dtype=src.dtype, device="cuda")
        out[st.new_req.long()] = src
        return out
    return full(st.new_k), full(st.new_v), full(st.new_idx)


def _scramble_last(st):
    zk = torch.zeros_like(st.new_k)
    zv = None if st.new_v is None else torch.zeros_like(st.new_v)
    zi = torch.zeros_like(st.new_idx)
    st.pool.append(0, st.new_req, st.new_pos, st.table_dev, len(st.lens), zk, zv, zi)


def _pool_bits(st):
    parts = [st.pool.k, st.pool.idx] + ([st.pool.v] if st.pool.v is not None else [])
    return [x.view(torch.int16).clone() for x in parts]


CASES = [
    ("tiny_b5", {}),
    ("gqa_b32_8k", {"lens": np.array([1, 9, 0, 300, 1000, 777, 513], np.int32), "page_size": 8}),
    ("gqa_b32_8k", {"lens": np.array([2048, 4100, 3000], np.int32), "index_heads": 4}),
    ("gqa_b32_8k", {"lens": np.array([700, 64, 65, 5000], np.int32), "index_heads": 8, "page_size": 16}),
    ("mla_mha_b64_4k", {"lens": np.array([100, 257], np.int32)}),
]


@pytest.mark.parametrize("name,kw", CASES + [
    # the latent layout (values are the first 512 dims of the 576-dim key row) with 4 query heads:
    # aliased values, 32-row tiles, and a sparse selection of 2048 out of 5000 positions
    ("mla_b64_32k", {"q_heads": 4, "lens": np.array([300, 2049, 5000], np.int32)})])
def test_fused_step_equals_separate_calls_and_oracle(tsa, name, kw):
    kw = dict(kw)
    hq = kw.pop("q_heads", None)
    if hq is None:
        st = _stage(name, **kw)
    else:
        import dataclasses
        from top_sparse_attention_amd import workload
        print(f"[stage] {name} q_heads={hq} {kw}", flush=True)
        st = workload.stage(dataclasses.replace(synth.get(name), num_q_heads=hq), **kw)
    kn, vn, inew = _new_rows(st)
    st.pool.append(0, st.new_req, st.new_pos, st.table_dev, len(st.lens), st.new_k, st.new_v, st.new_idx)
    tsa.sparse_decode_attn(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                           st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    ref_o, ref_t = st.out.clone(), st.topk.clone()
    pool_ref = _pool_bits(st)
    first = None
    for rep in range(2):
        _scramble_last(st)
        st.out.fill_(float("nan"))
        st.topk.fill_(-7)
        bad = torch.zeros(1, dtype=torch.int32, device="cuda")
        tsa.decode_step_fused(st.pool, 0, st.params, kn, vn, inew, st.q, st.qidx, st.widx, st.table_dev,
                              st.lens_dev, st.out, topk_out=st.topk, bad=bad)
        torch.cuda.synchronize()
        assert int(bad.item()) == 0
        for got, ref in zip(_pool_bits(st), pool_ref):
            assert torch.equal(got, ref), "pool rows differ"
        assert torch.equal(st.topk, ref_t), f"top-k differs (round {rep})"
        assert not torch.isnan(st.out).any()
        for b in np.nonzero(st.lens == 0)[0]:     # an empty request: zeros and no selection
            assert not st.out[b].any() and (st.topk[b] == -1).all()
        err = (st.out - ref_o).abs().max().item() / max(ref_o.abs().max().item(), 1e-30)
        assert err < 1e-5, f"attention differs from the separate calls by {err:.3g} (round {rep})"
        if first is None:
            first = st.out.clone()
        else:
            assert torch.equal(st.out, first), "two runs differ"
    w = st.w
    for b in range(len(st.lens)):
        L = int(st.lens[b])
        if L == 0:
            continue
        kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
        _, sel, o_ref = decode.request_step(st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv, w.top_k,
                                            w.sm_scale, v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
        tk = st.topk[b].cpu().numpy()
        assert np.array_equal(tk[:len(sel)], sel) and (tk[len(sel):] == -1).all(), f"request {b}"
        assert sdpa.normwise_rel_err(st.out[b].double().cpu().numpy(), o_ref) < 2e-3, f"request {b}"


def test_decode_step_takes_the_one_launch_path_for_short_contexts(tsa):
    """tsa_decode_step on the tiny example runs the same kernel: bit-identical outputs."""
    st = _stage("tiny_b5")
    kn, vn, inew = _new_rows(st)
    tsa.decode_step_fused(st.pool, 0, st.params, kn, vn, inew, st.q, st.qidx, st.widx, st.table_dev,
                          st.lens_dev, st.out, topk_out=st.topk)
    torch.cuda.synchronize()
    o1, t1 = st.out.clone(), st.topk.clone()
    st.out.fill_(float("nan"))
    tsa.decode_step(st.pool, 0, st.params, kn, vn, inew, st.q, st.qidx, st.widx, st.table_dev,
                    st.lens_dev, st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    assert torch.equal(st.out, o1) and torch.equal(st.topk, t1)


def test_fused_step_counts_missing_pages(tsa):
    st = _stage("gqa_b32_8k", lens=np.array([40, 300, 17], np.int32), page_size=8)
    kn, vn, inew = _new_rows(st)
    table = st.table.copy()
    b0 = 1
    P = st.pool.desc.page_size
    table[b0, (int(st.lens[b0]) - 1) // P] = -1
    tdev = torch.from_numpy(table).cuda()
    before = _pool_bits(st)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    tsa.decode_step_fused(st.pool, 0, st.params, kn * 0, vn * 0, inew * 0, st.q, st.qidx, st.widx, tdev,
                          st.lens_dev, st.out, topk_out=st.topk, bad=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1
    assert not torch.isnan(st.out).any()
    # the page of request b0's new token was not written; its top-k still holds valid positions
    pg = int(st.table[b0, (int(st.lens[b0]) - 1) // P])
    row = pg * P + (int(st.lens[b0]) - 1) % P
    k_now = st.pool.k.view(torch.int16).reshape(-1, st.w.num_kv_heads * st.w.head_dim_k)
    k_before = before[0].reshape(-1, st.w.num_kv_heads * st.w.head_dim_k)
    assert torch.equal(k_now[row], k_before[row])
    tk = st.topk[b0].cpu().numpy()
    valid = tk[tk >= 0]
    assert np.all(np.diff(valid) > 0) and valid.max() < int(st.lens[b0])


def test_fused_step_refuses_shapes_beyond_its_limits(tsa):
    st = _stage("mla_b64_32k", batch=1)     # 64 q heads x 512 value dims on one KV head
    kn, vn, inew = _new_rows(st)
    with pytest.raises(tsa.TsaError, match="one-launch"):
        tsa.decode_step_fused(st.pool, 0, st.params, kn, vn, inew, st.q, st.qidx, st.widx, st.table_dev,
                              st.lens_dev, st.out, topk_out=st.topk)
