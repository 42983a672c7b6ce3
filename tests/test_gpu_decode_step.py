"""tsa_decode_step: the decode step with each request's new token written at position seq_len - 1
inside the step (fused into the scoring launch for one-head indexers on the streaming kernel, a
separate launch for several heads or small pages; contexts of at most 1024 tokens run the one-launch
step).  Its outputs must equal the separate calls (kv_append, then the whole step) bit for
bit, and the oracle's within the attention bar; a token whose page is missing is counted and
not written.
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
    """Rows [B, ...] of every request's last token (zeros for empty requests)."""
    B = len(st.lens)
    def full(src):
        if src is None:
            return None
        out = torch.zeros((B,) + tuple(src.shape[1:]), dtype=src.dtype, device="cuda")
        out[st.new_req.long()] = src
        return out
    return full(st.new_k), full(st.new_v), full(st.new_idx)


def _scramble_last(st):
    """Overwrite every request's last token in the pool with zeros (what the step must restore)."""
    zk = torch.zeros_like(st.new_k)
    zv = None if st.new_v is None else torch.zeros_like(st.new_v)
    zi = torch.zeros_like(st.new_idx)
    st.pool.append(0, st.new_req, st.new_pos, st.table_dev, len(st.lens), zk, zv, zi)


@pytest.mark.parametrize("name,kw", [("tiny_b5", {}), ("gqa_b32_8k", {"batch": 6}),
                                     ("mla_b64_32k", {"batch": 3}),
                                     ("gqa_b32_8k", {"batch": 4, "index_heads": 16}),
                                     ("gqa_b32_8k", {"lens": np.array([1, 9, 300, 2000], np.int32), "page_size": 8}),
                                     ("prefix_b128_16k", {"batch": 6})])
def test_decode_step_equals_separate_calls(tsa, name, kw):
    st = _stage(name, **kw)
    kn, vn, inew = _new_rows(st)
    # reference: the separate calls
    st.pool.append(0, st.new_req, st.new_pos, st.table_dev, len(st.lens), st.new_k, st.new_v, st.new_idx)
    tsa.sparse_decode_attn(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                           st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    ref_o, ref_t = st.out.clone(), st.topk.clone()
    pool_ref = st.pool.k.view(torch.int16).clone()
    for rep in range(2):
        _scramble_last(st)
        st.out.fill_(float("nan"))
        st.topk.fill_(-7)
        bad = torch.zeros(1, dtype=torch.int32, device="cuda")
        tsa.decode_step(st.pool, 0, st.params, kn, vn, inew, st.q, st.qidx, st.widx, st.table_dev,
                        st.lens_dev, st.out, st.workspace, topk_out=st.topk, bad=bad)
        torch.cuda.synchronize()
        assert int(bad.item()) == 0
        assert torch.equal(st.pool.k.view(torch.int16), pool_ref), "pool rows differ"
        assert torch.equal(st.topk, ref_t), f"top-k differs (round {rep})"
        if st.params.max_len <= 1024:
            # short contexts take the one-launch step: one split instead of several, so the
            # attention equals the separate calls up to fp32 rounding
            err = (st.out - ref_o).abs().max().item() / max(ref_o.abs().max().item(), 1e-30)
            assert err < 1e-5, f"attention differs by {err:.3g} (round {rep})"
        else:
            assert torch.equal(st.out, ref_o), f"attention differs (round {rep})"
    # and the oracle, on the first requests
    w = st.w
    for b in range(min(3, len(st.lens))):
        L = int(st.lens[b])
        if L == 0:
            continue
        kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
        _, sel, o_ref = decode.request_step(st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv, w.top_k,
                                            w.sm_scale, v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
        tk = st.topk[b].cpu().numpy()
        assert np.array_equal(tk[:len(sel)], sel) and (tk[len(sel):] == -1).all()
        assert sdpa.normwise_rel_err(st.out[b].double().cpu().numpy(), o_ref) < 2e-3


def test_decode_step_counts_missing_pages(tsa):
    st = _stage("tiny_b5")
    kn, vn, inew = _new_rows(st)
    table = st.table.copy()
    b0 = 2
    last_page = (int(st.lens[b0]) - 1) // st.w.page_size
    table[b0, last_page] = -1                 # the new token's page is gone
    tdev = torch.from_numpy(table).cuda()
    before = st.pool.k.view(torch.int16).clone()
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    tsa.decode_step(st.pool, 0, st.params, kn * 0, vn * 0 if vn is not None else None, inew * 0, st.q,
                    st.qidx, st.widx, tdev, st.lens_dev, st.out, st.workspace, topk_out=st.topk, bad=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1
    # every other request's last token was overwritten with zeros; request b0's page was not touched
    changed = (before != st.pool.k.view(torch.int16)).reshape(-1, st.w.num_kv_heads * st.w.head_dim_k).any(dim=1)
    P = st.w.page_size
    rows_changed = set(torch.nonzero(changed).flatten().tolist())
    expected = set()
    for b in range(len(st.lens)):
        L = int(st.lens[b])
        if L == 0 or b == b0:
            continue
        pg = int(table[b, (L - 1) // P])
        slot = pg * P + (L - 1) % P
        if before.reshape(-1, st.w.num_kv_heads * st.w.head_dim_k)[slot].any():
            expected.add(slot)
    assert rows_changed == expected


def test_decode_step_argument_checks(tsa):
    st = _stage("tiny_b5")
    kn, vn, inew = _new_rows(st)
    with pytest.raises(tsa.TsaError, match="v_new"):
        tsa.decode_step(st.pool, 0, st.params, kn, None, inew, st.q, st.qidx, st.widx, st.table_dev,
                        st.lens_dev, st.out, st.workspace)
    with pytest.raises(tsa.TsaError, match="NULL new"):
        tsa.decode_step(st.pool, 0, st.params, None, vn, inew, st.q, st.qidx, st.widx, st.table_dev,
                        st.lens_dev, st.out, st.workspace)
