"""The captured step (tsa_step_graph_*): every replay equals the eager step bit for bit.

A graph records the same launches as the eager entry points, so its outputs must be identical,
replay after replay, with eager work and synchronisations between replays; it must also read
the current contents of its buffers (new queries) rather than values frozen at capture.
"""
import numpy as np
import pytest

import synth

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


def _eager(tsa, st):
    st.pool.append(0, st.new_req, st.new_pos, st.table_dev, len(st.lens), st.new_k, st.new_v, st.new_idx)
    tsa.sparse_decode_attn(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                           st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    return st.out.clone(), st.topk.clone()


@pytest.mark.parametrize("name,kw", [("tiny_b5", {}), ("gqa_b32_8k", {"batch": 8}),
                                     ("mla_b64_32k", {"batch": 4})])
def test_graph_replays_equal_eager(tsa, name, kw):
    st = _stage(name, **kw)
    out_ref, tk_ref = _eager(tsa, st)
    g = tsa.StepGraph(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                      st.out, st.workspace, topk_out=st.topk,
                      append=(st.new_req, st.new_pos, st.new_k, st.new_v, st.new_idx, None))
    for r in range(4):
        st.out.fill_(float("nan"))
        st.topk.fill_(-7)
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(st.topk, tk_ref), f"replay {r}: top-k differs"
        assert torch.equal(st.out, out_ref), f"replay {r}: output differs"
        _eager(tsa, st)                       # eager work between replays
    g.close()


def test_graph_reads_current_buffers(tsa):
    st = _stage("gqa_b32_8k", batch=6)
    g = tsa.StepGraph(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                      st.out, st.workspace, topk_out=st.topk)
    rng = np.random.default_rng(5)
    for r in range(3):
        qn = synth.f32_to_bf16_bits(rng.standard_normal(tuple(st.q.shape)).astype(np.float32))
        st.q.copy_(torch.from_numpy(qn.view(np.int16)).cuda())
        r_ = st.qidx.clone()
        st.qidx.copy_(torch.flip(r_, dims=[0]))          # other indexer queries, same shape
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        got_o, got_t = st.out.clone(), st.topk.clone()
        tsa.sparse_decode_attn(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                               st.out, st.workspace, topk_out=st.topk)
        torch.cuda.synchronize()
        assert torch.equal(got_t, st.topk) and torch.equal(got_o, st.out), f"round {r}"
    g.close()


def test_graph_create_checks_like_eager(tsa):
    st = _stage("tiny_b5")
    bad = tsa.decode_params(len(st.lens), st.params.num_q_heads, st.params.top_k, st.params.max_len,
                            st.params.sm_scale, index_heads=99)
    with pytest.raises(tsa.TsaError, match="index_heads"):
        tsa.StepGraph(st.pool, 0, bad, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                      st.out, st.workspace, topk_out=st.topk)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tsa.TsaError, match="workspace"):
        tsa.StepGraph(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev, st.lens_dev,
                      st.out, small, topk_out=st.topk)
    # the library still works after a refused capture
    _eager(tsa, st)
