"""Tie-heavy indexer scores through the whole long-context latent step, against the oracle.

The 64 x 32k latent workload's scores are integers from values in [-4, 4]: a few dozen ties at
the k-th score.  Here the same step (576/512 latent head, 64 query heads, top-2048, one indexer
head of 128 dims) runs on ragged batches whose indexer values are drawn from [-4, 4], from
[-1, 1] (hundreds of ties at the k-th score, many scores of 0 after the ReLU) and from {0} (every
score 0, so the selection is decided by position alone).  The batches hold full 32k contexts,
lengths just above and at top_k (dense) and an empty request.  Top-k sets must equal the
oracle's and the one-workgroup top-k kernel's on the same scores bit for bit, every selected
position the step writes is checked, and attention must be within the 2e-3 bar.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import decode, sdpa

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL_REL = 2e-3
LENS = np.array([32768, 2049, 32768, 2048, 0, 20001, 9000], dtype=np.int32)


@pytest.fixture(scope="module")
def tsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_sparse_attention_amd as m
    m.load()
    return m


@pytest.mark.parametrize("index_range", [4, 1, 0])
def test_tie_heavy_step_matches_oracle(tsa, index_range):
    from top_sparse_attention_amd import workload
    w = dataclasses.replace(synth.get("mla_b64_32k"), index_range=index_range)
    print(f"[tie-heavy step] index_range {index_range} lens {LENS.tolist()}", flush=True)
    st = workload.stage(w, seed=3, lens=LENS)
    B = len(LENS)
    ld = max(64, -(-st.params.max_len // 64) * 64)
    sc = torch.full((B, ld), float("nan"), dtype=torch.float32, device="cuda")
    tsa.indexer_scores(st.pool, 0, st.params, st.qidx, st.widx, st.table_dev, st.lens_dev, sc)
    st.topk.fill_(-7)
    st.step(append=False)
    ref_topk = torch.full_like(st.topk, -7)
    tsa.topk(st.params, sc, st.lens_dev, ref_topk)
    torch.cuda.synchronize()
    got = st.topk.cpu().numpy()
    assert np.array_equal(got, ref_topk.cpu().numpy()), "the step's selection differs from the top-k kernel on the same scores"
    scores = sc.cpu().numpy()
    out = st.out.double().cpu().numpy()
    worst = 0.0
    for b in range(B):
        L = int(LENS[b])
        if L == 0:
            assert (got[b] == -1).all(), "an empty request selects nothing"
            assert not np.any(out[b]), "an empty request's output is zero"
            continue
        kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
        s_ref, sel_ref, o_ref = decode.request_step(st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv,
                                                    w.top_k, w.sm_scale, v_from_k_dims=w.head_dim_v)
        assert np.array_equal(scores[b, :L].astype(np.float64), np.asarray(s_ref, np.float64)), f"scores, request {b}"
        exp = np.full(w.top_k, -1, dtype=np.int32)
        exp[:len(sel_ref)] = sel_ref
        assert np.array_equal(got[b], exp), f"top-k differs from the oracle, request {b}"
        err = sdpa.normwise_rel_err(out[b], o_ref)
        assert err < ATOL_REL, f"attention error {err} on request {b}"
        worst = max(worst, err)
    print(f"index_range {index_range}: max normwise attention error {worst:.3e}")
