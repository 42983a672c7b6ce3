"""Grouped-query attention with the splits of each (request, KV head) merged inside one workgroup.

With 64 to 256 (request, KV head) pairs the grouped-query matrix-core kernel runs the four splits
of a pair as the four waves of one workgroup and merges their running max, sum and accumulator
through LDS, with no partials in memory and no combine launch.  These shapes put it through
ragged batches whose lengths leave some waves a partial tile or no tokens at all (0, 1, around
one tile and around top_k), 64- and 128-dim heads, 1 to 16 query heads per KV head and selections
of 130 to 2,048 tokens.  Top-k sets must equal the oracle's and attention must be within the
2e-3 bar on every request.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import decode, sdpa

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ATOL_REL = 2e-3

# (head dim, KV heads, query heads per KV head, top_k, batch)
SHAPES = [(128, 4, 8, 512, 32), (64, 8, 16, 130, 16), (128, 2, 1, 2048, 64), (128, 8, 4, 200, 8),
          (128, 2, 8, 2048, 100)]   # the last: the tiered workload's head shape at 100 requests


@pytest.fixture(scope="module")
def tsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_sparse_attention_amd as m
    m.load()
    return m


@pytest.mark.parametrize("shape", SHAPES)
def test_gqa_workgroup_merge_matches_oracle(tsa, shape):
    from top_sparse_attention_amd import workload
    d, hkv, g, k, B = shape
    w = dataclasses.replace(synth.get("gqa_b32_8k"), head_dim_k=d, head_dim_v=d, num_kv_heads=hkv,
                            num_q_heads=hkv * g, top_k=k)
    rng = np.random.default_rng(7 + d + k)
    lens = rng.integers(1, 8193, size=B).astype(np.int32)
    edges = [0, 1, 31, 32, 33, k - 1, k, k + 1, 4 * 32 - 1, 8192]
    lens[:len(edges)] = edges[:B]
    print(f"[gqa merge] dims {d} kv heads {hkv} q heads per kv {g} top_k {k} lens {lens.tolist()}", flush=True)
    st = workload.stage(w, seed=5, lens=lens)
    st.step(append=False)
    torch.cuda.synchronize()
    got = st.topk.cpu().numpy()
    out = st.out.double().cpu().numpy()
    worst = 0.0
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            assert (got[b] == -1).all() and not np.any(out[b]), f"empty request {b}"
            continue
        kidx, kk, vv = synth.request_tokens(w, st.seed, b, L)
        _, sel_ref, o_ref = decode.request_step(st.q_np[b], st.qidx_np[b], st.widx_np, kidx, kk, vv, w.top_k,
                                                w.sm_scale, v_from_k_dims=0)
        exp = np.full(k, -1, dtype=np.int32)
        exp[:len(sel_ref)] = sel_ref
        assert np.array_equal(got[b], exp), f"top-k differs, request {b}"
        err = sdpa.normwise_rel_err(out[b], o_ref)
        assert err < ATOL_REL, f"attention error {err} on request {b} (length {L})"
        worst = max(worst, err)
    print(f"max normwise attention error {worst:.3e}")
