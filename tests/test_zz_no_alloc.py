"""The decode step that allocates nothing (tsa_decode_step_noalloc, workspace in the library's
own scratch array) against tsa_decode_step with a caller workspace, through the C ABI.

Two calls in a row share the one scratch array: first the latent workload at 8 requests x 32,768
tokens (top-2048; its split partials fill about 40 MiB of the array), then a smaller grouped-query
input (4 requests of 2,048..8,192 tokens, top-512).  Each call must give the same top-k sets and
attention outputs as the caller-workspace step (the same kernels: bit-identical), and both must
match the oracle (top-k sets exact, attention within 2e-3 normwise).
"""
import dataclasses

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


def _run(tsa, name, batch):
    from top_sparse_attention_amd import workload
    from oracle_pool import oracle_requests
    print(f"[no-alloc] staging {name} batch {batch}", flush=True)
    st = workload.stage(dataclasses.replace(synth.get(name)), batch=batch)
    B = len(st.lens)
    assert st.new_req is not None and len(st.new_req) == B
    tsa.decode_step(st.pool, 0, st.params, st.new_k, st.new_v, st.new_idx, st.q, st.qidx, st.widx,
                    st.table_dev, st.lens_dev, st.out, st.workspace, topk_out=st.topk)
    torch.cuda.synchronize()
    out_ws, topk_ws = st.out.clone(), st.topk.clone()
    st.out.fill_(float("nan"))
    st.topk.fill_(-7)
    tsa.decode_step_noalloc(st.pool, 0, st.params, st.new_k, st.new_v, st.new_idx, st.q, st.qidx,
                            st.widx, st.table_dev, st.lens_dev, st.out, topk_out=st.topk)
    torch.cuda.synchronize()
    assert torch.equal(st.topk, topk_ws)
    assert torch.equal(st.out, out_ws)
    ref = oracle_requests(st.w, st.seed, range(B), st.q_np, st.qidx_np, st.widx_np)
    tk = st.topk.cpu().numpy()
    out = st.out.double().cpu().numpy()
    errs = []
    for b in range(B):
        _, sel, o_ref = ref[b]
        exp = np.full(st.w.top_k, -1, dtype=np.int32)
        exp[:len(sel)] = sel
        assert np.array_equal(tk[b], exp), f"top-k differs, request {b}"
        errs.append(sdpa.normwise_rel_err(out[b], o_ref))
    assert max(errs) < ATOL_REL, max(errs)
    print(f"[no-alloc] {name} batch {batch}: max normwise error {max(errs):.3e}", flush=True)
    return st


def test_no_alloc_step_twice_second_smaller(tsa):
    big = _run(tsa, "mla_b64_32k", 8)
    need_big = tsa.workspace_bytes(big.pool, big.params)
    assert need_big > 32 << 20            # the first call uses most of the array
    del big
    torch.cuda.empty_cache()
    small = _run(tsa, "gqa_b32_8k", 4)
    assert tsa.workspace_bytes(small.pool, small.params) < need_big


def test_no_alloc_refuses_a_step_beyond_its_scratch(tsa):
    """A step whose workspace exceeds 64 MiB is refused with TSA_ERR_CAPACITY before any launch
    (256 requests x 65,536 tokens of scores alone need 64 MiB)."""
    from top_sparse_attention_amd import KvPool, _lib
    pool = KvPool(64, 64, 1, 576, 512, v_from_k=True, index_dim=128, allocate=True)
    p = tsa.decode_params(256, 64, 2048, 65536, 1.0 / 24.0)
    assert tsa.workspace_bytes(pool, p) > 64 << 20
    dummy = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(tsa.TsaError) as e:
        tsa.decode_step_noalloc(pool, 0, p, dummy, None, dummy, dummy, dummy,
                                dummy.float(), torch.zeros((256, 1024), dtype=torch.int32, device="cuda"),
                                dummy, dummy.float())
    assert e.value.status == _lib.TSA_ERR_CAPACITY
