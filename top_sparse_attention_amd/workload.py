"""Stage a synthetic workload on the GPU through libtsa (set-up path of tests and benchmarks).

Draws inputs from ``synth`` (seeded random numbers only), builds the pool and page tables
with the library, fills the pool with ``tsa_kv_append`` and keeps every device tensor a
decode step needs.  Nothing here computes any part of the step itself.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import KvPool, decode_params, sparse_decode_attn, workspace_bytes


def _dev(a: np.ndarray, device):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclasses.dataclass
class Staged:
    w: object
    seed: int
    lens: np.ndarray
    pool: KvPool
    table: np.ndarray
    num_pages: np.ndarray
    saved: int
    max_pages: int
    params: object
    table_dev: object
    lens_dev: object
    q: object
    qidx: object
    widx: object
    out: object
    topk: object
    workspace: object
    new_req: object = None   # the decode token of each request (re-appended by a step)
    new_pos: object = None
    new_k: object = None
    new_v: object = None
    new_idx: object = None

    def step(self, stream=None, append=True):
        """One decode step: append each request's newest token, then score, select, attend."""
        if append and self.new_req is not None:
            self.pool.append(0, self.new_req, self.new_pos, self.table_dev, len(self.lens),
                             self.new_k, self.new_v, self.new_idx, stream=stream)
        sparse_decode_attn(self.pool, 0, self.params, self.q, self.qidx, self.widx, self.table_dev,
                           self.lens_dev, self.out, self.workspace, topk_out=self.topk, stream=stream)


def stage(w, seed: int = 0, batch: Optional[int] = None, lens: Optional[np.ndarray] = None,
          free_order: Optional[np.ndarray] = None, device: str = "cuda", page_size: Optional[int] = None,
          index_heads: Optional[int] = None, fill: bool = True, share_prefix: bool = True,
          extra_pages: int = 0) -> Staged:
    """Stage workload ``w`` (a ``synth.Workload``).  ``batch`` keeps the first requests only;
    ``lens`` / ``page_size`` override the workload's (edge-case tests)."""
    import torch
    import synth

    custom = lens is not None or page_size is not None
    all_lens = synth.lens(w, seed) if lens is None else np.asarray(lens, dtype=np.int32)
    B = len(all_lens) if batch is None else int(batch)
    lens = np.ascontiguousarray(all_lens[:B], dtype=np.int32)
    P = w.page_size if page_size is None else int(page_size)
    pool_pages = w.pool_pages + int(extra_pages)
    if custom:
        pool_pages = int(sum(-(-int(L) // P) for L in lens)) + B + int(extra_pages)
    fo = synth.free_order(w, seed, pool_pages) if free_order is None else np.asarray(free_order, np.int32)
    pool = KvPool(len(fo), P, w.num_kv_heads, w.head_dim_k, w.head_dim_v, v_from_k=w.v_from_k,
                  index_dim=w.index_dim, free_order=fo, device=device)
    max_pages = max(1, int(-(-int(lens.max(initial=0)) // P)))
    grp, plen = synth.prefix_groups(w)
    if grp is not None and share_prefix:
        grp = grp[:B]
        table, num, saved = pool.build_tables(lens, max_pages, grp, plen)
    else:
        table, num, saved = pool.build_tables(lens, max_pages)
    H_I = w.index_heads if index_heads is None else int(index_heads)

    qidx_np = synth.index_queries(w, seed)[:B]
    if H_I != w.index_heads:
        rng = np.random.default_rng([seed, 77])
        r = w.index_range
        qidx_np = synth.f32_to_bf16_bits(rng.integers(-r, r + 1, size=(B, H_I, w.index_dim)).astype(np.float32))
        widx_np = rng.integers(-2, 4, size=H_I).astype(np.float32)
    else:
        widx_np = synth.index_weights(w)
    q_np = synth.queries(w, seed)[:B]

    table_dev = _dev(table, device)
    lens_dev = _dev(lens, device)
    max_len = int(lens.max(initial=0))
    params = decode_params(B, w.num_q_heads, w.top_k, max_len, w.sm_scale, index_heads=H_I)
    ws = torch.empty(max(workspace_bytes(pool, params), 256), dtype=torch.uint8, device=device)
    out = torch.empty((B, w.num_q_heads, w.head_dim_v), dtype=torch.float32, device=device)
    topk = torch.empty((B, w.top_k), dtype=torch.int32, device=device)
    st = Staged(w, seed, lens, pool, table, num, saved, max_pages, params, table_dev, lens_dev,
                _dev(q_np, device), _dev(qidx_np, device), _dev(widx_np, device), out, topk, ws)

    if fill:
        from concurrent.futures import ThreadPoolExecutor
        starts = []
        filled_prefix = set()
        for b in range(B):
            start = 0
            if grp is not None and share_prefix and grp[b] >= 0:
                g = int(grp[b])
                if g in filled_prefix:
                    start = (int(plen[g]) // P) * P     # shared full pages are already written
                filled_prefix.add(g)
            starts.append(start)
        work = [b for b in range(B) if lens[b] > 0]
        last_k, last_v, last_i = [], [], []
        with ThreadPoolExecutor(8) as ex:
            draws = ex.map(lambda b: synth.request_tokens(w, seed, b, int(lens[b]), start=starts[b]), work)
            for b, (kidx, kk, vv) in zip(work, draws):
                L, start = int(lens[b]), starts[b]
                req = torch.full((L - start,), b, dtype=torch.int32, device=device)
                pos = torch.arange(start, L, dtype=torch.int32, device=device)
                pool.append(0, req, pos, table_dev, B, _dev(kk, device),
                            None if vv is None else _dev(vv, device),
                            None if kidx is None else _dev(kidx, device))
                last_k.append(kk[-1])
                last_v.append(None if vv is None else vv[-1])
                last_i.append(None if kidx is None else kidx[-1])
        if work:
            nz = np.asarray(work, dtype=np.int32)
            st.new_req = _dev(nz, device)
            st.new_pos = _dev((lens[nz] - 1).astype(np.int32), device)
            st.new_k = _dev(np.stack(last_k), device)
            st.new_v = None if last_v[0] is None else _dev(np.stack(last_v), device)
            st.new_idx = None if last_i[0] is None else _dev(np.stack(last_i), device)
        torch.cuda.synchronize()
    st.widx_np = widx_np
    st.qidx_np = qidx_np
    st.q_np = q_np
    return st
