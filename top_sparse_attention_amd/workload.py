"""Stage a synthetic workload on the GPU through libtsa (set-up path of tests and benchmarks).

Draws inputs from ``synth`` (seeded random numbers only), builds the pool and page tables
with the library, fills the pool with ``tsa_kv_append`` and keeps every device tensor a
decode step needs.  Nothing here computes any part of the step itself.
"""
from __future__ import annotations

import dataclasses
import os
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

    qidx_np, widx_np = synth.index_inputs(w, seed, H_I, B)
    q_np = synth.queries(w, seed, B)
    if q_np.shape[0] != B or qidx_np.shape[0] != B:
        raise ValueError(f"query sets hold {q_np.shape[0]} / {qidx_np.shape[0]} rows for {B} requests")

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


@dataclasses.dataclass
class StagedTier:
    """A tiered workload: every page in pinned host memory, an HBM cache of ``cache_pages``
    slots managed by an LruTier, and the per-layer attention call over the cache."""
    w: object
    seed: int
    num_req: int
    length: int
    pages_per_req: int
    host_k: object
    host_v: object
    cache: KvPool
    tier: object
    params: object
    q: object
    lens_dev: object
    workspace: object

    def key(self, layer: int, req: int, page: int) -> int:
        return (layer * self.num_req + req) * self.pages_per_req + page

    def positions(self, step: int, layer: int, centres: dict):
        """Seeded per-(step, layer) positions for every request, int32 [num_req, top_k]."""
        import synth
        out = np.empty((self.num_req, self.w.top_k), dtype=np.int32)
        for r in range(self.num_req):
            out[r], centres[(layer, r)] = synth.tier_positions(self.w, self.seed, step, layer, r,
                                                               centres.get((layer, r)))
        return out

    def attend(self, table_dev, topk_dev, out, stream=None):
        """Attention of one layer over the cache, through its slot table."""
        from . import sparse_attn_gather
        sparse_attn_gather(self.cache, 0, self.params, self.q, topk_dev, table_dev, self.lens_dev,
                           out, self.workspace, stream=stream)


def stage_tier(w, seed: int = 0, num_req: Optional[int] = None, length: Optional[int] = None,
               num_layers: Optional[int] = None, top_k: Optional[int] = None,
               cache_pages: Optional[int] = None, unit: str = "page", device: str = "cuda") -> StagedTier:
    """Stage the tiered workload ``w`` (optionally scaled down): fill the pinned host copy of
    every (layer, request) page from ``synth`` and create an empty HBM cache.  The default
    cache holds ``w.cache_fraction`` of all pages.  ``unit`` "page" caches whole pages of
    ``w.page_size`` tokens, "token" single token rows (a cache pool with one-token pages and
    the same bytes: ``cache_pages`` pages of the workload hold that many times page_size
    token slots); the host copy is the same either way."""
    import torch
    import synth
    from . import LruTier

    R = w.batch if num_req is None else int(num_req)
    L = int(w.fixed_lens[0]) if length is None else int(length)
    NL = w.num_layers if num_layers is None else int(num_layers)
    k = w.top_k if top_k is None else int(top_k)
    w = dataclasses.replace(w, batch=R, fixed_lens=(L,) * R, num_layers=NL, top_k=k)
    P = w.page_size
    npr = -(-L // P)
    keys = NL * R * npr
    C = int(round(keys * w.cache_fraction)) if cache_pages is None else int(cache_pages)
    row = w.num_kv_heads * w.head_dim_k
    host_k = torch.empty((keys * P, row), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.empty((keys * P, row), dtype=torch.bfloat16, pin_memory=True)
    hk = host_k.view(torch.int16).numpy()
    hv = host_v.view(torch.int16).numpy()

    def fill(lr):
        layer, r = lr
        _, kk, vv = synth.request_tokens(w, seed, r, L, layer=layer)
        base = ((layer * R + r) * npr) * P
        hk[base:base + L] = kk.reshape(L, row).view(np.int16)
        hv[base:base + L] = vv.reshape(L, row).view(np.int16)

    # every (layer, request) has its own generators, so the draws can run side by side
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(16, max(1, len(os.sched_getaffinity(0))))) as ex:
        list(ex.map(fill, [(layer, r) for layer in range(NL) for r in range(R)]))
    if unit == "token":
        C, P, npr = C * P, 1, npr * P
    elif unit != "page":
        raise ValueError(f"unit must be 'page' or 'token', not {unit!r}")
    cache = KvPool(C, P, w.num_kv_heads, w.head_dim_k, w.head_dim_v, device=device)
    tier = LruTier(cache, NL, R, npr, host_k, host_v)
    q = _dev(synth.queries(w, seed), device)
    params = decode_params(R, w.num_q_heads, k, L, w.sm_scale)
    ws = torch.empty(max(workspace_bytes(cache, params), 256), dtype=torch.uint8, device=device)
    lens_dev = torch.full((R,), L, dtype=torch.int32, device=device)
    return StagedTier(w, seed, R, L, npr, host_k, host_v, cache, tier, params, q, lens_dev, ws)
