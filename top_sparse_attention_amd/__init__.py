"""Top-k sparse decode attention over a paged KV cache, native to AMD MI355X (gfx950).

A thin Python binding over libtsa (include/tsa.h): it marshals arguments and passes torch
tensors' device pointers and the current HIP stream.  Every step of the computation runs in
the library's HIP kernels; there is no Python or CPU fallback, and the first call raises if
libtsa.so has not been built (``python -m top_sparse_attention_amd.build``).

Host-side arrays (lengths, page tables as built) are numpy int32; device arrays are torch
tensors on the GPU.  bf16 device data may be passed as torch.bfloat16 or as int16/uint16 bit
patterns.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np

from . import _lib
from ._lib import DecodeParams, PoolDesc, TsaError, call, load  # noqa: F401

__all__ = ["KvPool", "DecodeParams", "TsaError", "load", "decode_params", "workspace_bytes",
           "indexer_scores", "topk", "indexer_topk", "sparse_attn_gather", "sparse_decode_attn",
           "abi_version", "StepGraph", "decode_step",
           "decode_step_fused", "decode_step_noalloc"]


def _i32p(a: Optional[np.ndarray]):
    if a is None:
        return None
    if a.dtype != np.int32 or not a.flags.c_contiguous:
        raise ValueError("host index arrays must be C-contiguous numpy int32")
    return a.ctypes.data_as(_lib.P_i32)


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else int(t.numel() * t.element_size())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _event(ev) -> Optional[int]:
    """Raw hipEvent_t of a torch.cuda.Event (or None)."""
    if ev is None:
        return None
    h = int(ev.cuda_event)
    if not h:
        raise ValueError("the event has not been recorded yet")
    return h


def abi_version() -> int:
    return int(load().tsa_abi_version())


def decode_params(batch, num_q_heads, top_k, max_len, sm_scale, index_heads=1) -> DecodeParams:
    return DecodeParams(int(batch), int(num_q_heads), int(index_heads), int(top_k), int(max_len),
                        float(sm_scale))


class KvPool:
    """A pool of fixed-size pages (caller-owned device memory) and its host metadata."""

    def __init__(self, num_pages, page_size, num_kv_heads, head_dim_k, head_dim_v, *,
                 num_layers=1, v_from_k=False, index_dim=0, free_order=None, device="cuda",
                 allocate=True):
        self.desc = PoolDesc(int(num_pages), int(page_size), int(num_layers), int(num_kv_heads),
                             int(head_dim_k), int(head_dim_v), int(bool(v_from_k)), int(index_dim))
        kb, vb, ib = _lib.sz(), _lib.sz(), _lib.sz()
        call("tsa_kv_pool_bytes", C.byref(self.desc), C.byref(kb), C.byref(vb), C.byref(ib))
        self.bytes = (kb.value, vb.value, ib.value)
        self.k = self.v = self.idx = None
        if allocate:
            import torch
            self.k = torch.empty(kb.value // 2, dtype=torch.bfloat16, device=device)
            self.v = torch.empty(vb.value // 2, dtype=torch.bfloat16, device=device) if vb.value else None
            self.idx = torch.empty(ib.value // 2, dtype=torch.bfloat16, device=device) if ib.value else None
        fo = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        if fo is not None and fo.shape != (self.desc.num_pages,):
            raise ValueError("free_order must list every page once")
        h = _lib.vp()
        call("tsa_kv_pool_create", C.byref(self.desc), _ptr(self.k), _ptr(self.v), _ptr(self.idx),
             _i32p(fo), C.byref(h))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _lib.load().tsa_kv_pool_destroy(self.handle)
            self.handle = _lib.vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---------------------------------------------------------------- metadata
    @property
    def page_size(self) -> int:
        return self.desc.page_size

    def usage(self):
        f, u = _lib.i32(), _lib.i32()
        call("tsa_kv_pool_usage", self.handle, C.byref(f), C.byref(u))
        return f.value, u.value

    def refcount(self, page: int) -> int:
        r = _lib.i32()
        call("tsa_kv_pool_refcount", self.handle, int(page), C.byref(r))
        return r.value

    def build_tables(self, lens, max_pages: int, prefix_group=None, prefix_len_of_group=None):
        """Returns (page_table int32 [n, max_pages], num_pages int32 [n], saved pages)."""
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        n = lens.shape[0]
        table = np.empty((n, max_pages), dtype=np.int32)
        num = np.empty(n, dtype=np.int32)
        saved = _lib.i64()
        pg = None if prefix_group is None else np.ascontiguousarray(prefix_group, dtype=np.int32)
        pl = None if prefix_len_of_group is None else np.ascontiguousarray(prefix_len_of_group, dtype=np.int32)
        ng = 0 if pl is None else pl.shape[0]
        call("tsa_page_table_build", self.handle, n, _i32p(lens), _i32p(pg), _i32p(pl), ng,
             int(max_pages), _i32p(table), _i32p(num), C.byref(saved))
        return table, num, saved.value

    def grow_tables(self, table: np.ndarray, num_pages: np.ndarray, new_lens):
        """Extend ``table`` / ``num_pages`` in place for the new lengths."""
        new_lens = np.ascontiguousarray(new_lens, dtype=np.int32)
        call("tsa_page_table_grow", self.handle, new_lens.shape[0], _i32p(new_lens), table.shape[1],
             _i32p(table), _i32p(num_pages))

    def release_tables(self, table: np.ndarray, num_pages: np.ndarray):
        call("tsa_page_table_release", self.handle, num_pages.shape[0], _i32p(table),
             _i32p(num_pages), table.shape[1])

    def append_check(self, req, pos, table: np.ndarray, num_pages: np.ndarray):
        req = np.ascontiguousarray(req, dtype=np.int32)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        call("tsa_kv_append_check", self.handle, req.shape[0], _i32p(req), _i32p(pos),
             num_pages.shape[0], _i32p(table), _i32p(num_pages), table.shape[1])

    # ---------------------------------------------------------------- device calls
    def append(self, layer, req_dev, pos_dev, table_dev, n_req, k_src, v_src=None, idx_src=None,
               bad_dev=None, stream=None):
        """Scatter rows into the pool (device arrays; see tsa_kv_append)."""
        max_pages = table_dev.shape[-1]
        call("tsa_kv_append", self.handle, int(layer), int(req_dev.numel()), _ptr(req_dev),
             _ptr(pos_dev), _ptr(table_dev), int(n_req), int(max_pages), _ptr(k_src), _ptr(v_src),
             _ptr(idx_src), _ptr(bad_dev), _stream(stream))


class LruTier:
    """HBM page cache with LRU eviction over a pinned host copy of every page (tsa_lru_*).

    ``cache`` is a one-layer KvPool holding the slots (no indexer, separate V); ``host_k`` /
    ``host_v`` are pinned host tensors, key-major pages (key = (layer * num_req + req) *
    pages_per_req + page).  With a metadata-only cache (allocate=False) the tier only does
    the bookkeeping."""

    def __init__(self, cache: KvPool, num_layers: int, num_req: int, pages_per_req: int,
                 host_k=None, host_v=None):
        self.cache = cache
        self.num_req = int(num_req)
        self.pages_per_req = int(pages_per_req)
        self._host = (host_k, host_v)       # kept alive: the GPU reads them
        h = _lib.vp()
        call("tsa_lru_create", cache.handle, int(num_layers), int(num_req), int(pages_per_req),
             _ptr(host_k), _ptr(host_v), C.byref(h))
        self.handle = h
        self.workspace = None

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _lib.load().tsa_lru_destroy(self.handle)
            self.handle = _lib.vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def preload(self, keys):
        keys = np.ascontiguousarray(keys, dtype=np.int64)
        call("tsa_lru_preload", self.handle, int(keys.shape[0]), keys.ctypes.data_as(_lib.P_i64))

    def plan(self, layer: int, tag: int, positions: np.ndarray, table: bool = True):
        """positions: int32 [n_req, k].  Returns (slot_table int32 [n_req, pages_per_req], or
        None when ``table`` is false, and the number of pending copies)."""
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        n_req, k = positions.shape
        out = np.empty((n_req, self.pages_per_req), dtype=np.int32) if table else None
        nf = _lib.i64()
        call("tsa_lru_plan", self.handle, int(layer), int(tag), int(n_req), _i32p(positions), int(k),
             _i32p(out) if table else None, C.byref(nf))
        return out, nf.value

    def workspace_bytes(self, n_req: int) -> int:
        b = _lib.sz()
        call("tsa_lru_workspace_bytes", self.handle, int(n_req), C.byref(b))
        return b.value

    def fetch(self, table_dev, stream=None):
        """Write the last plan's slots into ``table_dev`` (int32 [n_req, pages_per_req]) and copy
        the pending pages (enqueued on ``stream``)."""
        import torch
        n_req = int(table_dev.shape[0])
        if self.workspace is None:
            self.workspace = torch.empty(max(self.workspace_bytes(n_req), 256), dtype=torch.uint8,
                                         device=self.cache.k.device)
        call("tsa_lru_fetch", self.handle, n_req, None, _ptr(table_dev),
             _ptr(self.workspace), _nbytes(self.workspace), _stream(stream))

    def release(self, tag: int):
        call("tsa_lru_release", self.handle, int(tag))

    def release_layer(self, tag: int, done=None):
        """Unpin ``tag``'s pages; later fetches wait for ``done`` (a torch.cuda.Event recorded
        after the last kernel that reads those pages) before copying (tsa_lru_release_layer)."""
        call("tsa_lru_release_layer", self.handle, int(tag), _event(done))

    def prefetch(self, layer: int, tag: int, positions: np.ndarray, table_dev, stream=None, fetched=None):
        """Plan and fetch one layer on ``stream`` (after the events of released tags), then record
        ``fetched`` (a torch.cuda.Event) there (tsa_lru_prefetch)."""
        import torch
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        n_req, k = positions.shape
        if self.workspace is None:
            self.workspace = torch.empty(max(self.workspace_bytes(n_req), 256), dtype=torch.uint8,
                                         device=self.cache.k.device)
        if fetched is not None and not fetched.cuda_event:
            fetched.record(torch.cuda.current_stream() if stream is None else stream)   # creates it
        call("tsa_lru_prefetch", self.handle, int(layer), int(tag), int(n_req), _i32p(positions), int(k),
             _ptr(table_dev), _ptr(self.workspace), _nbytes(self.workspace), _stream(stream),
             _event(fetched))

    def stats(self):
        v = [_lib.i64() for _ in range(4)]
        call("tsa_lru_stats", self.handle, *[C.byref(x) for x in v])
        return {"hits": v[0].value, "misses": v[1].value, "evictions": v[2].value, "h2d_bytes": v[3].value}


def workspace_bytes(pool: KvPool, p: DecodeParams) -> int:
    n = _lib.sz()
    call("tsa_sparse_decode_workspace", pool.handle, C.byref(p), C.byref(n))
    return n.value


def indexer_scores(pool, layer, p, qidx, widx, table_dev, seq_lens, scores, stream=None):
    call("tsa_indexer_scores", pool.handle, int(layer), C.byref(p), _ptr(qidx), _ptr(widx),
         _ptr(table_dev), int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(scores),
         int(scores.shape[-1]), _stream(stream))


def topk(p, scores, seq_lens, out, stream=None):
    call("tsa_topk", C.byref(p), _ptr(scores), int(scores.shape[-1]), _ptr(seq_lens), _ptr(out),
         _stream(stream))


def indexer_topk(pool, layer, p, qidx, widx, table_dev, seq_lens, out, workspace, stream=None):
    call("tsa_indexer_topk", pool.handle, int(layer), C.byref(p), _ptr(qidx), _ptr(widx),
         _ptr(table_dev), int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(out), _ptr(workspace),
         _nbytes(workspace), _stream(stream))


def sparse_attn_gather(pool, layer, p, q, topk_idx, table_dev, seq_lens, out, workspace, stream=None):
    call("tsa_sparse_attn_gather", pool.handle, int(layer), C.byref(p), _ptr(q), _ptr(topk_idx),
         _ptr(table_dev), int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(out), _ptr(workspace),
         _nbytes(workspace), _stream(stream))


def decode_step(pool, layer, p, k_new, v_new, idx_new, q, qidx, widx, table_dev, seq_lens, out,
                workspace, topk_out=None, bad=None, stream=None):
    """The decode step with each request's new token written at position seq_len - 1 first
    (fused into the scoring launch where the pool allows; see tsa_decode_step)."""
    call("tsa_decode_step", pool.handle, int(layer), C.byref(p), _ptr(k_new), _ptr(v_new), _ptr(idx_new),
         _ptr(bad), _ptr(q), _ptr(qidx), _ptr(widx), _ptr(table_dev), int(table_dev.shape[-1]),
         _ptr(seq_lens), _ptr(out), _ptr(topk_out), _ptr(workspace), _nbytes(workspace), _stream(stream))


def decode_step_noalloc(pool, layer, p, k_new, v_new, idx_new, q, qidx, widx, table_dev, seq_lens, out,
                        topk_out=None, bad=None, stream=None):
    """tsa_decode_step with the library's own scratch array as the workspace (no allocation;
    calls that overlap on one GPU race; see tsa_decode_step_noalloc)."""
    call("tsa_decode_step_noalloc", pool.handle, int(layer), C.byref(p), _ptr(k_new), _ptr(v_new),
         _ptr(idx_new), _ptr(bad), _ptr(q), _ptr(qidx), _ptr(widx), _ptr(table_dev),
         int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(out), _ptr(topk_out), _stream(stream))


def decode_step_fused(pool, layer, p, k_new, v_new, idx_new, q, qidx, widx, table_dev, seq_lens, out,
                      topk_out=None, bad=None, stream=None):
    """The decode step as one launch, one workgroup per request (see tsa_decode_step_fused)."""
    call("tsa_decode_step_fused", pool.handle, int(layer), C.byref(p), _ptr(k_new), _ptr(v_new),
         _ptr(idx_new), _ptr(bad), _ptr(q), _ptr(qidx), _ptr(widx), _ptr(table_dev),
         int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(out), _ptr(topk_out), _stream(stream))


class StepGraph:
    """The decode step (optional kv_append, then scores, top-k, attention) recorded once into a HIP
    graph over these tensors; ``launch`` replays it (see tsa_step_graph_create).  The tensors
    must stay alive and keep their shapes while the graph exists."""

    def __init__(self, pool, layer, p, q, qidx, widx, table_dev, seq_lens, out, workspace,
                 topk_out=None, append=None):
        self._keep = [pool, p, q, qidx, widx, table_dev, seq_lens, out, workspace, topk_out]
        ap = None
        if append is not None:
            req, pos, k_src, v_src, idx_src, bad = append
            ap = _lib.AppendArgs(int(req.numel()), _ptr(req), _ptr(pos), _ptr(k_src), _ptr(v_src),
                                 _ptr(idx_src), _ptr(bad))
            self._keep += [ap, req, pos, k_src, v_src, idx_src, bad]
        h = C.c_void_p()
        call("tsa_step_graph_create", pool.handle, int(layer), C.byref(p),
             None if ap is None else C.byref(ap), _ptr(q), _ptr(qidx), _ptr(widx), _ptr(table_dev),
             int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(out), _ptr(topk_out), _ptr(workspace),
             _nbytes(workspace), C.byref(h))
        self.handle = h

    def launch(self, stream=None):
        call("tsa_step_graph_launch", self.handle, _stream(stream))

    def close(self):
        if getattr(self, "handle", None):
            call("tsa_step_graph_destroy", self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sparse_decode_attn(pool, layer, p, q, qidx, widx, table_dev, seq_lens, out, workspace,
                       topk_out=None, stream=None):
    call("tsa_sparse_decode_attn", pool.handle, int(layer), C.byref(p), _ptr(q), _ptr(qidx),
         _ptr(widx), _ptr(table_dev), int(table_dev.shape[-1]), _ptr(seq_lens), _ptr(out),
         _ptr(topk_out), _ptr(workspace), _nbytes(workspace),
         _stream(stream))
