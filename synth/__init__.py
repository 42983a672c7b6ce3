"""Seeded synthetic inputs for the sparse decode-attention workloads.

This module only draws numbers.  It holds none of the method's arithmetic: no
page counts, no scores, no selection, no softmax.  Both the CPU oracle (through
the tests) and the HIP path (through the tests and the benchmark) take their
inputs from here, so that the two sides see bit-identical data while sharing no
code with each other.

Every array is drawn from its own ``numpy.random.Generator`` keyed by
``(seed, workload id, stream, request, layer)``.  One request's tokens can
therefore be regenerated alone, which is how the oracle checks sampled requests
of the large workloads without holding the whole cache in host memory.

bf16 values are carried as raw ``uint16`` bit patterns (numpy has no bf16):
the fp32 draw is rounded to nearest, ties to even, and the upper 16 bits kept.

Workloads (the shapes the pages discuss, with synthetic values):

* ``tiny_b5``        five requests of 403/96/241/30/176 tokens at page size 16,
                     the worked example of the paged-KV page ("KV cache phân
                     trang, hay vì sao đặt trước theo độ dài tối đa là hoang
                     phí", opening table).  8 query heads over 1 KV head, d=64.
* ``gqa_b32_8k``     32 requests of U[2048, 8192] tokens, page size 64, pages
                     scattered over the pool, 32 q heads / 4 KV heads, d=128.
* ``mla_b64_32k``    64 requests x 32768 tokens, page size 64, 64 query heads
                     over one 576-dim latent KV head whose first 512 dims are
                     the values (the MQA mode of MLA, GLM5.3 sparse-attention
                     page, MLA-modes paragraph).  top-k 2048.
* ``prefix_b128_16k`` 128 requests sharing a 16384-token prefix plus a private
                     U[1024, 4096]-token suffix (paged-KV page, section "Chia
                     sẻ trang").  32 q heads / 8 KV heads, d=128.
* ``mla_b64_32k_ih64`` the 64 x 32k latent workload with a 64-head indexer
                     query (one indexer head per attention head) and integer
                     head weights in [-2, 3] (lightning-indexer paragraph: many
                     query heads, one key head, a weighted sum of per-head ReLU
                     logits).  Scores stay exact in fp32: |score| <= 64 x 3 x
                     128 x 4 x 4 = 393,216 < 2^24.
* ``mla_mha_b64_4k`` the MHA mode of the same latent attention (GLM5.3 page,
                     MLA-modes paragraph): 64 requests x 4096 tokens, 64 query
                     heads each with its own 192-dim key (128 projected + 64
                     rotary) and 128-dim value, top-k 2048.  Keys and values
                     are drawn directly (no trained up-projections).
* ``mla_b64_32k_h128`` the 64 x 32k latent workload with 128 query heads over the
                     latent head (GLM5.3 page, roofline paragraph: DeepSeek V3.2 runs
                     about 128 heads where GLM-5 runs 64).
* ``tiered_b256_64k`` 256 requests x 65536 tokens x 8 layers; the HBM page
                     cache holds a quarter of the pages (GLM5.3 sparse-attention
                     page, HiSparse paragraph).  Positions come from a seeded
                     80% locality-biased / 20% uniform mix.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "f32_to_bf16_bits", "lens", "free_order",
    "prefix_groups", "index_queries", "index_weights", "index_inputs", "queries",
    "request_tokens", "tier_positions",
]

# stream ids: one independent generator per kind of draw
_S_LENS, _S_FREE, _S_QIDX, _S_KIDX, _S_Q, _S_K, _S_V = 1, 2, 3, 4, 5, 6, 7
_S_PKIDX, _S_PK, _S_PV, _S_TIER, _S_WIDX = 8, 9, 10, 11, 12


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                      # integer id mixed into every seed
    batch: int
    page_size: int
    pool_pages: int               # physical pages in the pool (stated, see recipe)
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    v_from_k: bool                # values are the first head_dim_v dims of the key row
    index_dim: int                # 0 = no indexer (positions are given)
    index_heads: int
    index_range: int              # indexer q/k integers uniform in [-r, r]
    top_k: int
    kv_std: float                 # K/V ~ N(0, kv_std) (standard deviation)
    q_std: float
    fixed_lens: Optional[tuple] = None
    len_range: Optional[tuple] = None      # inclusive (lo, hi) for the private part
    prefix_len: int = 0                     # shared prefix tokens (one group: all requests)
    scattered: bool = True                  # free order is a seeded permutation
    num_layers: int = 1
    reserve: int = 0                        # naive per-request reservation (accounting only)
    cache_fraction: float = 1.0             # tiered: HBM slots / logical pages

    @property
    def sm_scale(self) -> float:
        # 1/sqrt(d_k) with d_k the key width the logits are taken over
        return 1.0 / float(np.sqrt(self.head_dim_k))


# Pool sizes are stated numbers: room for every request at its largest
# possible length plus one spare page per request for a decode append.
#   tiny:   61 pages used + 5 spare                           = 66
#   gqa:    32 x (8192/64) + 32                               = 4128
#   mla:    64 x (32768/64) + 64                              = 32832
#   mha:    64 x (4096/64) + 64                               = 4160
#   prefix: 256 shared + 128 x (4096/64) private + 128        = 8576
#   tiered: per layer 256 x (65536/64) = 262144 logical pages (host copy);
#           the HBM cache is 25% of all layers' pages          = 524288 slots
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_b5", 1, 5, 16, 66, 8, 1, 64, 64, False, 32, 1, 8, 64, 1.0, 1.0,
                 fixed_lens=(403, 96, 241, 30, 176), scattered=False, reserve=512),
        Workload("gqa_b32_8k", 2, 32, 64, 4128, 32, 4, 128, 128, False, 64, 1, 8, 512, 1.0, 1.0,
                 len_range=(2048, 8192), reserve=8192),
        Workload("mla_b64_32k", 3, 64, 64, 32832, 64, 1, 576, 512, True, 128, 1, 4, 2048, 0.5, 1.0,
                 fixed_lens=(32768,) * 64, reserve=32768),
        Workload("prefix_b128_16k", 4, 128, 64, 8576, 32, 8, 128, 128, False, 64, 1, 8, 1024, 1.0, 1.0,
                 len_range=(1024, 4096), prefix_len=16384, reserve=16384 + 4096),
        Workload("mla_b64_32k_ih64", 6, 64, 64, 32832, 64, 1, 576, 512, True, 128, 64, 4, 2048, 0.5, 1.0,
                 fixed_lens=(32768,) * 64, reserve=32768),
        Workload("mla_mha_b64_4k", 7, 64, 64, 4160, 64, 64, 192, 128, False, 128, 1, 4, 2048, 0.5, 1.0,
                 fixed_lens=(4096,) * 64, reserve=4096),
        Workload("mla_b64_32k_h128", 8, 64, 64, 32832, 128, 1, 576, 512, True, 128, 1, 4, 2048, 0.5, 1.0,
                 fixed_lens=(32768,) * 64, reserve=32768),
        Workload("tiered_b256_64k", 5, 256, 64, 524288, 16, 2, 128, 128, False, 0, 0, 0, 2048, 1.0, 1.0,
                 fixed_lens=(65536,) * 256, num_layers=8, reserve=65536, cache_fraction=0.25),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(seed: int, w: Workload, stream: int, *more: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, w.wid, stream, *more]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = np.right_shift(u, np.uint32(16))
    np.bitwise_and(r, np.uint32(1), out=r)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def lens(w: Workload, seed: int = 0) -> np.ndarray:
    """Context lengths in tokens (the decode token included), int32 [batch]."""
    if w.fixed_lens is not None:
        return np.asarray(w.fixed_lens, dtype=np.int32)
    lo, hi = w.len_range
    n = _rng(seed, w, _S_LENS).integers(lo, hi + 1, size=w.batch)
    return (n + w.prefix_len).astype(np.int32)


def free_order(w: Workload, seed: int = 0, num_pages: Optional[int] = None) -> np.ndarray:
    """Order in which the pool hands out physical page ids, int32 [num_pages]."""
    n = w.pool_pages if num_pages is None else int(num_pages)
    if not w.scattered:
        return np.arange(n, dtype=np.int32)
    return _rng(seed, w, _S_FREE, n).permutation(n).astype(np.int32)


def prefix_groups(w: Workload):
    """(group id per request, prefix length per group) or (None, None)."""
    if w.prefix_len == 0:
        return None, None
    return np.zeros(w.batch, dtype=np.int32), np.asarray([w.prefix_len], dtype=np.int32)


def index_queries(w: Workload, seed: int = 0) -> np.ndarray:
    """Indexer queries, bf16 bits [batch, index_heads, index_dim], integer-valued."""
    r = w.index_range
    v = _rng(seed, w, _S_QIDX).integers(-r, r + 1, size=(w.batch, w.index_heads, w.index_dim))
    return f32_to_bf16_bits(v.astype(np.float32))


def _weights(g: np.random.Generator, heads: int) -> np.ndarray:
    if heads == 1:
        return np.ones(1, dtype=np.float32)
    return g.integers(-2, 4, size=heads).astype(np.float32)


def index_weights(w: Workload, seed: int = 0) -> np.ndarray:
    """Per-head indexer weights, fp32 [index_heads]: 1 for a single head, else integers
    uniform in [-2, 3] (signed, so a ReLU taken after the weighting would show)."""
    return _weights(_rng(seed, w, _S_WIDX), w.index_heads)


def index_inputs(w: Workload, seed: int, heads: int, batch: Optional[int] = None):
    """Indexer queries and weights for ``heads`` indexer heads instead of the workload's own
    (head-count tests): bf16 bits [batch, heads, index_dim] and fp32 [heads]."""
    batch = w.batch if batch is None else int(batch)
    if heads == w.index_heads and batch <= w.batch:
        return index_queries(w, seed)[:batch], index_weights(w, seed)
    r = w.index_range
    g = _rng(seed, w, _S_QIDX, heads, batch)
    q = f32_to_bf16_bits(g.integers(-r, r + 1, size=(batch, heads, w.index_dim)).astype(np.float32))
    return q, _weights(_rng(seed, w, _S_WIDX, heads), heads)


def queries(w: Workload, seed: int = 0, batch: Optional[int] = None) -> np.ndarray:
    """Attention queries, bf16 bits [batch, num_q_heads, head_dim_k], N(0, q_std); ``batch``
    defaults to the workload's.  The rows are drawn in order, so a smaller batch is a prefix of
    a larger one."""
    n = w.batch if batch is None else int(batch)
    x = _rng(seed, w, _S_Q).standard_normal((n, w.num_q_heads, w.head_dim_k), dtype=np.float32)
    return f32_to_bf16_bits(x * np.float32(w.q_std))


def _normal_bits(g: np.random.Generator, shape, std: float) -> np.ndarray:
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def request_tokens(w: Workload, seed: int, req: int, length: int, layer: int = 0,
                   start: int = 0, stop: Optional[int] = None):
    """Logical cache contents of request ``req`` for positions [start, stop).

    Returns ``(kidx, k, v)``: indexer keys bf16 bits [n, index_dim] (None when
    the workload has no indexer), keys [n, num_kv_heads, head_dim_k] and values
    [n, num_kv_heads, head_dim_v] (None when values are a slice of the keys).
    Positions below the shared prefix come from the prefix stream and are the
    same for every request of the group.
    """
    stop = length if stop is None else stop
    assert 0 <= start <= stop <= length
    parts_i, parts_k, parts_v = [], [], []
    segs = []
    p = w.prefix_len
    if start < p:
        segs.append(("prefix", start, min(stop, p)))
    if stop > p:
        segs.append(("own", max(start, p), stop))
    for kind, a, b in segs:
        n = b - a
        if kind == "prefix":
            gi, gk, gv, base = (_rng(seed, w, _S_PKIDX, layer), _rng(seed, w, _S_PK, layer),
                                _rng(seed, w, _S_PV, layer), 0)
            total = p
        else:
            gi, gk, gv, base = (_rng(seed, w, _S_KIDX, req, layer), _rng(seed, w, _S_K, req, layer),
                                _rng(seed, w, _S_V, req, layer), p)
            total = length - p
        # draw the whole segment then slice, so a sub-range equals the full draw's slice
        off = a - base
        if w.index_dim:
            r = w.index_range
            ki = gi.integers(-r, r + 1, size=(total, w.index_dim))[off:off + n]
            parts_i.append(f32_to_bf16_bits(ki.astype(np.float32)))
        kk = _normal_bits(gk, (total, w.num_kv_heads, w.head_dim_k), w.kv_std)[off:off + n]
        parts_k.append(kk)
        if not w.v_from_k:
            parts_v.append(_normal_bits(gv, (total, w.num_kv_heads, w.head_dim_v), w.kv_std)[off:off + n])
    kidx = np.concatenate(parts_i) if parts_i else None
    k = np.concatenate(parts_k)
    v = np.concatenate(parts_v) if parts_v else None
    return kidx, k, v


def tier_positions(w: Workload, seed: int, step: int, layer: int, req: int,
                   centres_state: Optional[np.ndarray] = None, hotspots: int = 8,
                   walk_std: float = 64.0, spread_std: float = 512.0, local_frac: float = 0.8):
    """Token positions one (request, layer) attends at one step of the tiered workload.

    A seeded mix: ``local_frac`` of the k positions sit near one of ``hotspots``
    centres (centre + N(0, spread_std), clipped to the context), the rest are
    uniform over the context; duplicates are redrawn until k positions are
    distinct; the result is sorted.  Centres start uniform and random-walk by
    N(0, walk_std) tokens per step.  Returns (positions int32 [k], centres).
    """
    L = int(w.fixed_lens[req])
    k = w.top_k
    if centres_state is None:
        centres_state = _rng(seed, w, _S_TIER, req, layer, 1 << 20).uniform(0, L, size=hotspots)
    g = _rng(seed, w, _S_TIER, req, layer, step)
    centres = np.clip(centres_state + g.normal(0.0, walk_std, size=hotspots), 0, L - 1)
    chosen = set()
    out = []
    while len(out) < k:
        need = k - len(out)
        n_loc = int(round(need * local_frac))
        c = centres[g.integers(0, hotspots, size=n_loc)]
        loc = np.clip(np.rint(c + g.normal(0.0, spread_std, size=n_loc)), 0, L - 1).astype(np.int64)
        uni = g.integers(0, L, size=need - n_loc)
        for t in np.concatenate([loc, uni]).tolist():
            if t not in chosen:
                chosen.add(t)
                out.append(t)
                if len(out) == k:
                    break
    return np.sort(np.asarray(out, dtype=np.int32)), centres
