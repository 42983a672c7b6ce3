"""CPU oracle for top-k sparse decode attention over a paged KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything here.  The HIP
library never calls it and has no fallback to it.

A plain, slow, obviously-correct restatement of what the pages define, written
for checking by eye against them:

* ``paging``   page counts, last-page slack, naive-reservation waste, admission
               capacity, prefix sharing, and the page-table allocation policy
               (paged-KV page: "KV cache phân trang, hay vì sao đặt trước theo
               độ dài tối đa là hoang phí").
* ``indexer``  lightning-indexer scores: per-head dot product, ReLU, weighted sum
               over heads, computed exactly in int64 (GLM5.3 sparse-attention
               page: "Cơ chế chú ý thưa (Sparse Attention) trên GLM5.3 ảnh hưởng
               thế nào đến bộ nhớ HBM?", lightning-indexer paragraph).
* ``topk``     keep the k best-scored positions, dense when the context has at
               most k tokens (same paragraph), lowest position first on ties.
* ``sdpa``     softmax attention over the selected positions in float64.
* ``decode``   the three steps chained for one request.
* ``lru``      a strict LRU page cache simulator (GLM5.3 page, HiSparse paragraph;
               state-snapshot page "cat-it-di-nho-nhieu-hon", section "Lợi ích
               thì đo được rõ", for the sequential-scan pathology).
* ``roofline`` arithmetic intensity of MQA-mode MLA decode (GLM5.3 page, roofline
               paragraph; the equations themselves did not survive extraction).
* ``mla``      the MHA and MQA modes of latent attention and their costs (GLM5.3
               page, MLA-modes paragraph).

Nothing here imports the HIP package, and the HIP package imports nothing here.
Inputs come from ``synth`` (random draws only) or from literal arrays in tests.
"""
from . import paging, indexer, topk, sdpa, decode, lru, roofline, bf16  # noqa: F401
