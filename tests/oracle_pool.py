"""Runs the CPU oracle over many requests of a workload in parallel worker processes (test
infrastructure).

Each worker regenerates a request's cache contents from the seeded generators and runs the
oracle's decode step on them: scores (float64 of the exact integer sums), the top-k selection
and the float64 attention output.  Workers start with the "spawn" method, so they never inherit
a process that has initialised the GPU, and they import only numpy, the generators and the
oracle.  The pool is sized to the host's CPU share (at most 16 workers).
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

MAX_WORKERS = 16


def _one(args):
    import synth
    from oracle import decode
    w, seed, b, q_b, qidx_b, widx = args
    L = int(synth.lens(w, seed)[b])
    kidx, kk, vv = synth.request_tokens(w, seed, b, L)
    s, sel, o = decode.request_step(q_b, qidx_b, widx, kidx, kk, vv, w.top_k, w.sm_scale,
                                    v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
    return b, np.asarray(s, dtype=np.float64), np.asarray(sel, dtype=np.int32), np.asarray(o)


def oracle_requests(w, seed, reqs, q, qidx, widx, workers=None):
    """{request: (scores, selection, output)} for every request in ``reqs``; q / qidx / widx
    are the staged query arrays (bf16 bits) the GPU run used."""
    reqs = list(reqs)
    n = workers or min(MAX_WORKERS, len(os.sched_getaffinity(0)), max(1, len(reqs)))
    jobs = [(w, seed, b, q[b], qidx[b], widx) for b in reqs]
    if n <= 1:
        return {b: r for b, *r in map(_one, jobs)}
    out = {}
    with cf.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as ex:
        for b, s, sel, o in ex.map(_one, jobs, chunksize=1):
            out[b] = (s, sel, o)
    return out
