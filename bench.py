#!/usr/bin/env python3
"""Decode-step benchmark: top-k sparse attention over a paged KV cache on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = append each request's newest token (K/V/indexer key scatter), indexer scores over
every cached token, top-k selection, attention over the selected tokens (+ split combine).
Inputs are seeded synthetic data resident in HBM before timing starts.  The default workload
is 64 requests x 32768 tokens, top-2048, 64 query heads over one 576-dim latent KV head.

Prints ONE JSON line.  `value` = requests decoded per second (one token each) over K steps run
back to back; the steps rotate through 8 pre-drawn query sets, so each selects other rows than
the step before.  `step_ms` gives the median, p10 and p90 of per-step times, warm and with a
512 MiB scrub before each step.  `roofline` covers the dominant kernel (the indexer score,
which streams every cached indexer key); `roofline_attention` the gather-attention kernels.
Kernel durations come from HIP events recorded on the launch stream between the launches of a
second pass of the same steps.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s


def _src_hash(name: str) -> str:
    """Hash of what a kernel's machine code depends on: its source, the headers every kernel
    source includes, and the compiler flags.  Comment-only and blank lines are left out, so that
    editing a comment does not disown the counters taken on the same code."""
    csrc = os.path.join(ROOT, "top_sparse_attention_amd", "csrc")
    code = []
    for f in (name, "tsa_internal.h", "mfma_lds.h"):
        code += [ln.rstrip() for ln in open(os.path.join(csrc, f), encoding="utf-8")
                 if ln.strip() and not ln.lstrip().startswith("//")]
    from top_sparse_attention_amd import build as _build
    # the flags, without the include paths: those name where the tree sits, not what is built
    code.append(" ".join(f for f in _build.FLAGS if not f.startswith("-I")))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _has_traffic(key: str) -> bool:
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        return key in json.load(open(p))
    except Exception:
        return False


def _traffic(kernel_src: str, key: str):
    """Counter-measured HBM bytes per launch from a committed profile summary, or None when the
    kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p)).get(key)
    except Exception:
        return None
    if not d or d.get("src_sha256_16") != _src_hash(kernel_src):
        return None
    return d.get("bytes_per_launch")


def _oracle_rate(w, seed: int, budget_s: float):
    """Requests per second of the oracle's whole decode step over whole requests of workload w,
    until the time budget is spent; returns (rate, sample description)."""
    import synth
    from oracle import decode
    lens = synth.lens(w, seed)
    qi = synth.index_queries(w, seed)
    q = synth.queries(w, seed)
    wi = synth.index_weights(w, seed)
    done, spent, b, passes = 0, 0.0, 0, 0
    while spent < budget_s and b < len(lens):
        L = int(lens[b])
        kidx, kk, vv = synth.request_tokens(w, seed, b, L)
        # repeat each request so that one pass over all requests roughly fills the budget
        reps = 1 if done == 0 else max(1, int(budget_s / max(spent / done, 1e-9) / len(lens)))
        for _ in range(reps):
            t0 = time.perf_counter()
            decode.request_step(q[b], qi[b], wi, kidx, kk, vv, w.top_k, w.sm_scale,
                                v_from_k_dims=w.head_dim_v if w.v_from_k else 0)
            spent += time.perf_counter() - t0
            done += 1
        passes = max(passes, reps)
        b += 1
    return done / spent, (f"{done} request steps over the first {b} of {len(lens)} requests of {w.name} "
                          f"(full context each, up to {passes} repeats per request), {spent:.1f} s of "
                          f"oracle time; input generation not timed")


def _mem_available() -> int:
    """MemAvailable of this host in bytes (0 when unknown)."""
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemAvailable:"):
                return int(line.split()[1]) * 1024
    except Exception:
        pass
    return 0


def _probe_pinned(want: int, chunk: int = 4 << 30) -> int:
    """Bytes of pinned host memory this process can hold, up to `want`: pins 4 GiB blocks until
    the runtime refuses or `want` is reached, then frees them (and torch's pinned-block cache)."""
    import torch
    held, total = [], 0
    try:
        while total < want:
            held.append(torch.empty(chunk, dtype=torch.uint8, pin_memory=True))
            total += chunk
    except Exception:
        pass
    del held
    torch._C._host_emptyCache()
    return total


def cpu_baseline(w, seed: int, budget_s: float = 12.0):
    """The oracle as it stands, timed on this host on a bounded sample of the same workload
    (whole requests: scores over every token, full-sort top-k, float64 attention), twice: with
    the BLAS thread pool limited to one thread, and with every core this process may use.
    Returns requests (= decode tokens) per second of the all-core run, with the one-thread run
    beside it."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=1):
        one, one_sample = _oracle_rate(w, seed, budget_s)
    with threadpool_limits(limits=cores):
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        allc, all_sample = _oracle_rate(w, seed, budget_s)
    return {"value": allc, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": all_sample, "cpu": _cpu_model(), "host_cores": cores,
            "one_thread": {"value": one, "cores": 1, "sample": one_sample},
            "note": "integer scores and the top-k sort are single-threaded numpy; the BLAS thread "
                    "count changes only the float64 attention"}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


CALIB_KERNEL = "bitwise_not"   # torch's elementwise kernel name for the calibration copy
def _attn_src(w) -> str:
    """Source file of the attention kernel the library picks for workload w (for traffic keys)."""
    if w.v_from_k:
        return "attn_mfma.hip"
    G = w.num_q_heads // w.num_kv_heads
    if (w.head_dim_k, w.head_dim_v) in ((64, 64), (128, 128), (192, 128), (256, 256)) and G <= 16:
        return "attn_gqa.hip"      # the grouped-query matrix-core kernel's shapes
    return "attn_valu.hip"


TRAFFIC_KERNELS = {            # profiles/traffic.json key prefix -> (kernel-name test, source)
    "indexer_score": (lambda n: "indexer_score" in n, "indexer_score.hip"),
    "attention": (lambda n: "attn" in n and "combine" not in n, None),
    "combine": (lambda n: "combine" in n, "attn_valu.hip"),
    "topk": (lambda n: "topk" in n, "topk.hip"),
}


def copy_calibration(mib: int):
    """A plain streaming copy of known size (int32 bitwise-not: reads N bytes, writes N bytes),
    run three times, so that the FETCH_SIZE / WRITE_SIZE counters can be scaled to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] calibration copy: {mib} MiB read + {mib} MiB written per launch",
          file=sys.stderr, flush=True)
    del src, dst


def _counter_means(path: str, counter: str):
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, mib: int):
    """Per-launch HBM bytes of each kernel from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by bytes / counter of the calibration copy launched in the same process."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    calib = [k for k in fetch if CALIB_KERNEL in k]
    if not calib:
        raise SystemExit("no calibration copy in the counter CSV (run with --copy-calib-mib)")
    nbytes = mib * (1 << 20)
    cf = fetch[calib[0]]
    cw = [v for k in write if CALIB_KERNEL in k for v in write[k]]
    f_scale = nbytes / (np.mean(cf) * 1024.0)
    w_scale = nbytes / (np.mean(cw) * 1024.0)
    out_path = os.path.join(ROOT, "profiles", "traffic.json")
    doc = json.load(open(out_path)) if os.path.exists(out_path) else {}
    doc["_calibration"] = {"copy_bytes_each_way": nbytes, "fetch_kib": float(np.mean(cf)),
                           "write_kib": float(np.mean(cw)), "fetch_scale": round(f_scale, 4),
                           "write_scale": round(w_scale, 4)}
    doc[f"_calibration/{workload}"] = dict(doc["_calibration"])
    w = None
    try:
        import synth
        w = synth.get(workload)
    except Exception:
        pass
    for key, (match, src) in TRAFFIC_KERNELS.items():
        names = [k for k in fetch if match(k)]
        if not names:
            continue
        fk = np.mean([v for k in names for v in fetch[k]])
        wk = np.mean([v for k in write if match(k) for v in write[k]])
        if src is None:
            src = _attn_src(w) if w is not None else "attn_valu.hip"
        doc[f"{key}/{workload}"] = {
            "kernel": names[0][:120], "src_sha256_16": _src_hash(src),
            "fetch_kib": round(float(fk), 1), "write_kib": round(float(wk), 1),
            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
            "bytes_per_launch": int(fk * 1024 * f_scale + wk * 1024 * w_scale),
            "read_bytes": int(fk * 1024 * f_scale), "write_bytes": int(wk * 1024 * w_scale)}
    json.dump(doc, open(out_path, "w"), indent=1, sort_keys=True)
    print(json.dumps(doc, indent=1, sort_keys=True))


def bench_mla_modes(args):
    """Latent attention in its two modes (GLM5.3 page, MLA-modes paragraph) at several context
    lengths, on the same selected positions: the MQA mode (every one of the 64 heads reads one
    576-dim latent row per token; matrix-core kernel) against the MHA mode (each head reads its own
    192-dim key and 128-dim value; vector-ALU kernel with one query head per KV head).  Values
    are random bf16 drawn on the device; the parity of both modes is the tests' business.
    Prints one JSON line."""
    import torch
    import top_sparse_attention_amd as tsa
    from top_sparse_attention_amd import KvPool, decode_params, workspace_bytes

    tsa.load()
    B, H, K, P = 64, 64, 2048, 64
    scale = 1.0 / np.sqrt(192.0)
    rng = np.random.default_rng(args.seed)
    modes = {"mqa": dict(hkv=1, dk=576, dv=512, alias=True), "mha": dict(hkv=H, dk=192, dv=128, alias=False)}
    points = []
    for L in (256, 512, 1024, 2048, 4096, 8192):
        n_sel = min(L, K)
        pos = np.full((B, K), -1, dtype=np.int32)
        for b in range(B):
            pos[b, :n_sel] = np.sort(rng.choice(L, n_sel, replace=False))
        topk = torch.from_numpy(pos).cuda()
        lens = np.full(B, L, dtype=np.int32)
        pt = {"L": L, "selected": n_sel}
        for name, m in modes.items():
            npages = B * (-(-L // P)) + B
            pool = KvPool(npages, P, m["hkv"], m["dk"], m["dv"], v_from_k=m["alias"],
                          free_order=rng.permutation(npages).astype(np.int32))
            table, _, _ = pool.build_tables(lens, -(-L // P))
            pool.k.normal_(0.0, 0.5)
            if pool.v is not None:
                pool.v.normal_(0.0, 0.5)
            p = decode_params(B, H, K, L, scale)
            q = torch.randn((B, H, m["dk"]), device="cuda").to(torch.bfloat16)
            out = torch.empty((B, H, m["dv"]), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(workspace_bytes(pool, p), 256), dtype=torch.uint8, device="cuda")
            tdev = torch.from_numpy(table).cuda()
            ldev = torch.from_numpy(lens).cuda()
            call = lambda: tsa.sparse_attn_gather(pool, 0, p, q, topk, tdev, ldev, out, ws)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 20
            e0.record()
            for _ in range(n):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            row = m["hkv"] * (m["dk"] * 2 + (0 if m["alias"] else m["dv"] * 2))
            nbytes = B * n_sel * row + B * H * m["dk"] * 2 + B * H * m["dv"] * 4 + B * K * 4
            flops = 2.0 * B * n_sel * H * (m["dk"] + m["dv"])
            pt[f"{name}_us"] = round(us, 2)
            pt[f"{name}_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            pt[f"{name}_tflops"] = round(flops / (us * 1e-6) / 1e12, 1)
            del pool, q, out, ws, tdev, ldev
            torch.cuda.empty_cache()
        points.append(pt)
        print(f"[bench] L={L}: MQA {pt['mqa_us']} us, MHA {pt['mha_us']} us", file=sys.stderr, flush=True)
    faster = [pt["L"] for pt in points if pt["mha_us"] < pt["mqa_us"]]
    print(json.dumps({"metric": "MLA decode attention, MQA mode vs MHA mode (us per call, 64 requests, "
                                "64 heads, top-2048)", "unit": "us", "higher_is_better": False,
                      "dtype": "bf16", "data": "synthetic",
                      "mha_faster_at": faster, "points": points}), flush=True)


def bench_one_launch(args):
    """The one-launch step (tsa_decode_step_fused: each request's append, scores, top-k and
    attention in one workgroup) against the separate launches (kv_append, then scores, top-k and
    attention) on short-context shapes: the tiny worked example and 32-head / 4-KV-head requests
    of 256..2048 tokens at several batch sizes and top-k.  Both are timed with HIP events over
    back-to-back calls; at these sizes host launch time can exceed the kernels', so the kernel
    durations of record come from a kernel trace of this same run.  Prints one JSON line."""
    import torch
    import synth
    import top_sparse_attention_amd as tsa
    from top_sparse_attention_amd import workload

    tsa.load()
    cases = [("tiny_b5", None, None),
             ("gqa_b32_8k", (32, 256), None),
             ("gqa_b32_8k", (32, 1024), 64),
             ("gqa_b32_8k", (32, 1024), 128),
             ("gqa_b32_8k", (8, 1024), 128),
             ("gqa_b32_8k", (128, 1024), 64),
             ("gqa_b32_8k", (256, 512), 64),
             ("gqa_b32_8k", (32, 2048), 64)]
    points = []
    for name, shape, k in cases:
        kw = {} if shape is None else {"lens": np.full(shape[0], shape[1], np.int32)}
        st = workload.stage(synth.get(name), seed=args.seed, **kw)
        if k is not None:
            st.params.top_k = k          # the staged top-k buffers hold the workload's larger k
        B = len(st.lens)
        rows = []
        for src in (st.new_k, st.new_v, st.new_idx):
            if src is None:
                rows.append(None)
                continue
            full = torch.zeros((B,) + tuple(src.shape[1:]), dtype=src.dtype, device="cuda")
            full[st.new_req.long()] = src
            rows.append(full)
        kn, vn, inew = rows

        def one_launch():
            tsa.decode_step_fused(st.pool, 0, st.params, kn, vn, inew, st.q, st.qidx, st.widx,
                                  st.table_dev, st.lens_dev, st.out, topk_out=st.topk)

        def separate():
            st.pool.append(0, st.new_req, st.new_pos, st.table_dev, B, st.new_k, st.new_v, st.new_idx)
            tsa.sparse_decode_attn(st.pool, 0, st.params, st.q, st.qidx, st.widx, st.table_dev,
                                   st.lens_dev, st.out, st.workspace, topk_out=st.topk)

        pt = {"workload": name, "requests": B, "context": int(st.lens.max()), "top_k": int(st.params.top_k),
              "kv_heads": st.w.num_kv_heads, "q_heads": st.w.num_q_heads}
        for label, fn in (("one_launch_us", one_launch), ("separate_us", separate)):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 100
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            pt[label] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
        points.append(pt)
        print(f"[bench] {name} B={B} L={pt['context']} k={pt['top_k']}: one launch {pt['one_launch_us']} us, "
              f"separate {pt['separate_us']} us", file=sys.stderr, flush=True)
        del st
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode step, one launch vs separate launches (us per step, HIP events "
                                "over back-to-back calls)", "unit": "us", "higher_is_better": False,
                      "dtype": "bf16", "data": "synthetic", "points": points}), flush=True)


def bench_tier(args):
    """The tiered workload: per step, every layer plans its pages on the host, fetches the
    misses on a side stream and attends over the HBM cache; prints one JSON line with
    tokens/s (requests decoded per second), the hit rate and the host-to-device rate.  The
    host copy of every page holds seeded random bf16 values (a repeated block: the tier's
    timing does not depend on them); positions come from the seeded locality-biased
    generator and are drawn before timing."""
    import torch
    import synth
    import top_sparse_attention_amd as tsa
    from top_sparse_attention_amd import KvPool, LruTier, decode_params, workspace_bytes

    tsa.load()
    w = synth.get(args.workload)
    L = int(w.fixed_lens[0])
    NL, P, k = w.num_layers, w.page_size, w.top_k
    row = w.num_kv_heads * w.head_dim_k
    per_req = 2 * NL * L * row * 2                 # pinned host bytes of one request (K and V)
    R = args.tier_requests or w.batch
    avail = _mem_available()
    fit = int(avail // 2 // per_req) if avail else R
    reduced = fit < R
    if reduced:
        print(f"[bench] tier: {R} requests need {R * per_req / 2**30:.1f} GiB pinned; half of the "
              f"{avail / 2**30:.1f} GiB available holds {fit}", file=sys.stderr, flush=True)
        R = max(1, fit)
    # pinned host memory has its own limit below the host's memory: find what can be pinned
    pinnable = _probe_pinned(R * per_req + (4 << 30))
    if pinnable < R * per_req + (4 << 30):
        fit = max(1, int((pinnable - (4 << 30)) // per_req))
        print(f"[bench] tier: {pinnable / 2**30:.0f} GiB could be pinned; {R} requests need "
              f"{R * per_req / 2**30:.1f} GiB (+4 GiB headroom): running {fit}", file=sys.stderr, flush=True)
        R, reduced = fit, True
    w = dataclasses.replace(w, batch=R, fixed_lens=(L,) * R)
    npr = -(-L // P)
    keys = NL * R * npr
    C = int(round(keys * w.cache_fraction))
    print(f"[bench] tier: {R} requests x {L} tokens x {NL} layers, {keys} pages "
          f"({2 * keys * P * row * 2 / 2**30:.1f} GiB pinned), cache {C} slots", file=sys.stderr, flush=True)
    g = torch.Generator().manual_seed(args.seed)
    host_k = torch.empty((keys * P, row), dtype=torch.bfloat16, pin_memory=True)
    host_v = torch.empty((keys * P, row), dtype=torch.bfloat16, pin_memory=True)
    # a 64 MiB seeded random block repeated over the whole host copy (drawing every value
    # would take minutes; the tier's timing does not depend on them)
    block = torch.empty(1 << 25, dtype=torch.bfloat16)
    for i in range(0, block.numel(), 1 << 22):
        block[i:i + (1 << 22)].normal_(0.0, w.kv_std, generator=g)
    for name, t in (("K", host_k), ("V", host_v)):
        flat = t.view(-1)
        for i in range(0, flat.numel(), block.numel()):
            n = min(block.numel(), flat.numel() - i)
            flat[i:i + n].copy_(block[:n])
            if (i // block.numel()) % 256 == 255:
                print(f"[bench] tier: host {name} filled {(i + n) * 2 / 2**30:.0f} GiB", file=sys.stderr, flush=True)
    # the cache unit: whole pages, or single token rows (a pool of one-token pages holding the
    # same bytes); the host copy is the same either way
    CP, UP, unpr = (C, P, npr) if args.tier_unit == "page" else (C * P, 1, npr * P)
    cache = KvPool(CP, UP, w.num_kv_heads, w.head_dim_k, w.head_dim_v)
    tier = LruTier(cache, NL, R, unpr, host_k, host_v)
    # initial state: the last quarter of every (layer, request)'s pages (or tokens), in key order
    keep = max(1, unpr // 4)
    ar = np.arange(unpr - keep, unpr, dtype=np.int64)
    pre = np.concatenate([(l * R + r) * unpr + ar for l in range(NL) for r in range(R)])[:CP]
    tier.preload(pre)
    params = decode_params(R, w.num_q_heads, k, L, w.sm_scale)
    ws = torch.empty(max(workspace_bytes(cache, params), 256), dtype=torch.uint8, device="cuda")
    lens_dev = torch.full((R,), L, dtype=torch.int32, device="cuda")
    q = torch.from_numpy(synth.queries(w, args.seed).view(np.int16)).cuda()
    out = torch.empty((R, w.num_q_heads, w.head_dim_v), dtype=torch.float32, device="cuda")
    total_steps = args.warmup + args.steps
    centres, pos_all = {}, []
    for step in range(total_steps if args.tier_positions == "drawn" else 0):
        layer_pos = []
        for layer in range(NL):
            a = np.empty((R, k), dtype=np.int32)
            for r in range(R):
                a[r], centres[(layer, r)] = synth.tier_positions(w, args.seed, step, layer, r,
                                                                 centres.get((layer, r)))
            layer_pos.append(a)
        pos_all.append(layer_pos)
    pos_dev = [[torch.from_numpy(a).cuda() for a in lp] for lp in pos_all]
    use_indexer = args.tier_positions == "indexer"
    if use_indexer:
        # HiSparse's flow: the indexer keys of every token stay in HBM (256 B per token), each
        # layer scores them and selects its top-k on the GPU, and the selection is copied to the
        # host, which plans the fetch.  Keys are random integers in [-4, 4]; each layer's query
        # keeps 90 % of its dims from one step to the next, so selections drift over steps as
        # a slowly changing hidden state would make them.
        D_I = 128
        ipool = KvPool(R * npr, P, 1, 8, 8, num_layers=NL, v_from_k=True, index_dim=D_I)
        itab, _, _ = ipool.build_tables(np.full(R, L, dtype=np.int32), npr)
        itab_dev = torch.from_numpy(itab).cuda()
        gd = torch.Generator(device="cuda").manual_seed(args.seed)
        per_layer = ipool.idx.numel() // NL
        for l in range(NL):
            ipool.idx[l * per_layer:(l + 1) * per_layer].copy_(
                torch.randint(-4, 5, (per_layer,), generator=gd, device="cuda", dtype=torch.int16))
        rng = np.random.default_rng(args.seed + 1)
        qcur = rng.integers(-4, 5, size=(NL, R, D_I))
        qidx_all = []
        for step in range(total_steps):
            if step:
                redraw = rng.random((NL, R, D_I)) < 0.1
                qcur = np.where(redraw, rng.integers(-4, 5, size=(NL, R, D_I)), qcur)
            qidx_all.append(torch.from_numpy(qcur.astype(np.float32)).to(torch.bfloat16).cuda())
        iparams = decode_params(R, w.num_q_heads, k, L, w.sm_scale)
        iws = torch.empty(max(workspace_bytes(ipool, iparams), 256), dtype=torch.uint8, device="cuda")
        iw = torch.ones(1, dtype=torch.float32, device="cuda")
        sel_dev = [torch.empty((R, k), dtype=torch.int32, device="cuda") for _ in range(2)]
        sel_host = [torch.empty((R, k), dtype=torch.int32, pin_memory=True) for _ in range(2)]
        sel_ready = [torch.cuda.Event() for _ in range(2)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    table_dev = [torch.full((R, unpr), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    fetched = [torch.cuda.Event() for _ in range(2)]
    done = {}
    ev_attn = []
    host_s = {"prefetch": 0.0}
    gidx = 0

    def run_step(step, timed):
        nonlocal gidx
        for layer in range(NL):
            if use_indexer:
                sd, sh = sel_dev[gidx & 1], sel_host[gidx & 1]
                tsa.indexer_topk(ipool, layer, iparams, qidx_all[step][layer], iw, itab_dev, lens_dev, sd, iws)
                sh.copy_(sd, non_blocking=True)
                sel_ready[gidx & 1].record(main)
                sel_ready[gidx & 1].synchronize()
                positions, pos_layer = sh.numpy(), sd
            else:
                positions, pos_layer = pos_all[step][layer], pos_dev[step][layer]
            # plan, then the copies on the side stream after the attention of every layer whose
            # slots they may reuse (released below with its event), then `fetched` recorded there
            h0 = time.perf_counter()
            tier.prefetch(layer, gidx, positions, table_dev[gidx & 1], stream=side, fetched=fetched[gidx & 1])
            if timed:
                host_s["prefetch"] += time.perf_counter() - h0
            main.wait_event(fetched[gidx & 1])
            e0 = torch.cuda.Event(enable_timing=True) if timed else None
            if timed:
                e0.record(main)
            tsa.sparse_attn_gather(cache, 0, params, q, pos_layer, table_dev[gidx & 1], lens_dev,
                                   out, ws)
            ev = torch.cuda.Event(enable_timing=timed)
            ev.record(main)
            done[gidx] = ev
            if timed:
                ev_attn.append((e0, ev))
            if gidx > 0:
                tier.release_layer(gidx - 1, done[gidx - 1])
            gidx += 1

    for s_ in range(args.warmup):
        run_step(s_, False)
    torch.cuda.synchronize()
    st0 = tier.stats()
    t0 = time.perf_counter()
    for s_ in range(args.warmup, total_steps):
        run_step(s_, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st1 = tier.stats()
    hits, misses = st1["hits"] - st0["hits"], st1["misses"] - st0["misses"]
    h2d = st1["h2d_bytes"] - st0["h2d_bytes"]
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_attn]))
    ms_step = elapsed * 1e3 / args.steps
    res = {
        "metric": "tiered sparse decode tokens/s (8 layers per token) and HBM cache hit rate",
        "value": round(R / (ms_step * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "requests": R, "requests_of_config": synth.get(args.workload).batch,
                   "requests_reduced_to_fit_pinned_memory": reduced,
                   "context": L, "layers": NL, "top_k": k,
                   "page_size": P, "cache_unit": args.tier_unit, "cache_slots": CP,
                   "cache_bytes": CP * UP * row * 4, "logical_pages": keys, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim_k, "parallelism": "none",
                   "positions": args.tier_positions},
        "tier": {"hit_rate": round(hits / max(hits + misses, 1), 4), "hits": hits, "misses": misses,
                 "h2d_GBps": round(h2d / elapsed / 1e9, 2), "h2d_bytes_per_step": h2d // args.steps,
                 "attention_ms_per_layer": round(attn_ms, 4),
                 "host_prefetch_call_ms_per_step": round(host_s["prefetch"] * 1e3 / args.steps, 3)},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mla_b64_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for each of the two host runs (1 thread, all cores)")
    ap.add_argument("--query-sets", type=int, default=8,
                    help="pre-drawn query sets the steps rotate through (different rows per step)")
    ap.add_argument("--tier-requests", type=int, default=0,
                    help="requests of the tiered workload (default: the configuration's 256, 128 GiB of "
                         "pinned host memory; fewer if half of the available host memory cannot hold them)")
    ap.add_argument("--tier-positions", choices=("drawn", "indexer"), default="drawn",
                    help="tiered workload: positions from the seeded locality generator, or from an "
                         "indexer top-k per layer over HBM-resident indexer keys (copied to the host)")
    ap.add_argument("--tier-unit", choices=("page", "token"), default="page",
                    help="cache unit of the tiered workload: whole pages or single token rows")
    ap.add_argument("--mla-modes", action="store_true",
                    help="compare latent attention in MQA mode and MHA mode over context lengths and exit")
    ap.add_argument("--one-launch", action="store_true",
                    help="time the one-launch step against the separate launches on short contexts")
    ap.add_argument("--separate", action="store_true",
                    help="time the step as separate calls (kv_append, scores, top-k, attention) "
                         "instead of tsa_decode_step")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as one replay of a captured graph (tsa_step_graph_*)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run a plain streaming copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of a --copy-calib-mib run into "
                         "profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        if not args.copy_calib_mib:
            raise SystemExit("--summarize-counters needs the --copy-calib-mib size of the profiled run")
        summarize_counters(*args.summarize_counters, args.workload, args.copy_calib_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode step is sharded by request with no exchange "
              f"between GPUs, and the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import synth

    if args.mla_modes:
        bench_mla_modes(args)
        return
    if args.one_launch:
        bench_one_launch(args)
        return
    if synth.get(args.workload).num_layers > 1:
        bench_tier(args)
        return
    bench_step(args)


def _row_bytes(w) -> int:
    """Bytes of one selected token's K (and V, when stored apart) over all KV heads, bf16."""
    return w.num_kv_heads * w.head_dim_k * 2 + (0 if w.v_from_k else w.num_kv_heads * w.head_dim_v * 2)


def algorithmic_counts(w, lens):
    """Algorithmic bytes and FLOPs of one launch of the indexer score and of the gather-attention
    (with its combine) over requests of lengths `lens`:
      indexer:   every cached token's indexer key (bf16, D_I dims) read and its fp32 score written,
                 2 * H_I * D_I FLOPs per token;
      attention: min(len, k) selected rows per request (_row_bytes), the bf16 queries, the fp32
                 outputs and the int32 top-k indices, 2 * Hq * (dk + dv) FLOPs per selected row.
    Returns (indexer bytes, indexer FLOPs, attention bytes, attention FLOPs)."""
    lens = np.asarray(lens, dtype=np.int64)
    B, D_I = len(lens), w.index_dim
    idx_bytes = int((lens * (2 * D_I + 4)).sum())
    idx_flops = float(2 * w.index_heads * D_I * lens.sum())
    n_sel = np.minimum(lens, w.top_k)
    attn_bytes = int(n_sel.sum() * _row_bytes(w) + B * w.num_q_heads * w.head_dim_k * 2 +
                     B * w.num_q_heads * w.head_dim_v * 4 + B * w.top_k * 4)
    attn_flops = float(2 * n_sel.sum() * w.num_q_heads * (w.head_dim_k + w.head_dim_v))
    return idx_bytes, idx_flops, attn_bytes, attn_flops


def _pct(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(xs)), 5), "p10": round(float(np.percentile(xs, 10)), 5),
            "p90": round(float(np.percentile(xs, 90)), 5), "mean": round(float(xs.mean()), 5)}


def bench_step(args):
    """The single-layer decode step (every workload but the tiered one); prints the JSON line."""
    import torch
    import synth
    import top_sparse_attention_amd as tsa
    from top_sparse_attention_amd import workload

    tsa.load()
    w = synth.get(args.workload)
    if args.copy_calib_mib:
        copy_calibration(args.copy_calib_mib)
    print(f"[bench] staging {w.name}", file=sys.stderr, flush=True)
    t0 = time.time()
    st = workload.stage(w, seed=args.seed)
    print(f"[bench] staged in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    B = len(st.lens)
    stream = torch.cuda.current_stream()
    ld = int(np.ceil(max(st.params.max_len, 1) / 64) * 64)
    scores = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    H_I = st.params.index_heads

    # Query sets: set 0 is the staged one (the parity tests' case); the others are further seeded
    # draws of the attention and indexer queries, so that consecutive steps select different rows
    # and no step re-reads the rows the one before it gathered.
    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).cuda()
    qsets = [(st.q, st.qidx)]
    for i in range(1, max(1, args.query_sets)):
        qsets.append((dev(synth.queries(w, args.seed + i, B)),
                      dev(synth.index_inputs(w, args.seed + i, H_I, B)[0])))
    n_sets = len(qsets)

    def step(i, ev=None):
        q, qidx = qsets[i % n_sets]
        if ev is not None:
            ev[0].record(stream)
        if st.new_req is not None:
            st.pool.append(0, st.new_req, st.new_pos, st.table_dev, B, st.new_k, st.new_v, st.new_idx)
        if ev is not None:
            ev[1].record(stream)
        tsa.indexer_scores(st.pool, 0, st.params, qidx, st.widx, st.table_dev, st.lens_dev, scores)
        if ev is not None:
            ev[2].record(stream)
        tsa.topk(st.params, scores, st.lens_dev, st.topk)
        if ev is not None:
            ev[3].record(stream)
        tsa.sparse_attn_gather(st.pool, 0, st.params, q, st.topk, st.table_dev, st.lens_dev,
                               st.out, st.workspace)
        if ev is not None:
            ev[4].record(stream)

    timed = lambda i: step(i)
    launch = "separate calls"
    if st.new_req is not None and len(st.new_req) == B and not args.separate:
        # the library's whole step: the new token of every request written inside the step
        # (tsa_decode_step); the kernel-timing pass below runs the same kernels as separate calls
        k_new, v_new, i_new = st.new_k, st.new_v, st.new_idx
        launch = "tsa_decode_step"

        def timed(i):
            q, qidx = qsets[i % n_sets]
            tsa.decode_step(st.pool, 0, st.params, k_new, v_new, i_new, q, qidx, st.widx,
                            st.table_dev, st.lens_dev, st.out, st.workspace, topk_out=st.topk,
                            stream=stream)
    if args.graph:
        launch = "graph"
        graphs = [tsa.StepGraph(st.pool, 0, st.params, q, qidx, st.widx, st.table_dev, st.lens_dev,
                                st.out, st.workspace, topk_out=st.topk,
                                append=None if st.new_req is None else
                                (st.new_req, st.new_pos, st.new_k, st.new_v, st.new_idx, None))
                  for q, qidx in qsets]
        timed = lambda i: graphs[i % n_sets].launch(stream)
    for i in range(args.warmup):
        timed(i)
    torch.cuda.synchronize()
    # Throughput (`value`): K steps back to back, no event between kernels or steps (on this
    # runtime an event between two kernels leaves the GPU idle for a few microseconds).
    t0 = time.perf_counter()
    for i in range(args.steps):
        timed(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps

    # Step-time distribution: events around each step, back to back ("warm"), then with a
    # 512 MiB scrub written before each step outside its interval, so that neither L2 nor the
    # 256 MB last-level cache holds anything of the step before ("scrubbed").
    scrub = torch.zeros((512 << 20) // 4, dtype=torch.int32, device="cuda")
    dist = {}
    for label, do_scrub in (("warm", False), ("scrubbed", True)):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            if do_scrub:
                scrub.add_(1)
            evs[i][0].record(stream)
            timed(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        dist[label] = _pct([a.elapsed_time(b_) for a, b_ in evs])
    del scrub

    # Per-kernel durations: the same steps again as separate calls, with HIP events recorded on
    # the launch stream between the kernels.  An interval includes the launch gap before its
    # kernel, so these durations are upper bounds of the kernels' own.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    # the timed loop may have run other kernels (the one-launch step): warm the separate calls up
    # first, so that no first-launch cost lands in the event pass
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in events])  # ms
    t_append, t_index, t_topk, t_attn = per.mean(axis=0)
    # the last step of that pass used query set (K - 1) mod n_sets: its selection is in st.topk

    # algorithmic bytes per launch
    lens = st.lens.astype(np.int64)
    D_I = w.index_dim
    idx_bytes, idx_flops, attn_bytes, attn_flops = algorithmic_counts(w, lens)
    n_sel = np.minimum(lens, w.top_k)
    row = _row_bytes(w)

    attn_src = _attn_src(w)
    # Bytes HBM must deliver at the least.  Requests of a shared-prefix workload alias the same
    # prefix pages, so a row several requests read is counted once; elsewhere this equals the
    # algorithmic count.
    idx_unique, attn_unique = idx_bytes, attn_bytes
    grp, plen = synth.prefix_groups(w)
    if grp is not None:
        shared_tok = (int(plen[0]) // w.page_size) * w.page_size
        idx_unique = int((lens.sum() - (B - 1) * shared_tok) * 2 * D_I + lens.sum() * 4)
        tk = st.topk.cpu().numpy().astype(np.int64)
        P = w.page_size
        slots = [st.table[b][tk[b][tk[b] >= 0] // P].astype(np.int64) * P + tk[b][tk[b] >= 0] % P
                 for b in range(B)]
        n_unique = int(np.unique(np.concatenate(slots)).size)
        attn_unique = int(attn_bytes - n_sel.sum() * row + n_unique * row)

    def roof(nbytes, unique, ms, src, key):
        gbs = unique / (ms * 1e-3) / 1e9
        traffic = _traffic(src, key)
        if key.startswith("attention/") and traffic is not None and _has_traffic(f"combine/{w.name}"):
            # the timed attention call is the gather kernel plus the split combine (a workload
            # whose counter run saw no combine launch has one split)
            comb = _traffic("attn_valu.hip", f"combine/{w.name}")
            traffic = None if comb is None else traffic + comb
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
             "algorithmic_bytes": nbytes, "kernel_ms": round(ms, 5)}
        if unique != nbytes:
            r["unique_bytes"] = unique
            r["bytes_basis"] = "unique: rows aliased by several requests counted once"
        return r

    out = {
        "metric": "sparse decode attention tokens/s + achieved HBM GB/s vs peak, 32k ctx top-2048",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "requests": B, "context": int(lens.max()),
                   "top_k": w.top_k, "page_size": w.page_size, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim_k": w.head_dim_k, "head_dim_v": w.head_dim_v,
                   "index_dim": D_I, "index_heads": w.index_heads, "parallelism": "none",
                   "launch": launch, "query_sets": n_sets},
        "step_ms": dict(dist, note="per-step HIP events; 'scrubbed' writes 512 MiB before each step, "
                                   "outside its interval; 'warm' runs the steps back to back"),
        "kernels_ms": {"kv_append": round(t_append, 5), "indexer_score": round(t_index, 5),
                       "topk": round(t_topk, 5), "attention": round(t_attn, 5)},
        "kernel_timing": "HIP events between kernels on the launch stream, over a second pass of "
                         "the same steps as separate calls (the throughput pass has no events "
                         "between kernels)",
        "roofline": dict(roof(idx_bytes, idx_unique, t_index, "indexer_score.hip", f"indexer_score/{w.name}"),
                         flops=idx_flops, tflops=round(idx_flops / (t_index * 1e-3) / 1e12, 2)),
        "roofline_attention": dict(roof(attn_bytes, attn_unique, t_attn, attn_src, f"attention/{w.name}"),
                                   flops=attn_flops,
                                   tflops=round(attn_flops / (t_attn * 1e-3) / 1e12, 2)),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
