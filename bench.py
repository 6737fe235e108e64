#!/usr/bin/env python3
"""Benchmark of one CSA2 decode step on one MI355X.

A step = one decode query per sequence through the workload's whole layer
schedule (indexer scan + Top-K for Full layers, pool rescoring for Reindex
layers, sparse attention in every layer), replayed from a captured HIP graph.
Inputs (FP4 main KV, indexer keys, per-layer queries and windows) are built and
resident in HBM before the timed region.

Prints one JSON line.  Default workload: 8 sequences x 1,048,576 entries through
the 20-layer decoder schedule (Full + Reuse x 3, then 4 x [Reindex + Reuse x 3]).
Other workloads: --workload decode_64k_b64 | reindex_256k_b32 | mtp_64k_b64 |
full_decode_4k | prefill_32k | append_b64.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "CSA2 decode queries/s at 64K–1M ctx; achieved HBM GB/s vs MI355X peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m_b8")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--full-in-pool", action="store_true",
                    help="decode: Full layers take their Top-K inside the candidate pool built from "
                         "their own scores (the other reading of the Full selection)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size reference "
                         "for HBM byte counters)")
    ap.add_argument("--profile-call", choices=["scan", "attn", "select"], default=None,
                    help="decode workloads: after building the inputs, run only this call "
                         "--kernel-reps times (the first layer's indexer scan, its attention, or "
                         "the Full layer's pool + Top-K from its scores) and exit; for counter runs")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kv_cache_compression_03_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(name, *sources):
    """HBM bytes per launch from a committed counter summary under profiles/, or
    None when there is none or it was taken on other kernel sources."""
    tf = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(tf):
        return None
    rec = {}
    with open(tf) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
    # counters taken on an older kernel source no longer describe this one
    if rec.get("source_sha") != source_sha(*sources):
        return None
    return int(rec["hbm_bytes_per_launch"])


def copy_calibration(args, torch):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters of the same profiled command."""
    if not args.copy_calibration_mib:
        return
    n = args.copy_calibration_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {n} bytes read, {n} bytes written")
    del src, dst


def copy_bandwidth(torch, nbytes=1 << 30, reps=5) -> float:
    """Measured device-to-device copy rate (read + write bytes / s, GB/s) of a plain
    torch copy of `nbytes`: what this GPU's HBM delivers beside the 8 TB/s spec."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    return 2 * nbytes / t / 1e9


def algorithmic_bytes(wl) -> dict:
    """Bytes a step must move at least: every Full layer streams the indexer keys
    of all entries; a Reindex layer gathers the keys of its pool; every layer reads
    its selected FP4 entries, its window, its query and writes its output."""
    entry = wl.d // 2 + wl.d // 16          # FP4 codes + E4M3 scales
    ik = wl.d_i * 2
    # per query its selected entries, query and output; the window once per sequence
    per_attn = wl.Tq * (wl.K * entry + wl.H_q * wl.d * 2 + wl.H_q * wl.d * 4) + wl.S * wl.d
    layers = wl.layers
    full = layers.count("F") * wl.B * wl.N * ik
    reidx = layers.count("R") * wl.B * wl.PB * wl.PE * ik
    attn = len(layers) * wl.B * per_attn
    return {"full_scan": full, "reindex": reidx, "attention": attn, "total": full + reidx + attn}


def build_inputs(wl, torch, bd, sch):
    import synth
    dev = torch.device("cuda")
    B, N, d = wl.B, wl.N, wl.d
    codes = torch.empty(B, N, d // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(B, N, d // 16, dtype=torch.uint8, device=dev)
    kidx = torch.empty(B, N, wl.d_i, dtype=torch.bfloat16, device=dev)
    W = torch.from_numpy(synth.w_ik(wl).view(np.int16)).view(torch.bfloat16).to(dev)
    t0 = time.time()
    build_us = None
    if wl.T:
        # the cache from hidden states: compressor (m tokens per entry) -> FP4 + keys
        tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        H = tt(np.stack([synth.hidden(wl, b) for b in range(B)]))
        Wkv, Wz = (tt(x) for x in synth.compressor_weights(wl))
        kv = torch.empty(B, N, d, dtype=torch.float32, device=dev)
        def build():
            bd.csa2_compress(H, Wkv, Wz, wl.m, rope_dim=wl.rope_dim, out=kv)
            bd.csa2_quant_fp4(kv.view(B * N, d), codes=codes.view(B * N, d // 2),
                              scales=scales.view(B * N, d // 16), W_ik=W, k_idx=kidx.view(B * N, wl.d_i))
        for _ in range(2):
            build()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            build()
        e1.record()
        torch.cuda.synchronize()
        build_us = e0.elapsed_time(e1) * 1e3 / 10
        log(f"cache built from hidden states: {B} x {wl.T} tokens -> {N} entries, {build_us:.1f} us")
    else:
        workers = min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(workers) as ex:
            futs = [ex.submit(synth.main_kv, wl, b) for b in range(B)]
            for b, f in enumerate(futs):
                x = torch.from_numpy(f.result()).to(dev)
                bd.csa2_quant_fp4(x, codes=codes[b], scales=scales[b], W_ik=W, k_idx=kidx[b])
                del x
        torch.cuda.synchronize()
        log(f"cache built: {B} x {N} entries in {time.time() - t0:.1f}s")
    layers = []
    for li, mode in enumerate(wl.layers):
        qm = np.stack([synth.q_main(wl, li, b, wl.Tq) for b in range(B)])
        sw = np.stack([synth.swa_tokens(wl, li, b) for b in range(B)])
        qi = w = None
        if mode in "FR":
            qi = np.stack([synth.q_index(wl, li, b, wl.Tq) for b in range(B)])
            w = np.stack([synth.head_weights(wl, li, b, wl.Tq) for b in range(B)])
        tb = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        layers.append(sch.LayerBuffers(tb(qm), tt(sw), None if qi is None else tb(qi),
                                       None if w is None else tt(w)))
    return codes, scales, kidx, layers, build_us


def time_scan(wl, torch, bd, kidx, layers, reps):
    """Average duration of the indexer-scan kernel launch (the dominant kernel),
    measured with HIP events on the stream it is launched on."""
    st = torch.cuda.current_stream()
    scores = torch.empty(wl.B, wl.Tq, wl.N, dtype=torch.float32, device="cuda")
    lb = layers[0]
    for _ in range(3):
        bd.csa2_index_full(lb.q_idx, lb.w, kidx, scores=scores)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        bd.csa2_index_full(lb.q_idx, lb.w, kidx, scores=scores)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps / 1e3  # seconds


def oracle_threads() -> int:
    """Threads the oracle's numpy runs on (its BLAS thread pool; 1 if unknown)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


# entries of the oracle's bounded sample of a decode workload (the oracle's setup
# for a whole 1M-entry sequence alone -- quantiser and keys in float64 -- takes
# over a minute of host time)
CPU_SAMPLE_ENTRIES = 1 << 18


def cpu_baseline(wl, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload: decode
    steps of the first sequences (two, or one when the sample is shortened) through
    the whole layer schedule, repeated until `seconds` of CPU work.  Sequences
    longer than CPU_SAMPLE_ENTRIES entries are sampled as their first
    CPU_SAMPLE_ENTRIES entries and the rate is scaled by the entry ratio (the scan
    over all entries dominates a step), which the record states."""
    import synth
    from oracle.csa2 import LayerInputs, compress, decode_step, indexer_k, quant_fp4
    threads = oracle_threads()
    from oracle.csa2 import swa_window_rows
    W = synth.w_ik(wl)
    n_e = min(wl.N, CPU_SAMPLE_ENTRIES)
    nseq = 2 if n_e == wl.N else 1
    P, S = wl.N * wl.m, wl.S
    seqs = []
    for b in range(nseq):
        if wl.T:   # the cache from hidden states, through the oracle's compressor
            Wkv, Wz = synth.compressor_weights(wl)
            kv = compress(synth.hidden(wl, b), Wkv, Wz, wl.m, rope_dim=wl.rope_dim).astype(np.float32)
        else:
            kv = synth.main_kv(wl, b, 0, n_e)
        q8 = quant_fp4(kv)
        k = indexer_k(q8.codes, q8.scales, W)
        for t in range(wl.Tq):   # query t sees the window tokens up to its own position
            rows = (np.arange(S) if wl.Tq == 1 else
                    swa_window_rows(P + t, S, P + wl.Tq - S, S - wl.Tq + 1))
            lays = []
            for li, mode in enumerate(wl.layers):
                lays.append(LayerInputs(synth.q_main(wl, li, b, wl.Tq)[t],
                                        synth.swa_tokens(wl, li, b)[rows],
                                        synth.q_index(wl, li, b, wl.Tq)[t] if mode in "FR" else None,
                                        synth.head_weights(wl, li, b, wl.Tq)[t] if mode in "FR" else None))
            seqs.append((q8, k, lays))
    n, t0 = 0, time.perf_counter()
    while True:
        q8, k, lays = seqs[n % len(seqs)]
        decode_step(wl.layers, lays, q8.codes, q8.scales, k, K=wl.K, G=wl.G, PB=wl.PB, PE=wl.PE)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    rate = n / el
    rec = {"value": rate * n_e / wl.N, "unit": "queries/s", "cores": int(threads),
           "host_cpus": os.cpu_count(), "kind": "oracle"}
    if n_e == wl.N:
        rec["sample"] = (f"{n} single-query decode steps of sequences 0-{nseq - 1} of {wl.name} "
                         f"({'+'.join(wl.layers)}, {wl.N} entries), {el:.1f}s, float64 numpy on "
                         f"{threads} BLAS threads")
    else:
        rec["sample"] = (f"{n} single-query decode steps of sequence 0 of {wl.name} "
                         f"({'+'.join(wl.layers)}) over its first {n_e} entries, {el:.1f}s, "
                         f"float64 numpy on {threads} BLAS threads: {rate:.2f} steps/s, scaled by "
                         f"{n_e}/{wl.N} entries")
        rec["sample_rate"] = rate
    return rec


MFMA_BF16_PEAK_TFLOPS = 2500.0
APPENDS_PER_GRAPH = 16


def prefill_flops(wl) -> dict:
    """Dense-contraction flops of one prefill chunk: the causal indexer scoring
    (2 * h_i * d_i per visible (query, entry) pair) and the attention (2 * 2 * d
    per (query, head, key) for Q·K and P·V, over K selected entries + its window)."""
    vis = sum(min(wl.N, (t + 1) // wl.m) for t in range(wl.pos0, wl.T))
    idx = 2 * wl.h_i * wl.d_i * vis
    keys = sum(min(wl.K, min(wl.N, (t + 1) // wl.m)) + min(wl.n_win, t + 1) for t in range(wl.pos0, wl.T))
    attn = len(wl.layers) * wl.H_q * 4 * wl.d * keys
    comp = 2 * wl.chunk * wl.d_model * 2 * wl.d
    return {"indexer": idx, "attention": attn, "compressor": comp, "visible_pairs": vis}


def prefill_cpu_baseline(wl, seconds):
    """The oracle, as it stands, on a bounded sample of the prefill chunk: the
    chunk's entries are compressed (float64), quantised with the cached prefix and
    given their keys in untimed setup; then the chunk's last 64 query rows go
    through the per-query path (scores of every visible entry, Top-K, attention
    in every layer) until `seconds` of CPU work."""
    import synth
    from oracle.codecs import bf16_to_f64
    from oracle.csa2 import (compress, index_scores, indexer_k, quant_fp4, sparse_attention, topk,
                             visible_count)
    f = bf16_to_f64 if wl.h_dtype == "bf16" else (lambda a: a)
    Wkv, Wz = synth.compressor_weights(wl)
    kv_new = compress(f(synth.hidden(wl)), f(Wkv), f(Wz), wl.m, pos0=wl.pos0,
                      rope_dim=wl.rope_dim).astype(np.float32)
    pre, new = quant_fp4(synth.main_kv(wl, 0, 0, wl.n_pre)), quant_fp4(kv_new)
    codes = np.concatenate([pre.codes, new.codes])
    scales = np.concatenate([pre.scales, new.scales])
    k = indexer_k(codes, scales, synth.w_ik(wl))
    R, r0 = 64, wl.chunk - 64
    inputs = []
    for li, mode in enumerate(wl.layers):
        qi = synth.q_index(wl, li, 0, R, r0) if mode == "F" else None
        w = synth.head_weights(wl, li, 0, R, r0) if mode == "F" else None
        inputs.append((synth.q_main(wl, li, 0, R, r0), synth.swa_tokens(wl, li, 0), qi, w))
    none = np.full(wl.K, -1, dtype=np.int64)
    n, t0 = 0, time.perf_counter()
    while True:
        r = R - 1 - (n % R)
        pos = wl.pos0 + r0 + r
        nv = visible_count(pos, wl.N, wl.m)
        sel = none
        for mode, (qm, sw, qi, w) in zip(wl.layers, inputs):
            if mode == "F":
                sel = topk(index_scores(qi[r], w[r], k[:nv]), wl.K)
            sparse_attention(qm[r], codes, scales, none if mode == "S" else sel, sw, q_pos=pos,
                             swa_pos0=wl.swa_pos0, n_win=wl.n_win)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": n / el, "unit": "tokens/s", "cores": oracle_threads(), "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{n} query rows (the last 64 of the chunk, cycled) through scores of every "
                      f"visible entry, Top-{wl.K} and attention in {len(wl.layers)} layers, {el:.1f}s, "
                      f"float64 numpy; the chunk's compressor, quantisation and keys ran untimed "
                      f"in setup"}


def prefill_main(args, wl, torch, bd, sch):
    """One prefill chunk (compress, FP4 + indexer keys, Full + Reuse layers), from a
    captured graph; inputs resident in HBM.  value = chunk tokens / s."""
    import synth
    dev = torch.device("cuda")
    N, n_pre, Tq, d = wl.N, wl.n_pre, wl.chunk, wl.d
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    Wik = bf(synth.w_ik(wl))
    codes = torch.empty(1, N, d // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(1, N, d // 16, dtype=torch.uint8, device=dev)
    kidx = torch.empty(1, N, wl.d_i, dtype=torch.bfloat16, device=dev)
    bd.csa2_quant_fp4(tt(synth.main_kv(wl, 0, 0, n_pre)), codes=codes[0, :n_pre],
                      scales=scales[0, :n_pre], W_ik=Wik, k_idx=kidx[0, :n_pre])
    H = bf(synth.hidden(wl))
    Wkv, Wz = (bf(x) for x in synth.compressor_weights(wl))
    layers = []
    for li, mode in enumerate(wl.layers):
        layers.append(sch.LayerBuffers(
            bf(synth.q_main(wl, li, 0, Tq)[None]), tt(synth.swa_tokens(wl, li, 0)[None]),
            bf(synth.q_index(wl, li, 0, Tq)[None]) if mode == "F" else None,
            tt(synth.head_weights(wl, li, 0, Tq)[None]) if mode == "F" else None))
    torch.cuda.synchronize()
    log(f"prefill inputs built: {Tq} queries, {len(layers)} layers")
    run = sch.PrefillChunk(wl.layers, N, n_pre, Tq, d, wl.h_i, wl.d_i, wl.H_q, wl.S, wl.K, wl.m,
                           wl.pos0, wl.swa_pos0, wl.n_win, wl.rope_dim)
    copy_calibration(args, torch)
    step = lambda: run.step(H, Wkv, Wz, Wik, codes, scales, kidx, layers)
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        step = g.replay
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    step_s = e0.elapsed_time(e1) / 1e3 / args.steps
    log(f"timed {args.steps} chunks: {step_s * 1e6:.1f} us/chunk")
    # the indexer-scoring launch alone (the contraction the MFMA roofline is quoted for)
    lb = layers[0]
    st = torch.cuda.current_stream()
    for _ in range(2):
        bd.csa2_index_full(lb.q_idx, lb.w, kidx, q_pos=run.q_pos, m=wl.m, scores=run.scores)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(args.kernel_reps):
        bd.csa2_index_full(lb.q_idx, lb.w, kidx, q_pos=run.q_pos, m=wl.m, scores=run.scores)
    e1.record(st)
    e1.synchronize()
    idx_s = e0.elapsed_time(e1) / args.kernel_reps / 1e3
    fl = prefill_flops(wl)
    achieved = fl["indexer"] / idx_s / 1e12
    traffic = traffic_record(f"traffic_index_prefill_{wl.name}.txt", "index_prefill.hip", "common.h")
    log(f"indexer: {idx_s * 1e6:.1f} us/launch, {achieved:.1f} TFLOP/s")
    out = {
        "metric": "CSA2 prefill chunk tokens/s; indexer MFMA TFLOP/s vs MI355X bf16 peak",
        "value": Tq / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "chunk_tokens": Tq, "context_tokens": wl.T,
                   "entries": N, "m": wl.m, "d": d, "d_model": wl.d_model,
                   "indexer": f"{wl.h_i}x{wl.d_i}", "heads": wl.H_q, "top_k": wl.K,
                   "schedule": wl.schedule, "graph": not args.no_graph,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "indexer scoring (causal Q·K^T, bf16)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                     "launch_us": idx_s * 1e6, "algorithmic_flops_per_launch": fl["indexer"]},
        "chunk_flops": fl,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = prefill_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def append_main(args, wl, torch, bd):
    """Decode cache append: one new FP4 entry per sequence (with its indexer key)
    into one row of each sequence's cache, and the token's window KV into that
    position's slot of all L layer windows; one csa2_cache_append per step, 16
    steps (rows N-16 .. N-1) per graph replay; inputs resident in HBM.
    value = appended tokens / s."""
    import synth
    dev = torch.device("cuda")
    B, d, d_i, L, S, cap = wl.B, wl.d, wl.d_i, len(wl.layers), wl.S, wl.N
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    codes = torch.zeros(B, cap, d // 2, dtype=torch.uint8, device=dev)
    scales = torch.zeros(B, cap, d // 16, dtype=torch.uint8, device=dev)
    kidx = torch.zeros(B, cap, d_i, dtype=torch.bfloat16, device=dev)
    swa = torch.zeros(L, B, S, d, dtype=torch.uint8, device=dev)
    W = bf(synth.w_ik(wl))
    kv_h = np.stack([synth.main_kv(wl, b, cap - 1, cap)[0] for b in range(B)])
    win_h = synth.new_token_window(wl)
    kv, win = torch.from_numpy(kv_h).to(dev), torch.from_numpy(win_h).to(dev)
    copy_calibration(args, torch)
    # R appends per graph replay (rows N-R .. N-1, their window slots), as R decode
    # steps' appends would run: one replay per append would time the host's graph
    # launch rather than the device
    R = APPENDS_PER_GRAPH
    rows = [cap - R + i for i in range(R)]
    log(f"workload {wl.name}: B={B} d={d} d_i={d_i} windows {L} x {S}, rows {rows[0]}..{rows[-1]}, "
        f"{R} appends per graph")
    def step():
        for r in rows:
            bd.csa2_cache_append(codes, scales, r, kv=kv, W_ik=W, k_idx=kidx, win=win, swa=swa, slot=r % S)
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        step = g.replay
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    step_s = e0.elapsed_time(e1) / 1e3 / args.steps / R   # per append
    log(f"timed {args.steps * R} appends: {step_s * 1e6:.1f} us/append")
    # algorithmic bytes of one call: entries in, W_ik in, codes + scales + keys out,
    # window KV in, window codes out
    nbytes = B * d * 4 + d * d_i * 2 + B * (d // 2 + d // 16 + 2 * d_i) + L * B * d * 4 + L * B * d
    # the compressor at this shape (B sequences x m tokens), timed separately for
    # context: it makes the entries this call appends
    H = bf(synth.append_hidden(wl))
    Wkv_b, Wz_b = synth.compressor_weights(wl)
    Wkv, Wz = bf(Wkv_b), bf(Wz_b)
    kvo = torch.empty(B, 1, d, dtype=torch.float32, device=dev)
    for _ in range(2):
        bd.csa2_compress(H, Wkv, Wz, wl.m, pos0=cap * wl.m - wl.m, out=kvo)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.kernel_reps):
        bd.csa2_compress(H, Wkv, Wz, wl.m, pos0=cap * wl.m - wl.m, out=kvo)
    e1.record()
    torch.cuda.synchronize()
    comp_s = e0.elapsed_time(e1) / 1e3 / args.kernel_reps
    log(f"compressor at this shape: {comp_s * 1e6:.1f} us")
    out = {
        "metric": "CSA2 decode cache append: appended tokens/s; achieved HBM GB/s vs MI355X peak",
        "value": B / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps * R,
        "warmup": args.warmup * R,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "sequences": B, "d": d, "indexer_dim": d_i,
                   "windows": L, "window": S, "graph": not args.no_graph,
                   "appends_per_graph": R, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "cache_append_kernel (quantise, keys and window encode in one launch)",
                     "achieved": nbytes / step_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / step_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic_record(f"traffic_cache_append_{wl.name}.txt", "quant.hip", "common.h"),
                     "launch_us": step_s * 1e6, "algorithmic_bytes_per_launch": nbytes},
        "compress_at_this_shape_us": comp_s * 1e6,
    }
    if not args.no_cpu_baseline:
        from oracle.codecs import e4m3_encode
        from oracle.csa2 import indexer_k, quant_fp4
        W_h = synth.w_ik(wl)
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            q = quant_fp4(kv_h)
            indexer_k(q.codes, q.scales, W_h)
            e4m3_encode(win_h)
            n += 1
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n * B / el, "unit": "tokens/s", "cores": oracle_threads(),
                               "host_cpus": os.cpu_count(), "kind": "oracle",
                               "sample": f"{n} appends of all {B} sequences (quantise, key, window), "
                                         f"{el:.1f}s, float64 numpy"}
    print(json.dumps(out), flush=True)


def profile_call(args, wl, torch, bd, run, codes, scales, kidx, layers):
    """One call of the first layer, --kernel-reps times, eagerly (for counter runs:
    the kernels of that call are the only ones of the command besides setup)."""
    lb = layers[0]
    n = args.kernel_reps
    if args.profile_call == "scan":
        scores = torch.empty(wl.B, wl.Tq, wl.N, dtype=torch.float32, device="cuda")
        fn = lambda: bd.csa2_index_full(lb.q_idx, lb.w, kidx, scores=scores)
    elif args.profile_call == "select":
        scores = torch.empty(wl.B, wl.Tq, wl.N, dtype=torch.float32, device="cuda")
        pool = torch.empty(wl.B * wl.Tq, wl.PB * wl.PE, dtype=torch.int32, device="cuda")
        plen = torch.empty(wl.B * wl.Tq, dtype=torch.int32, device="cuda")
        sel = torch.empty(wl.B * wl.Tq, wl.K, dtype=torch.int32, device="cuda")
        ws = torch.empty(bd.csa2_index_full_workspace(wl.B, wl.Tq, wl.N, wl.h_i, wl.d_i, wl.G, wl.PB,
                                                      wl.PE, wl.K), dtype=torch.uint8, device="cuda")
        fn = lambda: bd.csa2_index_full(lb.q_idx, lb.w, kidx, scores=scores, pool=pool, pool_len=plen,
                                        K=wl.K, sel=sel, ws=ws)
    else:
        sel = torch.sort(torch.randint(0, wl.N, (wl.B, wl.Tq, wl.K), device="cuda"),
                         dim=-1).values.to(torch.int32)
        fn = lambda: bd.csa2_sparse_attn(lb.q_main, codes, scales, sel, lb.swa, out=run.out[0],
                                         ws=run.attn_ws)
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    log(f"profile call {args.profile_call}: {n} calls on {wl.name}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not "
              "part of this build", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from kv_cache_compression_03_amd import binding as bd
    from kv_cache_compression_03_amd import schedule as sch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bd.lib()
    wl = synth.workload(args.workload)
    if wl.chunk:
        return prefill_main(args, wl, torch, bd, sch)
    if wl.append:
        return append_main(args, wl, torch, bd)
    log(f"workload {wl.name}: B={wl.B} N={wl.N} d={wl.d} schedule={wl.schedule}")
    codes, scales, kidx, layers, build_us = build_inputs(wl, torch, bd, sch)
    copy_calibration(args, torch)
    run = sch.DecodeSchedule(wl.layers, wl.B, wl.N, wl.d, wl.h_i, wl.d_i, wl.H_q, wl.S, wl.K,
                             G=wl.G, PB=wl.PB, PE=wl.PE, Tq=wl.Tq, full_in_pool=args.full_in_pool)
    if args.profile_call:
        return profile_call(args, wl, torch, bd, run, codes, scales, kidx, layers)
    step_kw = {}
    if wl.Tq > 1:   # the queries sit at positions P .. P+Tq-1; the window ends at the last
        P = wl.N * wl.m
        q_pos = (P + torch.arange(wl.Tq, dtype=torch.int32, device="cuda")).repeat(wl.B, 1)
        step_kw = dict(q_pos=q_pos, swa_pos0=P + wl.Tq - wl.S, n_win=wl.S - wl.Tq + 1)
    if args.no_graph:
        step = lambda: run.step(codes, scales, kidx, layers, **step_kw)
    else:
        g = run.capture(codes, scales, kidx, layers, **step_kw)
        step = g.replay
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_s = e0.elapsed_time(e1) / 1e3 / args.steps
    log(f"timed {args.steps} steps: {step_s * 1e6:.1f} us/step (wall {t_wall / args.steps * 1e6:.1f} us)")

    ab = algorithmic_bytes(wl)
    scan_s = time_scan(wl, torch, bd, kidx, layers, args.kernel_reps)
    scan_bytes = wl.B * wl.N * wl.d_i * 2
    achieved = scan_bytes / scan_s / 1e9
    log(f"scan kernel: {scan_s * 1e6:.1f} us/launch, {achieved:.0f} GB/s")

    traffic = traffic_record(f"traffic_index_scores_{wl.name}.txt", "index.hip", "common.h")
    copy_gbs = copy_bandwidth(torch)
    log(f"device copy: {copy_gbs:.0f} GB/s (read + write)")

    out = {
        "metric": METRIC,
        "value": wl.B * wl.Tq / step_s,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "sequences": wl.B, "context_entries": wl.N, "m": wl.m,
                   "d": wl.d, "indexer": f"{wl.h_i}x{wl.d_i}", "heads": wl.H_q, "window": wl.S,
                   "top_k": wl.K, "schedule": wl.schedule, "queries_per_sequence": wl.Tq,
                   "full_top_k": "inside the pool" if args.full_in_pool else "global",
                   "graph": not args.no_graph, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": scan_kernel_name(wl) + " (Full-layer indexer scan)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "launch_us": scan_s * 1e6, "algorithmic_bytes_per_launch": scan_bytes,
                     "measured_copy_GB_s": copy_gbs, "frac_of_copy": achieved / copy_gbs},
        "step_hbm": {"algorithmic_bytes": ab["total"], "GB_s": ab["total"] / step_s / 1e9,
                     "frac": ab["total"] / step_s / 1e9 / HBM_PEAK_GBS, "breakdown": ab},
    }
    if wl.T:
        out["config"].update({"tokens": wl.T, "d_model": wl.d_model, "hidden": "f32"})
        out["cache_build_us"] = build_us
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def scan_kernel_name(wl) -> str:
    """The kernel csa2_index_full launches for the workload's scan: several query
    tiles per sequence take the multi-query kernel; one query over rows of at least
    2^19 entries (a multiple of 32, at least one 32-entry batch per CU) the scan
    that holds its scores in LDS; otherwise the one-shot scan."""
    if (wl.Tq * wl.h_i + 15) // 16 >= 2:
        return "index_scores_mq_kernel"
    if wl.Tq == 1 and wl.N >= 1 << 19 and wl.N % 32 == 0 and 256 <= wl.B * wl.N // 32 <= 256 * 1152:
        return "index_scores_persist_kernel"
    return "index_scores_kernel"


if __name__ == "__main__":
    main()
