#!/usr/bin/env python3
"""Decode-step benchmark of the HySparse2 cross-decoder hot path on one MI355X.

One step = full-attention layer over the whole cache (out, lse, scores) ->
token top-k + forced window -> 3 sparse layers over the shared index list,
all through the C ABI on the current stream, inputs resident in HBM.

Default workload: decode at 1M context with an FP8 (E4M3FN) cache -- B=1,
N=1048576, 32 q / 4 kv heads, head_dim 128, k=1024, window=128.  Prints ONE
JSON line on stdout (progress goes to stderr):
  value        microseconds per decode step (lower is better)
  hbm_gbps     algorithmic bytes of the step / step time
  roofline     the full-layer scan kernel against the 8 TB/s HBM peak, its
               duration from HIP events on the launch stream
  cpu_baseline the fp64 oracle on this host's cores, one whole step
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/decode-step (full scan + top-k + 3 sparse layers) & HBM GB/s at 1M ctx"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_TFLOPS = 2500.0
SCAN_SRCS = [os.path.join(ROOT, "long_context_sparse_full_amd", "csrc", f) for f in ("attn.hip", "hs2_internal.hpp", "select_common.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "full_scan_decode1m_fp8.md")
TRAFFIC_WORKLOAD = "decode1m_fp8"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def esize(kv: str) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1}[kv]


def algorithmic_bytes(spec) -> dict:
    """What the method itself must move per step (no implementation scratch)."""
    kv_bytes = 2 * spec.B * spec.Hkv * spec.N * spec.D * esize(spec.kv_dtype)
    scores = spec.B * spec.Tq * spec.Hkv * spec.N * 4
    gathered = 2 * spec.B * spec.Tq * spec.Hkv * spec.max_sel * spec.D * esize(spec.kv_dtype)
    return {"scan_kv": kv_bytes, "scores_write_read": 2 * scores, "gather_per_layer": gathered,
            "step": kv_bytes + 2 * scores + spec.n_sparse * gathered}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_entry(workload: str):
    """HBM bytes per scan launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from
    the committed rocprofv3 summary; None unless it was taken on this workload
    and on the current scan sources."""
    if workload != TRAFFIC_WORKLOAD or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                key, val = line[2:].split(":", 1)
                fields[key.strip()] = val.strip()
    src_hash = hashlib.sha256(b"".join(open(p, "rb").read() for p in SCAN_SRCS)).hexdigest()
    if fields.get("kernel_src_sha256") != src_hash or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="decode1m_fp8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-gather", type=int, default=1, choices=(0, 1),
                    help="sparse layers with the split-list gather (1, default) or one workgroup per (b, t, g) (0)")
    ap.add_argument("--topk-call", type=int, default=1, choices=(0, 1),
                    help="full layer + selection through hs2_full_attn_topk (1, default) or two calls (0)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="decode configs: only time the scan's read-pattern probe (with and without its code "
                         "stores) beside the scan itself")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from long_context_sparse_full_amd import hs2, synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the scale that turns those counters into HBM bytes
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(4):
            c0.record()
            dst.copy_(src)
            c1.record()
            torch.cuda.synchronize()
            log(f"[copy-probe] {n} B read + {n} B written in {c0.elapsed_time(c1):.3f} ms "
                f"({2 * n / c0.elapsed_time(c1) / 1e6:.1f} GB/s)")
        print(json.dumps({"copy_probe_bytes": n, "ms": c0.elapsed_time(c1)}), flush=True)
        return
    spec = synth.config(args.config)
    if spec.Tq != 1:
        return bench_chunk(spec, args)
    log(f"[bench] generating {spec.name}")
    t0 = time.time()
    inp = synth.make_inputs(spec)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()

    k, v, q = dev(inp.k), dev(inp.v), dev(inp.q_full)
    ks = dev(inp.k_scale) if inp.k_scale is not None else None
    vs = dev(inp.v_scale) if inp.v_scale is not None else None
    qs = [dev(x) for x in inp.q_sparse]
    B, Tq, Hq, D, Hkv, N = spec.B, spec.Tq, spec.Hq, spec.D, spec.Hkv, spec.N
    out = torch.empty_like(q)
    lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda")
    scores = torch.empty((B, Tq, Hkv, N), dtype=torch.float32, device="cuda")
    ws_full = torch.empty(hs2.full_attn_scores_workspace(k, v, Tq, Hq), dtype=torch.uint8, device="cuda")
    ws_topk = torch.empty(hs2.full_attn_topk_workspace(k, v, Tq, Hq), dtype=torch.uint8, device="cuda")
    if args.read_probe:
        # the scan's loads alone, then with its code stores, then the scan (same plan, grid and tiles)
        calls = (("scan_read_probe", lambda: hs2.debug_scan_read_probe(k, v, Hq, False, ks, vs, workspace=ws_full)),
                 ("scan_read_probe_codes", lambda: hs2.debug_scan_read_probe(k, v, Hq, True, ks, vs, workspace=ws_full)),
                 ("full_scan", lambda: hs2.full_attn_scores(k, v, q, spec.q_pos0, k_scale=ks, v_scale=vs, out=out,
                                                            lse=lse, scores=scores, workspace=ws_full)))
        res = {"workload": spec.name, "cache_bytes": int(k.numel() * k.element_size() + v.numel() * v.element_size())}
        for name, call in calls:
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            hs2.timing_enable(True)
            hs2.timing_reset()
            for _ in range(10):
                call()
            torch.cuda.synchronize()
            ms, n = hs2.timing_collect(name)
            hs2.timing_enable(False)
            hs2.timing_reset()
            res[f"{name}_us"] = round(ms * 1e3 / max(n, 1), 2)
            res[f"{name}_cache_read_tbps"] = round(res["cache_bytes"] / (ms * 1e-3 / max(n, 1)) / 1e12, 3)
            log(f"[read-probe] {name}: {res[f'{name}_us']} us")
        print(json.dumps({"read_probe": res}), flush=True)
        return
    idx = torch.empty((B, Tq, Hkv, spec.max_sel), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device="cuda")
    ws_sel = torch.empty(hs2.select_workspace(B, Tq, Hkv, N, 1), dtype=torch.uint8, device="cuda")
    sp_out = [torch.empty_like(q) for _ in qs]
    sp_lse = [torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda") for _ in qs]
    ws_gather = torch.zeros(max(hs2.sparse_attn_workspace(B, Tq, Hkv, D, spec.max_sel), 256), dtype=torch.uint8,
                            device="cuda")  # zero-filled once; every call leaves its counters at zero

    def step(layer1_events=None):
        if args.topk_call:
            hs2.full_attn_topk(k, v, q, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel, k_scale=ks,
                               v_scale=vs, out=out, lse=lse, scores=scores, idx=idx, count=cnt, workspace=ws_topk)
        else:
            hs2.full_attn_scores(k, v, q, spec.q_pos0, k_scale=ks, v_scale=vs, out=out, lse=lse, scores=scores,
                                 workspace=ws_full)
            hs2.select_topk_window(scores, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel, idx=idx,
                                   count=cnt, workspace=ws_sel)
        for i, ql in enumerate(qs):
            if i == 0 and layer1_events:
                layer1_events[0].record()
            if args.split_gather:
                hs2.sparse_attn_gather_ws(k, v, ql, idx, cnt, ws_gather, k_scale=ks, v_scale=vs, out=sp_out[i],
                                          lse=sp_lse[i])
            else:
                hs2.sparse_attn_gather(k, v, ql, idx, cnt, k_scale=ks, v_scale=vs, out=sp_out[i], lse=sp_lse[i])
            if i == 0 and layer1_events:
                layer1_events[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {ms_step * 1e3:.1f} us/step (events), {wall_ms * 1e3:.1f} us/step (wall)")

    # per-step distribution (an event pair around each step), warm and cold;
    # cold: a 512 MiB buffer read before each step, outside its events, evicts
    # L2 and the 256 MB memory-side cache with clean lines (a written buffer
    # would leave dirty lines whose write-back the next step would pay); the
    # first sparse layer is also timed on its own there (its rows then come
    # from HBM)
    def pct(xs, q):
        xs = sorted(xs)
        return round(xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))], 2)

    def one_step(layer1=None):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(layer1)
        b.record()
        return a, b

    flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    warm, cold, cold_l1 = [], [], []
    for _ in range(args.steps):
        warm.append(one_step())
    for i in range(args.steps):
        hs2.debug_stream_read(flush)
        la, lb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cold.append(one_step((la, lb)))
        cold_l1.append((la, lb))
    torch.cuda.synchronize()
    # the same cold steps again with every launch bracketed by events (these
    # events add a few us per launch, so the step distribution above has none)
    hs2.timing_reset()
    hs2.timing_enable(True)
    for i in range(args.steps):
        hs2.debug_stream_read(flush)
        step()
    torch.cuda.synchronize()
    cold_kernels = {}
    for name in hs2.timing_kernel_names():
        tot, n = hs2.timing_collect(name)
        if n and name != "stream_read":
            cold_kernels[name] = round(tot * 1e3 / n, 2)
    hs2.timing_enable(False)
    hs2.timing_reset()
    warm_us = [a.elapsed_time(b) * 1e3 for a, b in warm]
    cold_us = [a.elapsed_time(b) * 1e3 for a, b in cold]
    l1_us = [a.elapsed_time(b) * 1e3 for a, b in cold_l1]
    del flush
    gathered = algorithmic_bytes(spec)["gather_per_layer"]
    step_dist = {"warm_us": {"p10": pct(warm_us, 0.1), "p50": pct(warm_us, 0.5), "p90": pct(warm_us, 0.9)},
                 "cold_us": {"p10": pct(cold_us, 0.1), "p50": pct(cold_us, 0.5), "p90": pct(cold_us, 0.9)},
                 "cold_kernels_avg_us": cold_kernels,
                 "cold_sparse_layer1_us_p50": pct(l1_us, 0.5),
                 "cold_sparse_layer1_gbps": round(gathered / (pct(l1_us, 0.5) * 1e-6) / 1e9, 1)}
    log(f"[bench] step distribution: {json.dumps(step_dist)}")

    # the same step captured once in a HIP graph and replayed (the step has no
    # memsets, allocations or host syncs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record()
    for _ in range(args.steps):
        g.replay()
    gb.record()
    torch.cuda.synchronize()
    graph = {"us_per_step": round(ga.elapsed_time(gb) * 1e3 / args.steps, 2), "steps": args.steps}
    log(f"[bench] hip graph replay: {graph['us_per_step']} us/step")
    del g

    # per-kernel durations from HIP events bracketing each launch on its stream
    hs2.timing_reset()
    hs2.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for name in hs2.timing_kernel_names():
        tot, n = hs2.timing_collect(name)
        if n:
            kernels[name] = {"avg_us": round(tot * 1e3 / n, 3), "launches_per_step": n / args.steps}
    hs2.timing_enable(False)
    hs2.timing_reset()
    log(f"[bench] kernels: {json.dumps(kernels)}")

    ab = algorithmic_bytes(spec)
    scan_us = kernels["full_scan"]["avg_us"]
    achieved = ab["scan_kv"] / (scan_us * 1e-6) / 1e9
    roofline = {"kernel": "full_scan", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_entry(spec.name), "algorithmic_bytes_per_launch": ab["scan_kv"],
                "avg_launch_us": scan_us}

    gather_tp = gather_throughput(hs2, synth, k, v, ks, vs, spec, args) if spec.name == TRAFFIC_WORKLOAD else None
    extras = bench_extras(hs2, synth, k, v, ks, vs, q, spec, args) if spec.name == TRAFFIC_WORKLOAD else None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        log(f"[bench] oracle step on host ({threads} threads available)")
        c0 = time.perf_counter()
        _, _, s_or = oracle.full_attn_scores(inp.q_full, inp.k, inp.v, spec.q_pos0, k_scale=inp.k_scale,
                                             v_scale=inp.v_scale)
        c1 = time.perf_counter()
        idx_or, cnt_or = oracle.select_topk_window(s_or, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel)
        for ql in inp.q_sparse:
            oracle.sparse_attn(ql, inp.k, inp.v, idx_or, cnt_or, k_scale=inp.k_scale, v_scale=inp.v_scale)
        c2 = time.perf_counter()
        units = B * Tq * Hkv
        used = oracle.num_threads()
        cpu = {"value": round((c2 - c0) * 1e6, 1), "unit": "us/decode-step", "cores": used,
               "kind": "oracle",
               "sample": f"one whole decode step of {spec.name} ({units} kv-head units; with fewer units than "
                         f"threads the oracle's threads share each unit's positions and head dimensions), fp64; "
                         f"full layer {c1 - c0:.2f}s, select+3 sparse {c2 - c1:.2f}s",
               "threads_available": threads, "cpu_model": cpu_model()}
        log(f"[bench] oracle: {c2 - c0:.2f}s per step")

    line = {
        "metric": METRIC,
        "value": round(ms_step * 1e3, 2),
        "unit": "us/decode-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8e4m3-kv/bf16-q/f32-acc", "bf16": "bf16/f32-acc", "f32": "f32"}[spec.kv_dtype],
        "data": "synthetic (seeded; planted needle keys)",
        "config": {"workload": spec.name,
                   "full_and_select": "one call" if args.topk_call else "two calls", "B": B, "context": N, "Tq": Tq, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "kv_dtype": spec.kv_dtype, "top_k": spec.k, "window": spec.window,
                   "sparse_layers": spec.n_sparse},
        "hbm_gbps": round(ab["step"] / (ms_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_step": ab["step"],
        "wall_us_per_step": round(wall_ms * 1e3, 2),
        "step_distribution": step_dist,
        "hip_graph": graph,
        "kernels": kernels,
        "roofline": roofline,
        "gather_throughput": gather_tp,
        "extras": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def timed_us(call, reps, warm=2):
    """Average microseconds of `call` over reps, HIP events on the current stream."""
    import torch
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def bench_extras(hs2, synth, k, v, ks, vs, q, spec, args):
    """The other paths of the library at the decode workload's shapes:
    the competing-window selection, the decode step on a paged pool, 64-token
    block lists against token lists
    in the gather (throughput regime), sliding-window attention (decode at 1M
    FP8 and a 32K-token bf16 prefill on the banded matrix-core pass), and the
    K/V bridge of 4 layers (512-token block, and decoding's one-token append
    into 1M-row FP8 caches with the scales kept or maintained)."""
    import numpy as np
    import torch
    reps = max(5, args.steps)
    Hq, Hkv, D, N = spec.Hq, spec.Hkv, spec.D, spec.N
    ex = {}
    # full layer + top-k, both readings of the window (one call each)
    ws = torch.empty(hs2.full_attn_topk_workspace(k, v, 1, Hq), dtype=torch.uint8, device="cuda")
    o = [torch.empty(x, device="cuda", dtype=dt) for x, dt in (((1, 1, Hq, D), torch.bfloat16), ((1, 1, Hq), torch.float32),
                                                                ((1, 1, Hkv, N), torch.float32),
                                                                ((1, 1, Hkv, spec.max_sel), torch.int32),
                                                                ((1, 1, Hkv), torch.int32))]
    for label, comp in (("full_topk_us", False), ("full_topk_window_competes_us", True)):
        ex[label] = round(timed_us(lambda: hs2.full_attn_topk(
            k, v, q, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel, k_scale=ks, v_scale=vs, out=o[0],
            lse=o[1], scores=o[2], idx=o[3], count=o[4], workspace=ws, window_competes=comp), reps), 2)
    # the decode step (full layer + top-k, three sparse layers) on a paged
    # pool of 256-row pages in shuffled order, beside the same step on the
    # contiguous cache (the sparse layers take q as their query here)
    P = 256
    pps = -(-N // P)
    table = torch.from_numpy(np.random.default_rng(0xBA6E).permutation(pps).astype(np.int32)).view(1, pps).cuda()
    pools = []
    for src in (k, v):
        pool = torch.zeros((Hkv, pps * P, D), dtype=src.dtype, device="cuda")
        full_pages = N // P
        pool.view(Hkv, pps, P, D)[:, table[0, :full_pages].long()] = src[0, :, : full_pages * P].reshape(
            Hkv, full_pages, P, D)
        if N % P:
            t = int(table[0, full_pages])
            pool[:, t * P: t * P + N % P] = src[0, :, full_pages * P:]
        pools.append(pool)
    wsg = torch.zeros(hs2.sparse_attn_workspace(1, 1, Hkv, D, spec.max_sel), dtype=torch.uint8, device="cuda")
    go, gl = torch.empty_like(q), torch.empty((1, 1, Hq), dtype=torch.float32, device="cuda")

    def contiguous_step():
        hs2.full_attn_topk(k, v, q, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel, k_scale=ks, v_scale=vs,
                           out=o[0], lse=o[1], scores=o[2], idx=o[3], count=o[4], workspace=ws)
        for _ in range(3):
            hs2.sparse_attn_gather_ws(k, v, q, o[3], o[4], wsg, k_scale=ks, v_scale=vs, out=go, lse=gl)

    def paged_step():
        hs2.full_attn_topk_paged(pools[0], pools[1], table, P, N, q, spec.q_pos0, spec.k, spec.window,
                                 max_sel=spec.max_sel, k_scale=ks, v_scale=vs, out=o[0], lse=o[1], scores=o[2],
                                 idx=o[3], count=o[4], workspace=ws)
        for _ in range(3):
            hs2.sparse_attn_gather_paged(pools[0], pools[1], table, P, N, q, o[3], o[4], wsg, k_scale=ks,
                                         v_scale=vs, out=go, lse=gl)

    ex["paged_step"] = {"page_rows": P, "us": round(timed_us(paged_step, reps), 2),
                        "contiguous_us": round(timed_us(contiguous_step, reps), 2)}
    del ws, o, pools, wsg
    # gathers over token lists and over 64-token block lists (16 blocks + the 128-row window), 256 lists
    bq, rows = 256, spec.max_sel
    rng = np.random.default_rng(0xB10C)
    qg = (torch.randn(1, bq, Hq, D, device="cuda") * spec.q_std).to(torch.bfloat16)
    og = torch.empty_like(qg)
    tok_np, c_np = synth.random_index_lists(0x6A7 + bq, bq * Hkv, N, rows)
    blk_np = np.empty_like(tok_np)
    nb = spec.k // 64
    for u in range(bq * Hkv):
        blocks = np.sort(rng.choice((N - spec.window) // 64, nb, replace=False))
        blk_np[u, : nb * 64] = (blocks[:, None] * 64 + np.arange(64)[None, :]).ravel()
        blk_np[u, nb * 64:] = np.arange(N - spec.window, N)
    gb = bq * Hkv * rows * 2 * D * esize(spec.kv_dtype)
    cnt = torch.from_numpy(c_np.reshape(1, bq, Hkv)).cuda()
    for label, lists in (("token_lists", tok_np), ("block_lists", blk_np)):
        idx = torch.from_numpy(lists.reshape(1, bq, Hkv, -1)).cuda()
        us = timed_us(lambda: hs2.sparse_attn_gather(k, v, qg, idx, cnt, k_scale=ks, v_scale=vs, out=og,
                                                     want_lse=False), reps)
        ex[f"gather_256_{label}"] = {"avg_us": round(us, 2), "GBps": round(gb / (us * 1e-6) / 1e9, 1),
                                     "frac": round(gb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    del qg, og
    # sliding-window attention: decode at this cache, and a 32K-token bf16 prefill
    W = 128
    so = torch.empty_like(q)
    ex["swa128_decode_us"] = round(timed_us(lambda: hs2.swa_attn(k, v, q, spec.q_pos0, W, k_scale=ks, v_scale=vs,
                                                                 out=so, want_lse=False), reps), 2)
    Tp = 32768
    kp = torch.randn(1, Hkv, Tp, D, device="cuda").to(torch.bfloat16)
    vp = torch.randn(1, Hkv, Tp, D, device="cuda").to(torch.bfloat16)
    qp = (torch.randn(1, Tp, Hq, D, device="cuda") * spec.q_std).to(torch.bfloat16)
    op = torch.empty_like(qp)
    us = timed_us(lambda: hs2.swa_attn(kp, vp, qp, 0, W, out=op, want_lse=False), reps)
    flops = 4 * Hq * D * sum(min(W, t + 1) for t in range(Tp))
    # its HBM floor: the queries and the cache read once, the outputs written once
    sbytes = 2 * qp.numel() * qp.element_size() + kp.numel() * kp.element_size() + vp.numel() * vp.element_size()
    ex["swa128_prefill_32k"] = {"avg_us": round(us, 2), "tokens_per_s": round(Tp / (us * 1e-6), 1),
                                "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                                "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_TFLOPS, 4),
                                "algorithmic_flops": flops, "algorithmic_bytes": sbytes,
                                "GBps": round(sbytes / (us * 1e-6) / 1e9, 1),
                                "hbm_frac": round(sbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    del kp, vp, qp, op
    # K/V bridge of 4 layers from one hidden state
    L, dm = 4, 4096
    C = 2 * Hkv * D
    wl = (torch.randn(L, dm, C, device="cuda") / 64.0).to(torch.bfloat16)
    h512 = torch.randn(512, dm, device="cuda").to(torch.bfloat16)
    cb = [(torch.zeros(1, Hkv, 4096, D, device="cuda", dtype=torch.bfloat16),
           torch.zeros(1, Hkv, 4096, D, device="cuda", dtype=torch.bfloat16)) for _ in range(L)]
    us = timed_us(lambda: hs2.kv_bridge_layers(h512, wl, cb, 0, 1024), reps)
    ex["bridge_4_layers_512_tokens"] = {"avg_us": round(us, 2),
                                        "TFLOPs": round(2 * L * 512 * dm * C / (us * 1e-6) / 1e12, 1)}
    h1 = torch.randn(1, dm, device="cuda").to(torch.bfloat16)
    c8 = [(torch.zeros(1, Hkv, N, D, device="cuda", dtype=torch.uint8),
           torch.zeros(1, Hkv, N, D, device="cuda", dtype=torch.uint8),
           torch.full((1, Hkv), 1.0, device="cuda"), torch.full((1, Hkv), 1.0, device="cuda")) for _ in range(L)]
    wsb = torch.empty(max(hs2._bridge_layers_ws(L, 1, Hkv, D), 256), dtype=torch.uint8, device="cuda")
    for label, grow in (("keep", False), ("grow_no_growth", True)):
        us = timed_us(lambda: hs2.kv_bridge_layers(h1, wl, c8, 0, N - 1, grow=grow, workspace=wsb), reps)
        ex[f"append_1_token_4_layers_fp8_{label}_us"] = round(us, 2)
        ex[f"append_1_token_4_layers_fp8_{label}_weight_GBps"] = round(L * dm * C * 2 / (us * 1e-6) / 1e9, 1)
    del c8, cb, wl
    torch.cuda.empty_cache()
    log(f"[bench] extras: {json.dumps(ex)}")
    return ex


def gather_throughput(hs2, synth, k, v, ks, vs, spec, args):
    """The sparse-layer gather against the same 1M-position FP8 cache with B_q
    independent query streams, each with its own list of 1152 random rows per
    kv head (the decode step has B_q = 1).  Bytes = gathered K + V rows."""
    import numpy as np
    import torch
    res = []
    Hkv, D, N = spec.Hkv, spec.D, spec.N
    rows = spec.max_sel
    for bq in (1, 8, 64, 256):
        q = (torch.randn(1, bq, spec.Hq, D, device="cuda") * spec.q_std).to(torch.bfloat16)
        idx_np, c_np = synth.random_index_lists(0x6A7 + bq, bq * Hkv, N, rows)
        idx = torch.from_numpy(idx_np.reshape(1, bq, Hkv, -1)).cuda()
        cnt = torch.from_numpy(c_np.reshape(1, bq, Hkv)).cuda()
        ws = torch.zeros(max(hs2.sparse_attn_workspace(1, bq, Hkv, D, rows), 256), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(q)
        entry = {"B_q": bq, "rows_per_list": rows}
        for name, call in (("single", lambda: hs2.sparse_attn_gather(k, v, q, idx, cnt, k_scale=ks, v_scale=vs,
                                                                        out=out, want_lse=False)),
                           ("split", lambda: hs2.sparse_attn_gather_ws(k, v, q, idx, cnt, ws, k_scale=ks,
                                                                       v_scale=vs, out=out, want_lse=False))):
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            hs2.timing_reset()
            hs2.timing_enable(True)
            for _ in range(args.steps):
                call()
            torch.cuda.synchronize()
            tot, n = hs2.timing_collect("sparse_gather")
            hs2.timing_enable(False)
            hs2.timing_reset()
            us = tot * 1e3 / n
            gb = bq * Hkv * rows * 2 * D * esize(spec.kv_dtype)
            entry[name] = {"avg_us": round(us, 3), "GBps": round(gb / (us * 1e-6) / 1e9, 1),
                           "frac": round(gb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4), "bytes": gb}
        res.append(entry)
    log(f"[bench] gather throughput: {json.dumps(res)}")
    return res


def bench_chunk(spec, args):
    """Multi-query chunk: K/V bridge of the new tokens, full layer, token top-k
    and 64-token block selection, 3 sparse layers; tokens/s = Tq / chunk time."""
    import numpy as np
    import torch

    from long_context_sparse_full_amd import hs2, synth

    log(f"[bench] generating {spec.name}")
    inp = synth.make_inputs(spec)

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()

    k, v, q = dev(inp.k), dev(inp.v), dev(inp.q_full)
    qs = [dev(x) for x in inp.q_sparse]
    hidden, w = dev(inp.hidden), dev(inp.w_kv)
    B, Tq, Hq, D, Hkv, N = spec.B, spec.Tq, spec.Hq, spec.D, spec.Hkv, spec.N
    T = spec.bridge[0]
    out = torch.empty_like(q)
    lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda")
    scores = torch.empty((B, Tq, Hkv, N), dtype=torch.float32, device="cuda")
    ws_full = torch.empty(hs2.full_attn_scores_workspace(k, v, Tq, Hq), dtype=torch.uint8, device="cuda")
    ws_topk = torch.empty(hs2.full_attn_topk_workspace(k, v, Tq, Hq), dtype=torch.uint8, device="cuda")
    if args.read_probe:
        # the scan's loads alone, then with its code stores, then the scan (same plan, grid and tiles)
        calls = (("scan_read_probe", lambda: hs2.debug_scan_read_probe(k, v, Hq, False, ks, vs, workspace=ws_full)),
                 ("scan_read_probe_codes", lambda: hs2.debug_scan_read_probe(k, v, Hq, True, ks, vs, workspace=ws_full)),
                 ("full_scan", lambda: hs2.full_attn_scores(k, v, q, spec.q_pos0, k_scale=ks, v_scale=vs, out=out,
                                                            lse=lse, scores=scores, workspace=ws_full)))
        res = {"workload": spec.name, "cache_bytes": int(k.numel() * k.element_size() + v.numel() * v.element_size())}
        for name, call in calls:
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            hs2.timing_enable(True)
            hs2.timing_reset()
            for _ in range(10):
                call()
            torch.cuda.synchronize()
            ms, n = hs2.timing_collect(name)
            hs2.timing_enable(False)
            hs2.timing_reset()
            res[f"{name}_us"] = round(ms * 1e3 / max(n, 1), 2)
            res[f"{name}_cache_read_tbps"] = round(res["cache_bytes"] / (ms * 1e-3 / max(n, 1)) / 1e12, 3)
            log(f"[read-probe] {name}: {res[f'{name}_us']} us")
        print(json.dumps({"read_probe": res}), flush=True)
        return
    idx = torch.empty((B, Tq, Hkv, spec.max_sel), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device="cuda")
    bsel = spec.block_k * spec.block_size + spec.window
    bidx = torch.empty((B, Tq, Hkv, bsel), dtype=torch.int32, device="cuda")
    bcnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device="cuda")
    ws_sel = torch.empty(hs2.select_workspace(B, Tq, Hkv, N), dtype=torch.uint8, device="cuda")
    sp_out = [torch.empty_like(q) for _ in qs]

    def step():
        hs2.kv_bridge(hidden, w, k, v, 0, N - T)
        if args.topk_call:  # full layer and token top-k in one call
            hs2.full_attn_topk(k, v, q, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel, out=out, lse=lse,
                               scores=scores, idx=idx, count=cnt, workspace=ws_topk)
        else:
            hs2.full_attn_scores(k, v, q, spec.q_pos0, out=out, lse=lse, scores=scores, workspace=ws_full)
            hs2.select_topk_window(scores, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel, idx=idx,
                                   count=cnt, workspace=ws_sel)
        hs2.select_topk_window(scores, spec.q_pos0, spec.block_k, spec.window, block_size=spec.block_size,
                               max_sel=bsel, idx=bidx, count=bcnt, workspace=ws_sel)
        for i, ql in enumerate(qs):
            hs2.sparse_attn_gather(k, v, ql, idx, cnt, out=sp_out[i], want_lse=False)

    steps = max(1, min(args.steps, 5))
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    hs2.timing_reset()
    hs2.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for name in hs2.timing_kernel_names():
        tot, n = hs2.timing_collect(name)
        if n:
            kernels[name] = {"avg_us": round(tot * 1e3 / n, 3), "launches_per_step": n / steps}
    hs2.timing_enable(False)
    hs2.timing_reset()
    # the same bridge into an E4M3FN cache of the same shape (per-head scales)
    k8 = torch.zeros(k.shape, dtype=torch.uint8, device="cuda")
    v8 = torch.zeros_like(k8)
    sc8 = torch.full((B, Hkv), 1.0 / 112.0, dtype=torch.float32, device="cuda")
    for _ in range(2):
        hs2.kv_bridge(hidden, w, k8, v8, 0, N - T, k_scale=sc8, v_scale=sc8)
    torch.cuda.synchronize()
    hs2.timing_enable(True)
    for _ in range(steps):
        hs2.kv_bridge(hidden, w, k8, v8, 0, N - T, k_scale=sc8, v_scale=sc8)
    torch.cuda.synchronize()
    tot, n = hs2.timing_collect("kv_bridge")
    hs2.timing_enable(False)
    hs2.timing_reset()
    bridge_fp8_us = round(tot * 1e3 / max(n, 1), 3)
    del k8, v8
    # dense MFMA work of the chunk's full layer: query token t sees p_t + 1 positions;
    # QK^T and PV are 2 * Hq * D flops per (t, position) each; the score pass redoes QK^T
    visible = sum(spec.q_pos0 + t + 1 for t in range(Tq))
    flops_full = 2 * 2 * visible * Hq * D
    flops_score = 2 * visible * Hq * D
    roofline = None
    if "chunk_full" in kernels:
        us = kernels["chunk_full"]["avg_us"]
        tf = flops_full / (us * 1e-6) / 1e12
        roofline = {"kernel": "chunk_full", "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_TFLOPS, 4), "traffic": None,
                    "algorithmic_flops_per_launch": flops_full, "avg_launch_us": us}
        if "chunk_score" in kernels:
            us2 = kernels["chunk_score"]["avg_us"]
            roofline["score_pass"] = {"achieved": round(flops_score / (us2 * 1e-6) / 1e12, 1),
                                      "algorithmic_flops_per_launch": flops_score, "avg_launch_us": us2}
    cpu = None
    if not args.no_cpu_baseline:
        # bounded sample: the chunk's last S query tokens (each sees the whole
        # cache) through the same steps, and the bridge rows of S tokens
        import oracle
        S = 32
        threads = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        log(f"[bench] oracle on the last {S} query tokens ({threads} threads available)")
        c0 = time.perf_counter()
        oracle.kv_bridge(inp.hidden[-S:], inp.w_kv, Hkv, D)
        qp = spec.q_pos0 + Tq - S
        _, _, s_or = oracle.full_attn_scores(inp.q_full[:, -S:], inp.k, inp.v, qp)
        idx_or, cnt_or = oracle.select_topk_window(s_or, qp, spec.k, spec.window, max_sel=spec.max_sel)
        oracle.select_topk_window(s_or, qp, spec.block_k, spec.window, block_size=spec.block_size, max_sel=bsel)
        for ql in inp.q_sparse:
            oracle.sparse_attn(ql[:, -S:], inp.k, inp.v, idx_or, cnt_or)
        c1 = time.perf_counter()
        units = B * S * Hkv
        cpu = {"value": round(S / (c1 - c0), 2), "unit": "tokens/s", "cores": min(units, oracle.num_threads()),
               "kind": "oracle",
               "sample": f"the last {S} of the {Tq} query tokens of {spec.name} (each sees the whole cache): "
                         f"bridge rows, full layer, token and block selection, 3 sparse layers, fp64; "
                         f"{c1 - c0:.2f}s", "threads_available": threads, "cpu_model": cpu_model()}
        log(f"[bench] oracle: {c1 - c0:.2f}s for {S} tokens")
    print(json.dumps({"metric": "tokens/s per 512-query chunk (bridge + full + token & block select + 3 sparse)",
                      "value": round(Tq / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
                      "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16/f32-acc",
                      "data": "synthetic", "config": {"workload": spec.name, "Tq": Tq, "context": N,
                                                           "full_and_select": "one call" if args.topk_call else "two calls"},
                      "kernels": kernels, "kv_bridge_into_fp8_cache_us": bridge_fp8_us, "roofline": roofline,
                      "cpu_baseline": cpu}), flush=True)


if __name__ == "__main__":
    main()
