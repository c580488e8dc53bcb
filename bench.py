#!/usr/bin/env python3
"""Benchmark: ragged per-row top-2048 on one MI355X.

One step = one topk_ragged launch over the whole prefill-shaped batch (4096
rows, row_stride 65536, lengths 61440+i, K=2048, N(0,1) plus a per-row offset
U(-4,4)), inputs already resident in HBM.  Prints one JSON line:
rows/s as `value`, effective HBM GB/s (valid fp32 score bytes / time) and its
fraction of the 8 TB/s peak, the roofline of the kernel, the CPU oracle timed
on a bounded sample of the same rows, and per-launch figures for the other
workloads (timed over rotating input copies so the 256 MB last-level cache
cannot serve them).

`--workload NAME` makes another workload the timed one (for profiling each
configuration on its own); workloads smaller than 1 GiB then rotate over
copies of their input totalling at least 1 GiB, one copy per step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "rows/sec + effective HBM GB/s (fraction of peak) for ragged per-row top-2048"
CSRC = os.path.join(ROOT, "row_radix_top_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30
POOL_BYTES = 1 << 30


def kernel_sources() -> list[str]:
    """Every source of the HIP library, in a fixed order."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".hpp", ".h", ".cpp")))


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_{workload}.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_of(text: str) -> str:
    """C/C++ source without its comments and with runs of whitespace folded
    to one space: what the compiler sees, so that editing a comment does not
    invalidate a counter reading.  String and character literals are kept
    as written."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel and launcher sources' code (comments stripped, see
    code_of): a stored counter reading is used only while this matches the
    hash it was taken with."""
    h = hashlib.sha256()
    for path in kernel_sources():
        h.update(os.path.basename(path).encode())
        h.update(code_of(open(path, encoding="utf-8").read()).encode())
    return h.hexdigest()


def algorithmic_bytes(lengths: np.ndarray, row_stride: int, K: int) -> tuple[int, int]:
    """(valid score bytes, algorithmic bytes): every valid fp32 score read
    once, plus K int32 indices written and one int32 length read per row."""
    n = np.clip(lengths.reshape(-1).astype(np.int64), 0, row_stride)
    valid = int(4 * n.sum())
    rows = n.size
    return valid, valid + rows * (4 * K + 4)


def time_launches(fn, n: int):
    """Average ms per launch over n back-to-back launches (HIP events on the
    launch stream, which is torch's current stream)."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(n):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources; else None."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def read_ceiling(pool, lengths, valid_bytes: int, launches: int = 100) -> float:
    """Effective GB/s of the library's streaming-read reference kernel, which
    reads exactly the valid bytes the selection reads (same tiles, load
    width and prefetch ring) and selects nothing; over the same rotating
    copies as the timed steps."""
    import torch
    import row_radix_top_amd as rrt
    keys = torch.empty(pool.shape[1], dtype=torch.int32, device=pool.device)
    n = pool.shape[0]
    for i in range(3):
        rrt.read_reference(pool[i % n], lengths, out=keys)
    ms = time_launches(lambda i: rrt.read_reference(pool[i % n], lengths, out=keys), launches)
    return valid_bytes / (ms * 1e-3) / 1e9


def copy_calibration(dev, launches: int = 10) -> float:
    """Launches a plain device copy of COPY_BYTES bytes `launches` times (the
    reference kernel for scaling HBM counter readings); returns its GB/s."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms = time_launches(lambda i: dst.copy_(src), launches)
    del src, dst
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """Time the CPU oracle (as is) on the same workload, on a bounded sample:
    the first rows that take about budget_s / 12 seconds on all threads.
    After one warm-up run, 5 timed runs at all threads and 5 at one thread;
    medians reported (generation and transfers excluded)."""
    from oracle import topk_ragged_oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    probe = min(64, w.num_rows)
    topk_ragged_oracle(w.scores[:8], w.flat_lengths[:8], w.K, threads=threads)  # warm
    t0 = time.perf_counter()
    topk_ragged_oracle(w.scores[:probe], w.flat_lengths[:probe], w.K, threads=threads)
    t_probe = max(time.perf_counter() - t0, 1e-6)
    # One all-thread run takes about budget_s / 12, so that 6 of them plus
    # 6 one-thread runs of a 1/threads share stay near budget_s in all.
    rows = int(min(w.num_rows, max(probe, probe * (budget_s / 12.0) / t_probe)))
    rows1 = max(1, min(rows, int(round(rows / threads)) or 1))

    def med(nrows, nthreads):
        topk_ragged_oracle(w.scores[:nrows], w.flat_lengths[:nrows], w.K, threads=nthreads)  # warm-up run
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            topk_ragged_oracle(w.scores[:nrows], w.flat_lengths[:nrows], w.K, threads=nthreads)
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), ts

    t_all, _ = med(rows, threads)
    t_one, _ = med(rows1, 1)
    valid, _ = algorithmic_bytes(w.flat_lengths[:rows], w.row_stride, w.K)
    valid1, _ = algorithmic_bytes(w.flat_lengths[:rows1], w.row_stride, w.K)
    return {
        "value": rows / t_all,
        "unit": "rows/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {w.num_rows} rows of the same workload on {threads} threads, median of 5 "
                  f"runs after 1 warm-up ({t_all:.3f} s each, {valid / t_all / 1e9:.2f} effective GB/s); "
                  f"first {rows1} rows on 1 thread, median of 5 after 1 warm-up",
        "cpu_model": cpu_model(),
        "single_thread_rows_per_s": rows1 / t_one,
        "single_thread_effective_GBps": round(valid1 / t_one / 1e9, 3),
    }


def host_call_us(fn, n: int) -> float:
    """Host time per call (Python binding + C ABI + kernel enqueue), timed
    on the CPU over n calls without waiting for the GPU in between."""
    import time
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    return (t1 - t0) / n * 1e6


def graph_replay_ms(fn, n: int, replays: int = 5) -> float:
    """Average ms per launch when n launches are captured in one HIP graph
    and the graph is replayed: the device-side cost without host overhead."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (replays * n)
    del g
    return ms


def bench_other(name: str, copies_bytes: int = 1 << 30, launches: int = 200):
    """Per-launch time of another workload over rotating input copies."""
    import torch
    import row_radix_top_amd as rrt
    from row_radix_top_amd import workloads
    w = workloads.make_workload(name)
    dev = torch.device("cuda:0")
    one = torch.from_numpy(w.scores).to(dev)
    ncopy = max(1, min(16384, copies_bytes // max(1, one.numel() * 4)))
    pool = torch.empty((ncopy,) + tuple(one.shape), dtype=torch.float32, device=dev)
    pool.copy_(one.unsqueeze(0).expand_as(pool))
    L = torch.from_numpy(w.flat_lengths).to(dev)
    out = torch.empty((w.num_rows, w.K), dtype=torch.int32, device=dev)
    ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev), dev)
    plan = rrt.query_plan(pool[0], w.K)

    def launch(i):
        rrt.topk_ragged(pool[i % ncopy], L, w.K, out=out, workspace=ws, next_n=w.next_n)

    for i in range(min(20, ncopy)):
        launch(i)
    ms = time_launches(launch, launches)
    host_us = host_call_us(launch, launches)
    graph_ms = graph_replay_ms(launch, min(launches, 100))
    valid, _ = algorithmic_bytes(w.flat_lengths, w.row_stride, w.K)
    res = {
        "us_per_launch": round(ms * 1e3, 3),
        "graph_us_per_launch": round(graph_ms * 1e3, 3),
        "host_us_per_call": round(host_us, 3),
        "rows_per_s": w.num_rows / (ms * 1e-3),
        "effective_GBps": round(valid / (ms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(valid / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "rotating_copies": ncopy,
        "path": plan["path"], "block": plan["block"], "grid": plan["grid"], "wg_per_row": plan["wg_per_row"],
    }
    del pool, ws, out
    torch.cuda.empty_cache()
    return res


def decode_latency(launches: int = 400):
    """Per-launch host and device overhead on the decode shape (64 rows,
    row_stride 32768, K=2048, no workspace): what a decode step pays.

    host: the Python binding's call, and the bare C-ABI call through ctypes
    with ready pointers (enqueue only, no waiting on the GPU).  device:
    eager back-to-back launches and hipGraph replay (HIP events), next to two
    floors on the same input, both replayed from a hipGraph so that the host
    cost of a call (about as long as these kernels) does not set the pace: a
    launch whose rows are all empty (it reads no scores and only writes the
    -1 padding) and the streaming-read reference (reads every valid score,
    selects nothing)."""
    import ctypes
    import time
    import torch
    import row_radix_top_amd as rrt
    from row_radix_top_amd import binding, workloads
    w = workloads.make_workload("decode")
    dev = torch.device("cuda:0")
    one = torch.from_numpy(w.scores).to(dev)
    ncopy = max(1, min(1024, (1 << 30) // (one.numel() * 4)))
    pool = torch.empty((ncopy,) + tuple(one.shape), dtype=torch.float32, device=dev)
    pool.copy_(one.unsqueeze(0).expand_as(pool))
    L = torch.from_numpy(w.flat_lengths).to(dev)
    Z = torch.zeros_like(L)
    out = torch.empty((w.num_rows, w.K), dtype=torch.int32, device=dev)
    keys = torch.empty(w.num_rows, dtype=torch.int32, device=dev)
    nbytes = rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev)
    assert nbytes == 0, "the decode shape needs no workspace"
    lib = binding.load()
    sp = int(torch.cuda.current_stream(dev).cuda_stream)
    ptrs = [pool[i].data_ptr() for i in range(ncopy)]
    lp, op = L.data_ptr(), out.data_ptr()
    fn = lib.topk_ragged

    def abi(i):
        rc = fn(ptrs[i % ncopy], w.row_stride, lp, w.num_rows, 1, w.K, op, None, sp)
        if rc != 0:
            raise rrt.TopKError(rc, "topk_ragged", lib.topk_ragged_last_error().decode())

    def py(i):
        rrt.topk_ragged(pool[i % ncopy], L, w.K, out=out)

    # The C-ABI call's host cost, taken apart with calls of the same library:
    # a call that returns a constant (the ctypes floor), and the plan alone
    # (device lookup, occupancy cache, planning; no launch).  What remains of
    # a launching call is hipLaunchKernel.
    plan = binding.Plan()
    plan_p = ctypes.byref(plan)
    qp = lib.topk_ragged_query_plan
    ver = lib.topk_ragged_version

    def plan_only(i):
        rc = qp(ptrs[i % ncopy], w.num_rows, w.row_stride, w.K, None, sp, plan_p)
        if rc != 0:
            raise rrt.TopKError(rc, "topk_ragged_query_plan", lib.topk_ragged_last_error().decode())

    for i in range(20):
        abi(i)
    torch.cuda.synchronize()
    ctypes_us = host_call_us(lambda i: ver(), launches)
    plan_us = host_call_us(plan_only, launches)
    abi_us = host_call_us(abi, launches)
    res = {
        "config": "decode: 64 rows, row_stride 32768, lengths U{1..32768}, K=2048, no workspace",
        "eager_us_per_launch": round(time_launches(abi, launches) * 1e3, 3),
        "graph_us_per_launch": round(graph_replay_ms(py, 100) * 1e3, 3),
        "host_us_per_call_binding": round(host_call_us(py, launches), 3),
        "host_us_per_call_c_abi": round(abi_us, 3),
        "host_us_ctypes_floor": round(ctypes_us, 3),
        "host_us_plan_only": round(plan_us, 3),
        "host_us_library": round(plan_us - ctypes_us, 3),
        "host_us_hip_launch": round(abi_us - plan_us, 3),
        "empty_rows_us_per_launch": round(graph_replay_ms(
            lambda i: rrt.topk_ragged(pool[i % ncopy], Z, w.K, out=out), 100) * 1e3, 3),
        "read_reference_us_per_launch": round(graph_replay_ms(
            lambda i: rrt.read_reference(pool[i % ncopy], L, out=keys), 100) * 1e3, 3),
    }
    del pool
    torch.cuda.empty_cache()
    return res


def extensions(w, scores, L, launches: int = 20):
    """Per-launch time of the extended entry points on the prefill-shaped
    batch, beside the plain launch: row offsets (a flat ragged layout),
    values, K = 4096, bf16 scores (the same batch rounded), and a transposed view
    (each row packed from a column stride of num_rows, then selected)."""
    import torch
    import row_radix_top_amd as rrt
    dev = scores.device
    out = torch.empty((w.num_rows, w.K), dtype=torch.int32, device=dev)
    vals = torch.empty((w.num_rows, w.K), dtype=torch.float32, device=dev)
    ws = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev), dev)
    n = np.clip(w.flat_lengths.astype(np.int64), 0, w.row_stride)
    starts = torch.from_numpy(np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int32)).to(dev)
    res = {"workload": "prefill-shaped batch (the bench line's)"}
    res["plain_us"] = round(time_launches(lambda i: rrt.topk_ragged(scores, L, w.K, out=out, workspace=ws),
                                          launches) * 1e3, 2)
    res["row_offsets_us"] = round(time_launches(
        lambda i: rrt.topk_ragged(scores, L, w.K, out=out, workspace=ws, row_offsets=starts), launches) * 1e3, 2)
    res["values_us"] = round(time_launches(
        lambda i: rrt.topk_ragged_values(scores, L, w.K, out=out, out_values=vals, workspace=ws), launches) * 1e3, 2)
    # K = 4096 (the large layout).
    out4 = torch.empty((w.num_rows, 4096), dtype=torch.int32, device=dev)
    ws4 = rrt.new_workspace(rrt.workspace_size(w.num_rows, w.row_stride, 4096, device=dev), dev)
    res["k4096_us"] = round(time_launches(lambda i: rrt.topk_ragged(scores, L, 4096, out=out4, workspace=ws4),
                                          launches) * 1e3, 2)
    del out4, ws4
    # The same scores rounded to bf16 (half the bytes).
    sb = scores.to(torch.bfloat16)
    bf_us = time_launches(lambda i: rrt.topk_ragged_bf16(sb, L, w.K, out=out, workspace=ws), launches) * 1e3
    valid = 2 * int(n.sum())
    res["bf16_us"] = round(bf_us, 2)
    res["bf16_rows_per_s"] = w.num_rows / (bf_us * 1e-6)
    res["bf16_effective_GBps"] = round(valid / (bf_us * 1e-6) / 1e9, 1)
    del ws, sb
    # The same scores as a transposed view: column stride num_rows.
    st = torch.empty((w.row_stride, w.num_rows), dtype=torch.float32, device=dev)
    st.copy_(scores.t())
    view = st.t()
    sws = rrt.new_workspace(rrt.strided_workspace_size(w.num_rows, w.row_stride, w.K, device=dev), dev)
    res["transposed_view_us"] = round(time_launches(
        lambda i: rrt.topk_ragged_strided(view, L, w.K, workspace=sws, out=out), launches) * 1e3, 2)
    del st, view, sws, out, vals
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads")
    ap.add_argument("--check", action="store_true", help="compare sampled rows with the oracle")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); rows are independent, "
              "so more GPUs would each run this same kernel on their own block of rows.", file=sys.stderr)
        return 2

    import torch
    import row_radix_top_amd as rrt
    from row_radix_top_amd import binding, workloads

    binding.load()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    log(f"generating workload {args.workload}")
    w = workloads.make_workload(args.workload)
    one = torch.from_numpy(w.scores).to(dev)
    # Inputs smaller than 1 GiB rotate over copies totalling at least 1 GiB,
    # one copy per step, so that the 256 MB last-level cache cannot serve them.
    ncopy = max(1, min(16384, -(-POOL_BYTES // max(1, one.numel() * 4)))) if one.numel() * 4 < POOL_BYTES else 1
    if ncopy > 1:
        pool = torch.empty((ncopy,) + tuple(one.shape), dtype=torch.float32, device=dev)
        pool.copy_(one.unsqueeze(0).expand_as(pool))
        del one
    else:
        pool = one.unsqueeze(0)
    lengths = torch.from_numpy(w.flat_lengths).to(dev)
    out = torch.empty((w.num_rows, w.K), dtype=torch.int32, device=dev)
    nbytes = rrt.workspace_size(w.num_rows, w.row_stride, w.K, device=dev)
    ws = rrt.new_workspace(nbytes, dev)
    plan = rrt.query_plan(pool[0], w.K)
    log(f"plan {plan}, {ncopy} input copies")

    def step(i=0):
        rrt.topk_ragged(pool[i % ncopy], lengths, w.K, out=out, workspace=ws, next_n=w.next_n)

    # The streaming-read ceiling is measured first: its launches also bring the
    # GPU out of idle before the warmup and timed steps.
    valid, alg = algorithmic_bytes(w.flat_lengths, w.row_stride, w.K)
    ceiling = read_ceiling(pool, lengths, valid)
    log(f"streaming-read reference: {ceiling:.1f} GB/s")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_ev = time_launches(lambda i: step(args.warmup + i), args.steps)
    wall = time.perf_counter() - t0
    log(f"{args.steps} steps: {ms_ev:.4f} ms/step (events), wall {wall:.3f} s")

    if args.check:
        from oracle import topk_ragged_oracle
        rows = np.linspace(0, w.num_rows - 1, min(64, w.num_rows)).astype(int)
        exp = topk_ragged_oracle(w.scores[rows], w.flat_lengths[rows], w.K)
        got = out.cpu().numpy()[rows]
        assert np.array_equal(got, exp), "bench output differs from the oracle"
        log("sampled rows match the oracle")

    if args.copy_calibration:
        log(f"copy calibration: {copy_calibration(dev):.1f} GB/s (read + write)")
    sec = ms_ev * 1e-3
    rows_per_s = w.num_rows / sec
    eff = valid / sec / 1e9
    achieved = alg / sec / 1e9
    traffic = measured_traffic(w.name)
    kname = ("topk_single_kernel" if plan["path"] == 1 else "topk_multi_kernel") + \
        f"<vec={plan['vec']}, block={plan['block']}, idx16={bool(plan['idx16'])}>"
    result = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_ev,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.description,
            "num_rows": w.num_rows, "row_stride": w.row_stride, "K": w.K, "next_n": w.next_n,
            "parallelism": "single GPU",
        },
        "effective_GBps": round(eff, 1),
        "frac_of_hbm_peak": round(eff / HBM_PEAK_GBPS, 4),
        "read_reference_GBps": round(ceiling, 1),
        "frac_of_read_reference": round(eff / ceiling, 4),
        "input_copies": ncopy,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": kname,
            "algorithmic_bytes_per_launch": alg,
        },
        "plan": {k: plan[k] for k in ("path", "block", "grid", "wg_per_row", "kmax", "vec", "idx16", "resident_cap")},
    }
    del pool

    if not args.no_others:
        others = {}
        for name in ("small", "decode", "mtp", "long_k1024", "long_k2048"):
            if name == w.name:
                continue
            log(f"timing {name}")
            others[name] = bench_other(name)
        result["workloads"] = others
        log("decode launch latency")
        result["decode_latency"] = decode_latency()
        if w.name == "prefill":
            log("extended entry points")
            scores = torch.from_numpy(w.scores).to(dev)
            result["extensions"] = extensions(w, scores, lengths)
            del scores

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
