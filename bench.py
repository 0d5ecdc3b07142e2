#!/usr/bin/env python3
"""Benchmark of the paged decode-attention step on one MI355X.

A step is one pass of the whole path over one batch: append each sequence's
new token with pa_reshape_and_cache, then attend in the workload's own mode:
one pass per (sequence, KV head) with pa_decode, or, for the long-context
workload whose definition names split-sequence partitions, pa_decode_split
followed by the pa_reduce_lse merge (--mode overrides).  The default workload
is the largest one that fits one GPU: 256 sequences with an E4M3 cache and a
4096-token window.  Inputs are seeded synthetic data already resident in HBM
when timing starts.

Prints ONE JSON line.  `value` is KV GB/s of the whole step (in-window K+V
bytes read per step / wall time per step).  `roofline` is the decode kernel's
algorithmic bytes per launch / its average launch time (HIP events on the
launch stream) against 8 TB/s.  `cpu_baseline` times the CPU oracle on the
host cores over the same workload.

With --extend NAME the step is the multi-token one instead: append every
sequence's chunk of new tokens, then pa_extend; `value` is TFLOP/s of the
attention (4 * head_dim flops per (query head, token, attended key)) and the
roofline is the extend kernel against the bf16 dense matrix-core peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attention: KV GB/s (% of MI355X HBM peak) + µs/call"
EXTEND_METRIC = "paged extend attention: TFLOP/s (% of MI355X bf16 dense matrix peak)"
DEFAULT_CFG = 5
# Decode mode of each workload: only the long-context mixed batch is defined
# with split-sequence partitions (512 tokens) and an LSE reduce; the others are
# served by one pass per (sequence, KV head).
DEFAULT_MODE = {1: "unsplit", 2: "unsplit", 3: "split", 4: "unsplit", 5: "unsplit"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def family_sources(family: str, names) -> list:
    """The device sources a kernel family is built from: the extend kernel's
    file, or the decode driver, its tiles and instances; both include
    common.h and params.h and are launched through dispatch.*"""
    shared = ("common.h", "params.h", "dispatch.h", "dispatch.cpp")
    if family == "extend":
        return [f for f in names if f == "extend_mfma.hip" or f in shared]
    return [f for f in names if f.startswith(("decode_", "tile_")) or f in shared]


def kernel_source_hash(family: str = "decode") -> str:
    """Hash of the sources one kernel family is built from (recorded traffic
    stays valid while they are unchanged)."""
    csrc = os.path.join(ROOT, "paged_kv_cache_267_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(family_sources(family, os.listdir(csrc))):
        if f.endswith((".h", ".hip", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def decode_algorithmic_bytes(wl, partition_size: int | None) -> int:
    """Bytes the decode kernel must move per launch: in-window K+V, the query,
    the block-table entries it reads, and its outputs (partials + LSEs when
    split, the output rows otherwise)."""
    import numpy as np
    from paged_kv_cache_267_amd.workloads import ELEM_BYTES
    eq = ELEM_BYTES[wl.q_dtype]
    L = wl.seq_lens.astype(np.int64)
    lo = np.maximum(0, L - wl.sliding_window) if wl.sliding_window > 0 else np.zeros_like(L)
    bs = wl.block_size
    blocks = np.where(L > lo, (L + bs - 1) // bs - lo // bs, 0)
    table = int(blocks.sum()) * 4 * wl.num_kv_heads
    q = wl.num_seqs * wl.num_q_heads * wl.head_dim * eq
    if partition_size:
        P = partition_size
        parts = np.where(L > lo, (L + P - 1) // P - lo // P, 0)
        out = int(parts.sum()) * wl.num_q_heads * (wl.head_dim + 1) * 4
    else:
        out = wl.num_seqs * wl.num_q_heads * wl.head_dim * eq
    return wl.kv_bytes() + q + table + out


def load_traffic(kernel_hash: str, workload: str, mode: str):
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    key = f"{workload}/{mode}"
    r = rec.get(key)
    if not r or r.get("kernel_hash") != kernel_hash:
        return None
    return r.get("bytes_per_launch")


def record_traffic(fetch_csv: str, write_csv: str, key: str, khash: str, copy_mib: int,
                   kernel: str = "decode_persistent_kernel") -> dict:
    """HBM bytes per launch of the decode kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled so that the
    plain device copy of copy_mib MiB in the same run reads / writes exactly
    its size.  Merged into profiles/decode_traffic.json under key (kernel:
    the name the counter rows carry)."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    pick = lambda d, s: [v for k, vs in d.items() if s in k for v in vs]
    copy_kib = copy_mib * 1024.0
    sf = copy_kib / max(pick(f, "copyBuffer"))
    sw = copy_kib / max(pick(w, "copyBuffer"))
    df, dwr = pick(f, kernel), pick(w, kernel)
    fb = statistics.mean(df) * 1024 * sf
    wb = statistics.mean(dwr) * 1024 * sw
    rec = {"kernel_hash": khash, "bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb),
           "write_bytes": int(wb), "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
           "dispatches": [len(df), len(dwr)],
           "source": "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of bench.py"}
    try:
        allrec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        allrec = {}
    allrec[key] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return rec


def read_ceiling(chunk_bytes: int, gib: int = 2, reps: int = 10):
    """What HBM delivers to this access pattern on this GPU: the library's
    gather-read probe over a fresh 2 GiB buffer cut into chunks of one
    (block, head) tile, read once in a seeded random order (a paged gather)
    and once in order (a streaming read), each averaged over reps calls."""
    import torch
    import paged_kv_cache_267_amd as pa
    n = (gib << 30) // chunk_bytes
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(1234)
    res = {}
    for name, ids in (("gather", torch.randperm(n, generator=g)), ("linear", torch.arange(n))):
        ids = ids.to(torch.int32).cuda()
        pa.pa_probe_gather_read(buf, ids, chunk_bytes, sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            pa.pa_probe_gather_read(buf, ids, chunk_bytes, sink)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        res[f"{name}_GB/s"] = round((gib << 30) / (us * 1e-6) / 1e9, 1)
    del buf
    res["probe"] = (f"pa_probe_gather_read: {gib} GiB in {chunk_bytes}-byte chunks, "
                    "random order (gather) and in order (linear)")
    return res


def per_launch_us(fn, n: int, stream) -> float:
    """Average duration of one launch of fn: n launches back to back on the
    stream, HIP events around them (no marker between launches)."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def queued_launch_us(fn, n: int, stream) -> tuple:
    """Average GPU duration of one launch of fn for kernels of a few
    microseconds, which back to back would run at the host's launch rate:
    the n launches are queued behind a head start of device fills, so the GPU
    meets them already enqueued and runs them back to back.  Returns (us per
    launch, whether the host had enqueued all n before the GPU reached them)."""
    import torch
    fn()
    torch.cuda.synchronize()
    pad = torch.empty(64 << 20, dtype=torch.float32, device="cuda")   # 256 MiB
    h0, h1, a, b = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    h0.record(stream)
    for _ in range(max(8, n // 2)):
        pad.fill_(1.0)
    h1.record(stream)
    a.record(stream)
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    host_us = (time.perf_counter() - t0) * 1e6
    b.record(stream)
    torch.cuda.synchronize()
    del pad
    return a.elapsed_time(b) * 1e3 / n, host_us < h0.elapsed_time(h1) * 1e3


def timed_steps(step, n: int, stream):
    """The timed region: n steps launched back to back, synchronised on both
    sides; returns (wall seconds, GPU event microseconds per step)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(n):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, a.elapsed_time(b) * 1e3 / n


def graph_check_and_time(step, out, n: int, warmup: int, stream) -> dict:
    """The step captured in a HIP graph: three replays must reproduce the
    eager output bit for bit; then n replays are timed (reported only: on
    this platform a replay costs more than the eager launches it holds)."""
    import torch
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    bits = (lambda t: t.view(torch.int16)) if out.dtype == torch.bfloat16 else (lambda t: t)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(bits(out), bits(ref)):
            raise RuntimeError("graph replay differs from the eager step")
    for _ in range(warmup):
        g.replay()
    T, ev_us = timed_steps(g.replay, n, stream)
    del g
    return {"ms_per_step": round(T / n * 1e3, 4), "event_us_per_step": round(ev_us, 2),
            "check": "3 replays bit-identical to the eager step output"}


def settle(step, ms: float) -> dict:
    """Run the step untimed until `ms` milliseconds of sustained GPU work have
    passed.  The GPU raises its clocks only under sustained load: after an
    idle spell its first launches run several times slower and the next few
    dozen still ramp, so a timed region that follows a short warm-up measures
    the ramp rather than the steady state of a busy server."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= ms:
            return {"ms": round(el, 1), "steps": n,
                    "why": "untimed sustained load before the warm-up steps, so the timed "
                           "steps run at the steady-state clocks"}


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, on the host cores, over the whole workload;
    repeated until at least budget_s seconds of work (at least once)."""
    import oracle
    from tests.helpers import oracle_caches, oracle_decode
    kc, vc = oracle_caches(wl)
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle_decode(wl, kc, vc)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 50:
            break
    return {"value": round(wl.kv_bytes() * runs / el / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"whole workload ({wl.num_seqs} seqs x {wl.num_q_heads} q heads), "
                      f"{runs} run(s), {el:.1f} s, fp64, {round(el / runs * 1e3, 1)} ms/call"}


def extend_flops(wl) -> int:
    """Algorithmic flops of one extend launch: QK and PV, 2 * head_dim each,
    per (query head, token, attended key)."""
    return 4 * wl.head_dim * wl.num_q_heads * wl.attended_pairs()


def extend_cpu_baseline(wl, budget_s: float):
    """The oracle on a seeded sample of output rows, timed on the host cores
    until about budget_s seconds of work; rate in the same flop count."""
    import numpy as np
    import oracle
    from tests.helpers import oracle_caches
    kc, vc = oracle_caches(wl)
    rng = np.random.default_rng(7)
    total = wl.num_tokens * wl.num_q_heads
    qsl, L = wl.query_start_loc, wl.seq_lens.astype(np.int64)
    seq_of = np.searchsorted(qsl, np.arange(wl.num_tokens), side="right") - 1
    pos = L[seq_of] - (qsl[seq_of + 1] - qsl[seq_of]) + (np.arange(wl.num_tokens) - qsl[seq_of])
    keys = pos + 1 if wl.sliding_window <= 0 else np.minimum(pos + 1, wl.sliding_window)
    done_rows = flops = 0
    t0 = time.perf_counter()
    while True:
        rows = np.sort(rng.choice(total, size=min(256, total), replace=False)).astype(np.int32)
        oracle.extend(wl.query, kc, vc, wl.block_tables, wl.seq_lens, qsl,
                      block_size=wl.block_size, scale=wl.scale, num_kv_heads=wl.num_kv_heads,
                      q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype,
                      sliding_window=wl.sliding_window, k_scale=wl.k_scale,
                      v_scale=wl.v_scale, rows=rows)
        done_rows += rows.size
        flops += int(4 * wl.head_dim * keys[rows // wl.num_q_heads].sum())
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done_rows} random (token, head) rows of {total} in batches of 256, "
                      f"{el:.1f} s, fp64"}


def run_extend(args):
    import numpy as np
    import torch
    from paged_kv_cache_267_amd import workloads as W
    from paged_kv_cache_267_amd.harness import DeviceWorkload

    wl = W.extend_config(args.extend)
    dw = DeviceWorkload(wl)
    dw.fill_history()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: {wl.description}", file=sys.stderr, flush=True)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    settled = settle(dw.step_extend, args.settle_ms) if args.settle_ms > 0 else None
    for _ in range(args.warmup):
        dw.step_extend()
    torch.cuda.synchronize()
    T, step_event_us = timed_steps(dw.step_extend, args.steps, stream)
    t_app, q_app = queued_launch_us(dw.append_new, args.steps, stream)
    t_ext = per_launch_us(dw.extend, args.steps, stream)
    graph = None
    if not args.no_graph:
        graph = graph_check_and_time(dw.step_extend, dw.out, args.steps, args.warmup, stream)
    ms_step = T / args.steps * 1e3
    fl = extend_flops(wl)
    value = fl / (ms_step * 1e-3) / 1e12
    achieved = fl / (t_ext * 1e-6) / 1e12
    G = wl.num_q_heads // wl.num_kv_heads
    rec = {
        "metric": EXTEND_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{wl.q_dtype} q / {wl.kv_dtype} kv, bf16 matrix products, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "global_batch": wl.num_seqs, "query_tokens": wl.num_tokens,
                   "max_query_len": wl.max_query_len,
                   "seq_len_mean": float(wl.seq_lens.mean()), "parallelism": "single GPU"},
        "step_breakdown_us": {"reshape_and_cache": round(t_app, 2), "extend": round(t_ext, 2),
                              "event_per_step": round(step_event_us, 2),
                              "wall_per_step": round(ms_step * 1e3, 2),
                              "short_kernels_queued": q_app},
        "step_timing": ("K eager steps back to back on one stream (wall clock, synchronised on "
                        "both sides); the extend kernel's time from K back-to-back launches "
                        "between two HIP events; the append's from K launches queued behind "
                        "device fills, so that they run back to back at the GPU's rate, not the "
                        "host's"),
        "graph": graph,
        "settle": settled,
        "flops_per_step": fl,
        "kv_bytes_per_step": wl.kv_bytes(),
        "unique_kv_bytes_per_step": int(wl.unique_kv_bytes()),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(kernel_source_hash("extend"), wl.name, "extend"),
                     "kernel": f"extend_kernel<{1 if wl.kv_dtype == 'bf16' else 2}, "
                               f"{wl.head_dim}, {wl.block_size}, ...>, G={G}",
                     "algorithmic_flops_per_launch": fl, "avg_launch_us": round(t_ext, 2),
                     "kernel_hash": kernel_source_hash("extend")},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample) ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = extend_cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=DEFAULT_CFG, help="workload 1..5")
    ap.add_argument("--mode", choices=["split", "unsplit"], default=None,
                    help="decode mode (default: the workload's own, see DEFAULT_MODE)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed sustained run of the step before the warm-up steps, in ms "
                         "(0: none); see settle()")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a reference "
                         "kernel of known traffic for hardware-counter scaling)")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: store the decode kernel's HBM bytes per launch from "
                         "rocprofv3 counter CSVs of this configuration (with "
                         "--calibrate-copy-mib set as in those runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager launches only (default: the step is also "
                         "captured in a HIP graph, checked against the eager result, and the "
                         "headline is the graph replay time)")
    ap.add_argument("--cold-reps", type=int, default=30,
                    help="calls timed one by one after a 1 GiB read+write flush of the caches "
                         "(0: skip)")
    ap.add_argument("--kernel", choices=["auto", "valu", "mfma"], default="auto",
                    help="decode kernel family (auto: matrix cores for GQA groups >= 8)")
    ap.add_argument("--extend", default=None,
                    help="time the multi-token step on this extend workload instead "
                         "(chunked_prefill_bf16, prefix_extend_bf16, extend_fp8_window)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU leg "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.extend:
        if args.record_traffic:
            assert args.calibrate_copy_mib > 0, "--calibrate-copy-mib must name the copy size"
            from paged_kv_cache_267_amd import workloads as W
            rec = record_traffic(*args.record_traffic, f"{args.extend}/extend",
                                 kernel_source_hash("extend"), args.calibrate_copy_mib,
                                 kernel="extend_kernel")
            print(json.dumps({f"{args.extend}/extend": rec}))
            return
        run_extend(args)
        return

    import numpy as np
    import torch
    import paged_kv_cache_267_amd as pa
    from paged_kv_cache_267_amd import workloads as W
    from paged_kv_cache_267_amd.harness import DeviceWorkload

    wl = W.config(args.config)
    if args.mode is None:
        args.mode = DEFAULT_MODE[args.config]
    pa.pa_set_decode_kernel(args.kernel)
    kv_code = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8_e4m3": pa.PA_FP8_E4M3}[wl.kv_dtype]
    kernel = pa.pa_decode_kernel_name(kv_code, wl.num_q_heads, wl.num_kv_heads)
    split = args.mode == "split"
    psize = args.partition_size or wl.partition_size
    khash = kernel_source_hash()
    mode_key = f"{kernel}/{args.mode}{psize if split else ''}"
    if args.record_traffic:
        assert args.calibrate_copy_mib > 0, "--calibrate-copy-mib must name the copy size"
        rec = record_traffic(*args.record_traffic, f"{wl.name}/{mode_key}", khash,
                             args.calibrate_copy_mib)
        print(json.dumps({f"{wl.name}/{mode_key}": rec}))
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dw = DeviceWorkload(wl, partition_size=psize)
    dw.fill_history()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: {wl.description}; mode={args.mode} partition={psize}",
          file=sys.stderr, flush=True)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    tile_bytes = wl.head_dim * wl.block_size * W.ELEM_BYTES[wl.kv_dtype]
    ceiling = None if args.no_ceiling else read_ceiling(tile_bytes)

    stream = torch.cuda.current_stream()
    settled = settle(lambda: dw.step(split=split), args.settle_ms) if args.settle_ms > 0 else None
    for _ in range(args.warmup):
        dw.step(split=split)
    torch.cuda.synchronize()

    # the timed region: K whole steps (append, attend, merge) back to back
    T, step_event_us = timed_steps(lambda: dw.step(split=split), args.steps, stream)
    # each kernel of the step on its own: K back-to-back launches
    t_app, q_app = queued_launch_us(dw.append_new, args.steps, stream)
    t_dec = per_launch_us(dw.decode_split if split else dw.decode_unsplit, args.steps, stream)
    t_red, q_red = queued_launch_us(dw.reduce, args.steps, stream) if split else (0.0, True)

    graph = None
    if not args.no_graph:
        graph = graph_check_and_time(lambda: dw.step(split=split), dw.out, args.steps,
                                     args.warmup, stream)

    cold = None
    if args.cold_reps > 0:
        # each call after a 1 GiB read+write pass that evicts L2 and the MALL,
        # then a 512 MiB read of another buffer that writes the dirty lines back
        # (so no write-back of the flush overlaps the timed call)
        flush = torch.zeros((1 << 30) // 4, dtype=torch.float32, device="cuda")
        clean = torch.zeros((512 << 20) // 4, dtype=torch.float32, device="cuda")
        dec_us, call_us = [], []
        for _ in range(args.cold_reps):
            flush.add_(1.0)
            clean.sum()
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record(stream)
            if split:
                dw.decode_split()
            else:
                dw.decode_unsplit()
            b.record(stream)
            if split:
                dw.reduce()
            c.record(stream)
            torch.cuda.synchronize()
            dec_us.append(a.elapsed_time(b) * 1e3)
            call_us.append(a.elapsed_time(c) * 1e3)
        del flush, clean
        pct = lambda v: {"p10": round(float(np.percentile(v, 10)), 2),
                         "median": round(float(np.median(v)), 2),
                         "p90": round(float(np.percentile(v, 90)), 2)}
        cold = {"reps": args.cold_reps, "decode_us": pct(dec_us), "call_us": pct(call_us),
                "decode_kv_GB/s_median": round(wl.kv_bytes() / (np.median(dec_us) * 1e-6) / 1e9, 1),
                "flush": "1 GiB read+write, then a 512 MiB read, before each call"}

    ms_step = T / args.steps * 1e3
    kv = wl.kv_bytes()
    value = kv / (ms_step * 1e-3) / 1e9
    alg = decode_algorithmic_bytes(wl, psize if split else None)
    achieved = alg / (t_dec * 1e-6) / 1e9
    traffic = load_traffic(khash, wl.name, mode_key)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{wl.q_dtype} q / {wl.kv_dtype} kv, fp32 accumulate", "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "global_batch": wl.num_seqs, "seq_len_mean": float(wl.seq_lens.mean()),
                   "seq_len_max": int(wl.seq_lens.max()), "mode": args.mode,
                   "partition_size": psize if split else None, "parallelism": "single GPU"},
        "step_breakdown_us": {"reshape_and_cache": round(t_app, 2), "decode": round(t_dec, 2),
                              "reduce_lse": round(t_red, 2),
                              "event_per_step": round(step_event_us, 2),
                              "wall_per_step": round(ms_step * 1e3, 2),
                              "short_kernels_queued": bool(q_app and q_red)},
        "step_timing": ("K eager steps back to back on one stream (wall clock, synchronised on "
                        "both sides); the decode kernel's time from K back-to-back launches "
                        "between two HIP events; the append's and the LSE merge's from K "
                        "launches queued behind device fills, so that they run back to back at "
                        "the GPU's rate, not the host's"),
        "graph": graph,
        "settle": settled,
        "kv_bytes_per_step": kv,
        "unique_kv_bytes_per_step": int(wl.unique_kv_bytes()),
        "cold": cold,
        "pct_of_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_over_algorithmic": round(traffic / alg, 4) if traffic else None,
                     "kernel": f"decode_persistent_kernel<{'MfmaTile' if kernel == 'mfma' else 'ValuTile'}"
                               f"<{kv_code}, {wl.head_dim}, {wl.block_size}, "
                               f"{wl.num_q_heads // wl.num_kv_heads}>>",
                     "algorithmic_bytes_per_launch": alg, "avg_launch_us": round(t_dec, 2),
                     "kernel_hash": khash},
        "read_ceiling": ceiling,
        "cpu_baseline": None,
    }
    if ceiling:
        rec["roofline"]["frac_of_gather_ceiling"] = round(achieved / ceiling["gather_GB/s"], 4)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
