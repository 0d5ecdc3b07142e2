"""CPU checks of bench.py's accounting, the numerators of every reported
roofline fraction, against brute-force enumeration of what the kernels read,
write and compute; the scaling of the HBM counters into the traffic record;
and the one-GPU guard.

Decode bytes per launch, per (sequence, KV head): the in-window keys' K and V,
the table entries of the blocks holding them, the G query rows and the G
output rows (or, split, a partition output + LSE per non-empty partition).
Extend flops: 2 * head_dim for QK and 2 * head_dim for PV per (query head,
new token, key the token attends to causally inside its window).
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench
from paged_kv_cache_267_amd import workloads as W


def brute_decode_bytes(wl, partition_size):
    e, eq = W.ELEM_BYTES[wl.kv_dtype], W.ELEM_BYTES[wl.q_dtype]
    total = 0
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        lo = max(0, L - wl.sliding_window) if wl.sliding_window > 0 else 0
        keys = list(range(lo, L))
        for _ in range(wl.num_kv_heads):
            total += 2 * len(keys) * wl.head_dim * e
            total += 4 * len({j // wl.block_size for j in keys})
        total += wl.num_q_heads * wl.head_dim * eq
        if partition_size:
            parts = {j // partition_size for j in keys}
            total += len(parts) * wl.num_q_heads * (wl.head_dim + 1) * 4
        else:
            total += wl.num_q_heads * wl.head_dim * eq
    return total


DECODE_CASES = [
    dict(seq_lens=[0, 1, 16, 17, 100, 333], num_q_heads=8, num_kv_heads=2, head_dim=64,
         block_size=16, kv_dtype="bf16"),
    dict(seq_lens=[5, 64, 65, 700], num_q_heads=4, num_kv_heads=4, head_dim=128, block_size=32,
         kv_dtype="f32", q_dtype="f32", sliding_window=37),
    dict(seq_lens=[1, 2, 129, 1000], num_q_heads=16, num_kv_heads=2, head_dim=128,
         block_size=64, kv_dtype="fp8_e4m3", sliding_window=1),
    dict(seq_lens=[300, 301, 0, 48], num_q_heads=8, num_kv_heads=1, head_dim=64,
         block_size=16, kv_dtype="fp8_e4m3", sliding_window=200),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
@pytest.mark.parametrize("partition_size", [None, 64, 128])
def test_decode_bytes_equal_enumeration(case, partition_size):
    kw = dict(DECODE_CASES[case])
    if partition_size and partition_size % kw["block_size"]:
        pytest.skip("partition size not a multiple of the block size")
    wl = W.random_case(700 + case, **kw)
    assert bench.decode_algorithmic_bytes(wl, partition_size) == \
        brute_decode_bytes(wl, partition_size)


def test_decode_bytes_named_config_closed_form():
    # the tiny f32 workload (4 sequences) holds no window and no split: 2 L D e per (sequence, KV head),
    # ceil(L / bs) table entries, one query and one output row per query head
    wl = W.config(1)
    e, eq, D = W.ELEM_BYTES[wl.kv_dtype], W.ELEM_BYTES[wl.q_dtype], wl.head_dim
    L = [int(x) for x in wl.seq_lens]
    expect = sum(wl.num_kv_heads * (2 * l * D * e + 4 * -(-l // wl.block_size)) for l in L)
    expect += 2 * wl.num_seqs * wl.num_q_heads * D * eq
    assert bench.decode_algorithmic_bytes(wl, None) == expect


@pytest.mark.parametrize("window", [0, 1, 50])
def test_extend_flops_equal_enumeration(window):
    wl = W.random_case(811, seq_lens=[1, 40, 200, 7, 90], q_lens=[1, 40, 17, 7, 3],
                       num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                       sliding_window=window)
    pairs = 0
    for L, n in zip(wl.seq_lens, wl.q_lens):
        for p in range(int(L) - int(n), int(L)):
            lo = max(0, p - window + 1) if window > 0 else 0
            pairs += max(0, p - lo + 1)
    assert bench.extend_flops(wl) == 4 * wl.head_dim * wl.num_q_heads * pairs


def test_traffic_record_scales_by_the_copy(tmp_path, monkeypatch):
    # the copy of 512 MiB reads as half its size and writes as its size: the
    # decode kernel's counters are scaled by x2 and x1
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    rows = [("FETCH_SIZE", "copyBuffer", 512 * 1024 / 2),
            ("FETCH_SIZE", "decode_persistent_kernel<T>", 1000.0),
            ("FETCH_SIZE", "decode_persistent_kernel<T>", 1002.0),
            ("FETCH_SIZE", "reshape_and_cache_kernel", 99.0)]
    wrows = [("WRITE_SIZE", "copyBuffer", 512 * 1024),
             ("WRITE_SIZE", "decode_persistent_kernel<T>", 8.0)]

    def csv(path, rs):
        with open(path, "w") as fh:
            fh.write("Counter_Name,Kernel_Name,Counter_Value\n")
            for c, k, v in rs:
                fh.write(f"{c},{k},{v}\n")
    csv(tmp_path / "f.csv", rows)
    csv(tmp_path / "w.csv", wrows)
    rec = bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl/mode",
                               "abc", 512)
    assert rec["fetch_bytes"] == 1001 * 2 * 1024
    assert rec["write_bytes"] == 8 * 1024
    assert rec["bytes_per_launch"] == 1001 * 2 * 1024 + 8 * 1024
    assert bench.load_traffic("abc", "wl", "mode") == rec["bytes_per_launch"]
    assert bench.load_traffic("other-hash", "wl", "mode") is None   # stale: kernel changed
    assert json.load(open(tmp_path / "traffic.json"))["wl/mode"]["kernel_hash"] == "abc"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
