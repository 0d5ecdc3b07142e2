"""pa_decode_split_noalloc against the allocating split path.

The entry point runs pa_decode_split and pa_reduce_lse with the partition
workspace in the library's own device array.  Through the C ABI it must give
exactly what pa_decode_split + pa_reduce_lse give with a caller-allocated
workspace (the same kernels on the same data, so bit for bit), on two calls in
a row, the second with a smaller input (the array keeps the first call's
contents), and both must be within the oracle's tolerance (bf16 KV: max abs
<= 1e-2, mean <= 1e-3; E4M3: max <= 2e-2; f32: max <= 1e-4).
"""
from __future__ import annotations

import numpy as np
import pytest

import paged_kv_cache_267_amd as pa
from paged_kv_cache_267_amd import workloads as W
from tests.helpers import err_stats, oracle_caches, oracle_decode

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-3), "fp8_e4m3": (2e-2, 2e-3), "f32": (1e-4, 1e-5)}


def _same_bits(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _check_pair(wl, psize):
    import torch
    from paged_kv_cache_267_amd.harness import DeviceWorkload
    print(f"[gpu-case] noalloc {wl.kv_dtype} S{wl.num_seqs} Hq{wl.num_q_heads} "
          f"Hkv{wl.num_kv_heads} D{wl.head_dim} bs{wl.block_size} W{wl.sliding_window} "
          f"P{psize}", flush=True)
    dw = DeviceWorkload(wl, partition_size=psize)
    dw.fill_history()
    dw.append_new()
    # the allocating path: caller-owned workspace, split then merge
    dw.decode_split()
    dw.reduce()
    ref_dev = dw.out.clone()
    dw.out.fill_(7.0)
    pa.pa_decode_split_noalloc(dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                               dw.seq_lens, block_size=wl.block_size, scale=wl.scale,
                               out=dw.out, num_kv_heads=wl.num_kv_heads, partition_size=psize,
                               sliding_window=wl.sliding_window, k_scale=wl.k_scale,
                               v_scale=wl.v_scale)
    torch.cuda.synchronize()
    assert _same_bits(dw.out, ref_dev), "noalloc output differs from split + reduce"
    kc, vc = oracle_caches(wl)
    ref = oracle_decode(wl, kc, vc)
    got = dw.out_f64()
    mx, mean = err_stats(got, ref)
    tmax, tmean = TOL[wl.kv_dtype]
    print(f"    noalloc vs oracle: max abs {mx:.3e} mean abs {mean:.3e}", flush=True)
    assert np.isfinite(got).all() and mx <= tmax and mean <= tmean, (mx, mean)


@pytest.mark.parametrize("kvdt", ["bf16", "fp8_e4m3", "f32"])
def test_noalloc_two_calls_second_smaller(kvdt):
    qdt = "f32" if kvdt == "f32" else "bf16"
    G = 1 if kvdt == "f32" else 8
    big = W.random_case(9100, seq_lens=[0, 5, 700, 3000, 33, 1500, 64, 2049], num_q_heads=2 * G,
                        num_kv_heads=2, head_dim=128, block_size=16, q_dtype=qdt,
                        kv_dtype=kvdt, sliding_window=2500)
    small = W.random_case(9101, seq_lens=[17, 1, 300], num_q_heads=G, num_kv_heads=1,
                          head_dim=64, block_size=32, q_dtype=qdt, kv_dtype=kvdt)
    _check_pair(big, 256)
    _check_pair(small, 64)


def test_noalloc_long_context_workload():
    """The long-context mixed batch (two 65536-token sequences, split 512): its
    67.6 MB workspace is the largest of the named workloads."""
    wl = W.config(3)
    assert pa.pa_decode_split_workspace_bytes(16, 64, 128, 128) <= pa.NOALLOC_SCRATCH_BYTES
    import torch
    from paged_kv_cache_267_amd.harness import DeviceWorkload
    print("[gpu-case] noalloc long-context workload", flush=True)
    dw = DeviceWorkload(wl, partition_size=512)
    dw.fill_history()
    dw.append_new()
    dw.decode_split()
    dw.reduce()
    ref_dev = dw.out.clone()
    dw.out.zero_()
    pa.pa_decode_split_noalloc(dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                               dw.seq_lens, block_size=wl.block_size, scale=wl.scale,
                               out=dw.out, num_kv_heads=wl.num_kv_heads, partition_size=512)
    torch.cuda.synchronize()
    assert _same_bits(dw.out, ref_dev)
