"""Device-side set-up of a seeded workload: upload, cache fill, decode step.

torch allocates device memory and provides the stream; every step of the path
(cache append, decode, partition merge) is a libpa.so call.
"""
from __future__ import annotations

import numpy as np

from . import (pa_decode, pa_decode_split, pa_extend, pa_reduce_lse, pa_reshape_and_cache)
from .workloads import POISON_BYTE, Workload


def _torch_dtype(dt: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[dt]


def _upload(arr: np.ndarray, dt: str, device):
    """Raw host elements (float32 / uint16 bf16 bits / uint8 codes) -> device tensor."""
    import torch
    a = np.ascontiguousarray(arr)
    if dt == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


class DeviceWorkload:
    """A Workload resident in HBM: query, poisoned caches filled by the library's
    own reshape_and_cache, block tables, lengths and the step's new tokens."""

    def __init__(self, wl: Workload, device="cuda", partition_size: int | None = None):
        import torch
        self.wl = wl
        self.device = torch.device(device)
        self.partition_size = partition_size if partition_size is not None else wl.partition_size
        d = self.device
        self.query = _upload(wl.query, wl.q_dtype, d)
        n = wl.num_blocks * wl.num_kv_heads * wl.head_dim * wl.block_size
        kvt = _torch_dtype(wl.kv_dtype)
        nbytes = n * torch.empty((), dtype=kvt).element_size()
        self.key_cache = torch.full((nbytes,), POISON_BYTE, dtype=torch.uint8, device=d).view(kvt)
        self.value_cache = torch.full((nbytes,), POISON_BYTE, dtype=torch.uint8,
                                      device=d).view(kvt)
        self.block_tables = torch.from_numpy(wl.block_tables).to(d)
        self.seq_lens = torch.from_numpy(wl.seq_lens).to(d)
        self.hist_key = _upload(wl.hist_key, wl.kv_dtype, d)
        self.hist_value = _upload(wl.hist_value, wl.kv_dtype, d)
        self.hist_slots = torch.from_numpy(wl.hist_slots).to(d)
        self.new_key = _upload(wl.new_key, wl.kv_dtype, d)
        self.new_value = _upload(wl.new_value, wl.kv_dtype, d)
        self.new_slots = torch.from_numpy(wl.new_slots).to(d)
        # outputs and partition workspace start as NaN: a row or partition the
        # kernels fail to write shows up in every comparison
        self.out = torch.full_like(self.query, float("nan"))
        P = wl.max_blocks_per_seq * wl.block_size
        self.max_parts = max(1, -(-P // self.partition_size))
        S, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
        self.part_out = torch.full((S, Hq, self.max_parts, D), float("nan"), dtype=torch.float32,
                                   device=d)
        self.part_lse = torch.full((S, Hq, self.max_parts), float("nan"), dtype=torch.float32,
                                   device=d)
        self.query_start_loc = (torch.from_numpy(wl.query_start_loc).to(d)
                                if wl.query_start_loc is not None else None)

    # -- steps ------------------------------------------------------------------
    def fill_history(self):
        pa_reshape_and_cache(self.hist_key, self.hist_value, self.key_cache, self.value_cache,
                             self.hist_slots, block_size=self.wl.block_size)

    def append_new(self, stream=None):
        pa_reshape_and_cache(self.new_key, self.new_value, self.key_cache, self.value_cache,
                             self.new_slots, block_size=self.wl.block_size, stream=stream)

    def _kw(self):
        wl = self.wl
        return dict(block_size=wl.block_size, scale=wl.scale, num_kv_heads=wl.num_kv_heads,
                    sliding_window=wl.sliding_window, k_scale=wl.k_scale, v_scale=wl.v_scale)

    def decode_unsplit(self, stream=None):
        pa_decode(self.query, self.key_cache, self.value_cache, self.block_tables, self.seq_lens,
                  out=self.out, stream=stream, **self._kw())
        return self.out

    def decode_split(self, stream=None):
        pa_decode_split(self.query, self.key_cache, self.value_cache, self.block_tables,
                        self.seq_lens, partition_size=self.partition_size,
                        max_num_partitions=self.max_parts, part_out=self.part_out,
                        part_lse=self.part_lse, stream=stream, **self._kw())
        return self.part_out, self.part_lse

    def reduce(self, stream=None):
        pa_reduce_lse(self.part_out, self.part_lse, self.seq_lens,
                      partition_size=self.partition_size,
                      sliding_window=self.wl.sliding_window, out=self.out, stream=stream)
        return self.out

    def extend(self, stream=None):
        """Multi-token attention of every sequence's new chunk (extend workloads)."""
        pa_extend(self.query, self.key_cache, self.value_cache, self.block_tables,
                  self.seq_lens, self.query_start_loc, out=self.out,
                  max_query_len=self.wl.max_query_len, stream=stream, **self._kw())
        return self.out

    def step_extend(self, stream=None):
        """One extend step: append the chunks' K/V, then attend."""
        self.append_new(stream)
        return self.extend(stream)

    def step(self, split: bool = True, stream=None):
        """One decode step: append the new tokens, attend, merge partitions."""
        self.append_new(stream)
        if split:
            self.decode_split(stream)
            return self.reduce(stream)
        return self.decode_unsplit(stream)

    # -- host copies --------------------------------------------------------------
    def out_f64(self) -> np.ndarray:
        import torch
        return self.out.to(torch.float64).cpu().numpy().reshape(-1, self.wl.head_dim)

    def cache_bytes(self):
        import torch
        return (self.key_cache.view(torch.uint8).cpu().numpy(),
                self.value_cache.view(torch.uint8).cpu().numpy())
