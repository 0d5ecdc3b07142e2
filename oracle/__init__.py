"""CPU oracle for paged decode attention: numpy front end of pa_oracle.c.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``paged_kv_cache_267_amd``) and imports nothing
from it; both are fed the same bytes by the seeded input generator.

All arithmetic lives in ``pa_oracle.c`` (fp64, plain definitions; the header
of that file cites the passages of the pages each function follows).  This
module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# oracle dtype codes (private to the oracle)
_DT = {"f32": 0, "bf16": 1, "fp8_e4m3": 2}
_NP = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}

_lib = None


def build() -> str:
    """Compile pa_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-D_DEFAULT_SOURCE",
           "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.ora_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.ora_fp8_e4m3_value.restype = D
    lib.ora_fp8_e4m3_encode.argtypes = [D]
    lib.ora_fp8_e4m3_encode.restype = ctypes.c_uint8
    lib.ora_bf16_value.argtypes = [ctypes.c_uint16]
    lib.ora_bf16_value.restype = D
    lib.ora_num_threads.argtypes = []
    lib.ora_num_threads.restype = I
    lib.ora_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
    lib.ora_reshape_and_cache_fp8.argtypes = [P, P, I, P, P, P, I, I, I, I, I, F, F]
    lib.ora_reshape_and_cache.restype = I
    lib.ora_decode.argtypes = [P, P, P, P, P, I, F, I, I, I, I, I, I, I, I, F, F, P, I, P]
    lib.ora_decode.restype = None
    lib.ora_decode_split.argtypes = [P, P, P, P, P, I, F, I, I, I, I, I, I, I, I, F, F, I, I, P,
                                     I, P, P]
    lib.ora_decode_split.restype = None
    lib.ora_reduce_lse.argtypes = [P, P, I, I, I, P]
    lib.ora_reduce_lse.restype = None
    lib.ora_extend.argtypes = [P, P, P, P, P, P, I, F, I, I, I, I, I, I, I, I, F, F, P, I, P]
    lib.ora_extend.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().ora_num_threads())


def fp8_e4m3_value(codes) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8) as float64."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.ora_fp8_e4m3_value(int(c)) for c in codes.ravel()],
                    dtype=np.float64).reshape(codes.shape)


def fp8_e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code (ties to even, saturating at 448, NaN -> 0x7F)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.ora_fp8_e4m3_encode(float(v)) for v in x.ravel()],
                    dtype=np.uint8).reshape(x.shape)


def bf16_value(bits) -> np.ndarray:
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.ora_bf16_value(int(b)) for b in bits.ravel()],
                    dtype=np.float64).reshape(bits.shape)


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, *, num_kv_heads,
                      head_dim, block_size, num_blocks, kv_dtype) -> None:
    """In place: write each token's K/V into its slot (bit copy)."""
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    assert key.dtype == _NP[kv_dtype] and value.dtype == _NP[kv_dtype]
    assert key_cache.dtype == _NP[kv_dtype] and value_cache.dtype == _NP[kv_dtype]
    rc = _load().ora_reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(slots), int(slots.shape[0]), num_kv_heads, head_dim,
                                       block_size, num_blocks, _DT[kv_dtype])
    if rc != 0:
        raise ValueError("slot outside the block pool")


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, *, src_dtype,
                          num_kv_heads, head_dim, block_size, num_blocks, k_scale,
                          v_scale) -> None:
    """In place: quantise each token's K/V (f32 or bf16 bits) to E4M3 codes
    of x / scale and write them into its slot of the E4M3 caches."""
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    assert key.dtype == _NP[src_dtype] and value.dtype == _NP[src_dtype]
    assert key_cache.dtype == np.uint8 and value_cache.dtype == np.uint8
    rc = _load().ora_reshape_and_cache_fp8(_ptr(key), _ptr(value), _DT[src_dtype],
                                           _ptr(key_cache), _ptr(value_cache), _ptr(slots),
                                           int(slots.shape[0]), num_kv_heads, head_dim,
                                           block_size, num_blocks, float(k_scale),
                                           float(v_scale))
    if rc != 0:
        raise ValueError("slot outside the block pool")


def _rows(rows, S, Hq):
    if rows is None:
        rows = np.arange(S * Hq, dtype=np.int32)
    return np.ascontiguousarray(rows, dtype=np.int32)


def _common(query, q_dtype, key_cache, value_cache, kv_dtype, block_tables, seq_lens):
    query = np.ascontiguousarray(query)
    assert query.dtype == _NP[q_dtype] and query.ndim == 3
    assert key_cache.dtype == _NP[kv_dtype] and value_cache.dtype == _NP[kv_dtype]
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    return query, bt, sl


def decode(query, key_cache, value_cache, block_tables, seq_lens, *, block_size, scale,
           num_kv_heads, q_dtype, kv_dtype, sliding_window=0, k_scale=1.0, v_scale=1.0,
           rows=None) -> np.ndarray:
    """Decode attention for rows (s * num_q_heads + h); returns float64 [nrows, D]."""
    query, bt, sl = _common(query, q_dtype, key_cache, value_cache, kv_dtype, block_tables,
                            seq_lens)
    S, Hq, D = query.shape
    rows = _rows(rows, S, Hq)
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    _load().ora_decode(_ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(sl),
                       block_size, float(scale), S, Hq, num_kv_heads, D, bt.shape[1],
                       int(sliding_window), _DT[q_dtype], _DT[kv_dtype], float(k_scale),
                       float(v_scale), _ptr(rows), int(rows.shape[0]), _ptr(out))
    return out


def decode_split(query, key_cache, value_cache, block_tables, seq_lens, *, block_size, scale,
                 num_kv_heads, q_dtype, kv_dtype, partition_size, max_partitions,
                 sliding_window=0, k_scale=1.0, v_scale=1.0, rows=None):
    """Per-partition outputs [nrows, P, D] and natural-log LSEs [nrows, P] (float64)."""
    query, bt, sl = _common(query, q_dtype, key_cache, value_cache, kv_dtype, block_tables,
                            seq_lens)
    S, Hq, D = query.shape
    rows = _rows(rows, S, Hq)
    po = np.zeros((rows.shape[0], max_partitions, D), dtype=np.float64)
    pl = np.zeros((rows.shape[0], max_partitions), dtype=np.float64)
    _load().ora_decode_split(_ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(sl),
                             block_size, float(scale), S, Hq, num_kv_heads, D, bt.shape[1],
                             int(sliding_window), _DT[q_dtype], _DT[kv_dtype], float(k_scale),
                             float(v_scale), int(partition_size), int(max_partitions),
                             _ptr(rows), int(rows.shape[0]), _ptr(po), _ptr(pl))
    return po, pl


def extend(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, *,
           block_size, scale, num_kv_heads, q_dtype, kv_dtype, sliding_window=0, k_scale=1.0,
           v_scale=1.0, rows=None) -> np.ndarray:
    """Multi-token attention for rows (qrow * num_q_heads + h) of the query
    array [num_tokens, num_q_heads, D]; sequence s owns query rows
    query_start_loc[s] .. query_start_loc[s+1]-1.  float64 [nrows, D]."""
    query, bt, sl = _common(query, q_dtype, key_cache, value_cache, kv_dtype, block_tables,
                            seq_lens)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    T, Hq, D = query.shape
    S = sl.shape[0]
    assert qsl.shape == (S + 1,) and qsl[0] == 0 and qsl[-1] == T and np.all(np.diff(qsl) >= 0)
    rows = _rows(rows, T, Hq)
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    _load().ora_extend(_ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(bt), _ptr(sl),
                       _ptr(qsl), block_size, float(scale), S, Hq, num_kv_heads, D, bt.shape[1],
                       int(sliding_window), _DT[q_dtype], _DT[kv_dtype], float(k_scale),
                       float(v_scale), _ptr(rows), int(rows.shape[0]), _ptr(out))
    return out


def reduce_lse(part_out, part_lse) -> np.ndarray:
    """Merge per-partition results by their LSE weights; float64 [nrows, D]."""
    po = np.ascontiguousarray(part_out, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    n, P, D = po.shape
    out = np.zeros((n, D), dtype=np.float64)
    _load().ora_reduce_lse(_ptr(po), _ptr(pl), n, D, P, _ptr(out))
    return out
