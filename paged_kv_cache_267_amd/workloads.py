"""Seeded synthetic inputs for paged decode attention.

This module is the only code the HIP library's tests/bench and the CPU oracle
share.  It holds none of the attention arithmetic: it draws sequence lengths,
a physical-block permutation and N(0,1) values, and turns them into the bytes
both sides receive (query, the tokens to be cached with their slots, block
tables, lengths).  Each side fills its own cache from those tokens with its own
``reshape_and_cache``.

Element encodings use library casts only: ``torch`` round-to-nearest-even
casts to bfloat16 and to ``float8_e4m3fn`` (the OCP E4M3 format).

Block placement follows the block pool of "vLLM 0.5 deep dive: PagedAttention
architecture" (chenxutan.com), section 2.1: a request of n tokens holds
ceil(n / block_size) physical blocks taken from a pool, and its block table
lists them in logical order.  Physical ids are dealt from a seeded random
permutation of the pool, so logically adjacent blocks are scattered, as in the
paging picture of "vLLM deployment and PagedAttention" (crazysre.cn), section
"Core concept".
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Every byte of a fresh cache holds this value: 0xFFFFFFFF (f32), 0xFFFF (bf16)
# and 0xFF (E4M3) are all NaN, so a read of an unwritten slot poisons the row.
POISON_BYTE = 0xFF

DTYPES = ("f32", "bf16", "fp8_e4m3")
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}
NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}
FP8_E4M3_MAX = 448.0


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a request of num_tokens tokens occupies (ceil division)."""
    return -(-int(num_tokens) // int(block_size))


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    seq_lens: np.ndarray        # int32 [S]: keys each query sees (after the append)
    block_tables: np.ndarray    # int32 [S, max_blocks_per_seq], -1 padding
    num_blocks: int
    query: np.ndarray           # [S, Hq, D] (extend: [num_tokens, Hq, D]): float32 or bf16 bits
    hist_key: np.ndarray        # [T, Hkv, D] raw elements of tokens already in the cache
    hist_value: np.ndarray
    hist_slots: np.ndarray      # int32 [T]
    new_key: np.ndarray         # [N, Hkv, D] tokens the decode step appends first
    new_value: np.ndarray
    new_slots: np.ndarray       # int32 [N]
    scale: float
    sliding_window: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0
    partition_size: int = 512
    description: str = ""
    # extend workloads: int32 [S + 1]; sequence s owns query rows
    # query_start_loc[s] .. query_start_loc[s+1]-1 (None: decode, one row each)
    query_start_loc: np.ndarray | None = None

    @property
    def q_lens(self) -> np.ndarray:
        if self.query_start_loc is None:
            return np.ones(self.num_seqs, dtype=np.int64)
        return np.diff(self.query_start_loc.astype(np.int64))

    @property
    def num_tokens(self) -> int:
        return int(self.query.shape[0])

    @property
    def max_query_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_partitions(self) -> int:
        return max(1, -(-self.max_blocks_per_seq * self.block_size // self.partition_size))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def effective_lens(self) -> np.ndarray:
        """Keys per query after the window: min(L, W) (W = 0: L)."""
        L = self.seq_lens.astype(np.int64)
        if self.sliding_window > 0:
            return np.minimum(L, self.sliding_window)
        return L

    def key_span(self) -> np.ndarray:
        """Keys the sequence's query tokens see together: from the first
        token's window start to L (decode: effective_lens)."""
        L = self.seq_lens.astype(np.int64)
        if self.sliding_window <= 0:
            return L
        first = L - self.q_lens        # position of the first query token
        return L - np.maximum(0, first + 1 - self.sliding_window)

    def attended_pairs(self) -> int:
        """(query token, key) pairs of one KV head's query group, summed over
        sequences: sum over tokens of the keys each one attends to."""
        total = 0
        W = self.sliding_window
        for L, n in zip(self.seq_lens.astype(np.int64), self.q_lens):
            pos = np.arange(L - n, L, dtype=np.int64)
            keys = pos + 1
            if W > 0:
                keys = np.minimum(keys, W)
            total += int(np.maximum(keys, 0).sum())
        return total

    def kv_bytes(self) -> int:
        """K + V bytes one call must read: in-window tokens only."""
        return int(self.key_span().sum()) * self.num_kv_heads * self.head_dim * 2 * \
            ELEM_BYTES[self.kv_dtype]

    def unique_kv_bytes(self) -> int:
        """Distinct K + V bytes read (shared-prefix blocks counted once)."""
        seen = set()
        total = 0
        for s in range(self.num_seqs):
            L = int(self.seq_lens[s])
            lo = L - int(self.key_span()[s])
            for j in range(lo, L):
                key = (int(self.block_tables[s, j // self.block_size]), j % self.block_size)
                if key not in seen:
                    seen.add(key)
                    total += 1
        return total * self.num_kv_heads * self.head_dim * 2 * ELEM_BYTES[self.kv_dtype]


# ---------------------------------------------------------------------------
# encodings (library casts)

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_fp8_codes(x: np.ndarray, scale: float) -> np.ndarray:
    import torch
    y = np.ascontiguousarray(x, dtype=np.float32) / np.float32(scale)
    t = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _encode(x: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "fp8_e4m3":
        return to_fp8_codes(x, scale)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# the generic builder

def build(name: str, rng: np.random.Generator, seq_lens, *, num_q_heads: int,
          num_kv_heads: int, head_dim: int, block_size: int, q_dtype: str, kv_dtype: str,
          sliding_window: int = 0, shared_prefix: int = 0, pool_factor: float = 1.25,
          num_blocks: int | None = None, partition_size: int = 512,
          poison_out_of_window: bool = False, zero_query: bool = False,
          description: str = "", q_lens=None) -> Workload:
    """Draw one workload.  Draw order: (1) lengths are given, (2) the pool
    permutation, (3) Q, (4) K of every distinct token, (5) V likewise.

    Distinct tokens are ordered: the shared prefix (if any), then for each
    sequence its private tokens in position order.  The last q_lens[s] tokens
    of sequence s (decode: q_lens = None, the last token, position L-1) are
    the step's new tokens, one query row each: they are not in the history
    and are written by the step's own cache append.
    """
    L = np.asarray(seq_lens, dtype=np.int64)
    extend = q_lens is not None
    # decode: one query row per sequence, whose token (if L > 0) is new
    n_new = np.asarray(q_lens, dtype=np.int64) if extend else np.minimum(L, 1)
    if extend:
        assert n_new.shape == L.shape and (n_new >= 1).all() and (n_new <= L).all(), \
            "every sequence brings 1..L new tokens"
    if shared_prefix:
        assert (L - n_new >= shared_prefix).all(), "new tokens lie after the shared prefix"
    S = int(L.shape[0])
    bs = int(block_size)
    D = int(head_dim)
    Hkv = int(num_kv_heads)
    if shared_prefix:
        assert shared_prefix % bs == 0, "a shared prefix must fill whole blocks"
        assert (L > shared_prefix).all(), "every sequence must extend the shared prefix"
    pfx_blocks = shared_prefix // bs
    private_blocks = [blocks_needed(int(n) - shared_prefix, bs) for n in L]
    needed = pfx_blocks + sum(private_blocks)
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * needed)), needed + 1)
    assert num_blocks > needed, "the pool keeps at least one unassigned (poisoned) block"
    perm = rng.permutation(num_blocks).astype(np.int32)

    max_blocks = max(1, max(blocks_needed(int(n), bs) for n in L)) if S else 1
    tables = np.full((S, max_blocks), -1, dtype=np.int32)
    cursor = 0
    pfx_ids = perm[cursor:cursor + pfx_blocks]
    cursor += pfx_blocks
    for s in range(S):
        tables[s, :pfx_blocks] = pfx_ids
        nb = private_blocks[s]
        tables[s, pfx_blocks:pfx_blocks + nb] = perm[cursor:cursor + nb]
        cursor += nb
    spare_block = int(perm[-1])                       # never dealt out

    # distinct tokens: (sequence, position) in draw order
    tok_seq, tok_pos = [], []
    if shared_prefix:
        tok_seq.append(np.zeros(shared_prefix, dtype=np.int64))
        tok_pos.append(np.arange(shared_prefix, dtype=np.int64))
    for s in range(S):
        n = int(L[s])
        tok_seq.append(np.full(n - shared_prefix, s, dtype=np.int64))
        tok_pos.append(np.arange(shared_prefix, n, dtype=np.int64))
    tok_seq = np.concatenate(tok_seq) if tok_seq else np.zeros(0, np.int64)
    tok_pos = np.concatenate(tok_pos) if tok_pos else np.zeros(0, np.int64)
    T = int(tok_seq.shape[0])
    slots = (tables[tok_seq, tok_pos // bs].astype(np.int64) * bs + tok_pos % bs).astype(np.int32)
    is_new = tok_pos >= (L[tok_seq] - n_new[tok_seq])

    q = rng.standard_normal((int(n_new.sum()) if extend else S, num_q_heads, D),
                            dtype=np.float32)
    if zero_query:
        q[:] = 0.0
    kf = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    vf = rng.standard_normal((T, Hkv, D), dtype=np.float32)

    k_scale = v_scale = 1.0
    if kv_dtype == "fp8_e4m3":
        k_scale = float(np.float32(np.abs(kf).max() / FP8_E4M3_MAX)) if T else 1.0
        v_scale = float(np.float32(np.abs(vf).max() / FP8_E4M3_MAX)) if T else 1.0
    kq = _encode(kf, kv_dtype, k_scale)
    del kf
    vq = _encode(vf, kv_dtype, v_scale)
    del vf

    if poison_out_of_window and sliding_window > 0:
        for s in range(S):
            # blocks wholly before the window of the first query token
            lo = max(0, int(L[s] - n_new[s]) + 1 - sliding_window)
            tables[s, :lo // bs] = spare_block

    return Workload(
        name=name, num_seqs=S, num_q_heads=num_q_heads, num_kv_heads=Hkv, head_dim=D,
        block_size=bs, q_dtype=q_dtype, kv_dtype=kv_dtype,
        seq_lens=L.astype(np.int32), block_tables=tables, num_blocks=int(num_blocks),
        query=_encode(q, q_dtype),
        hist_key=np.ascontiguousarray(kq[~is_new]), hist_value=np.ascontiguousarray(vq[~is_new]),
        hist_slots=np.ascontiguousarray(slots[~is_new]),
        new_key=np.ascontiguousarray(kq[is_new]), new_value=np.ascontiguousarray(vq[is_new]),
        new_slots=np.ascontiguousarray(slots[is_new]),
        scale=float(np.float32(1.0 / math.sqrt(D))), sliding_window=int(sliding_window),
        k_scale=k_scale, v_scale=v_scale, partition_size=int(partition_size),
        description=description,
        query_start_loc=(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
                         if extend else None))


# ---------------------------------------------------------------------------
# the five named configurations

SEED_BASE = 26700

CONFIG_NAMES = {
    1: "tiny_f32",
    2: "llama3_8b_layer_bf16",
    3: "long_context_mixed_bf16",
    4: "shared_prefix_bf16",
    5: "fp8_kv_sliding_window",
}


def config(cfg: int, **overrides) -> Workload:
    """The five decode workloads, drawn from seed 26700 + cfg."""
    rng = np.random.default_rng(SEED_BASE + cfg)
    if cfg == 1:
        return build(CONFIG_NAMES[1], rng, [1, 17, 33, 100], num_q_heads=4, num_kv_heads=4,
                     head_dim=64, block_size=16, q_dtype="f32", kv_dtype="f32", num_blocks=64,
                     partition_size=32,
                     description="4 seqs, lens {1,17,33,100}, 4/4 heads, D 64, bs 16, "
                                 "64-block pool, f32", **overrides)
    if cfg == 2:
        lens = rng.integers(512, 4096, size=64, endpoint=True)
        return build(CONFIG_NAMES[2], rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     block_size=16, q_dtype="bf16", kv_dtype="bf16",
                     description="batch 64, 32/8 heads, D 128, bs 16, bf16, "
                                 "lens U[512,4096], pool 1.25x", **overrides)
    if cfg == 3:
        short = rng.integers(256, 2048, size=14, endpoint=True)
        lens = rng.permutation(np.concatenate([[65536, 65536], short]))
        return build(CONFIG_NAMES[3], rng, lens, num_q_heads=64, num_kv_heads=8, head_dim=128,
                     block_size=32, q_dtype="bf16", kv_dtype="bf16", partition_size=512,
                     description="16 seqs (2 x 65536 + 14 x U[256,2048]), 64/8 heads, D 128, "
                                 "bs 32, bf16, split 512 + LSE reduce", **overrides)
    if cfg == 4:
        suffix = rng.integers(16, 512, size=128, endpoint=True)
        lens = 2048 + suffix + 1
        return build(CONFIG_NAMES[4], rng, lens, num_q_heads=64, num_kv_heads=8, head_dim=128,
                     block_size=16, q_dtype="bf16", kv_dtype="bf16", shared_prefix=2048,
                     description="128 seqs sharing a 2048-token prefix + U[16,512] suffix + 1 "
                                 "appended token, 64/8 heads, D 128, bs 16, bf16", **overrides)
    if cfg == 5:
        lens = np.clip(np.rint(rng.lognormal(mean=math.log(1500.0), sigma=1.0, size=256)),
                       1, 32768).astype(np.int64)
        return build(CONFIG_NAMES[5], rng, lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     block_size=16, q_dtype="bf16", kv_dtype="fp8_e4m3", sliding_window=4096,
                     description="batch 256, lens lognormal(median 1500, sigma 1) capped 32768, "
                                 "32/8 heads, D 128, bs 16, fp8 e4m3 KV (per-tensor scales), "
                                 "bf16 Q, window 4096", **overrides)
    raise ValueError(f"no config {cfg}")


def random_case(seed: int, *, seq_lens, num_q_heads=4, num_kv_heads=1, head_dim=128,
                block_size=16, q_dtype="bf16", kv_dtype="bf16", sliding_window=0,
                partition_size=64, shared_prefix=0, poison_out_of_window=False,
                zero_query=False, q_lens=None) -> Workload:
    """A small case for parity sweeps (lengths given, everything else drawn)."""
    rng = np.random.default_rng(seed)
    return build(f"random_{seed}", rng, seq_lens, num_q_heads=num_q_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                 q_dtype=q_dtype, kv_dtype=kv_dtype, sliding_window=sliding_window,
                 partition_size=partition_size, shared_prefix=shared_prefix,
                 poison_out_of_window=poison_out_of_window, zero_query=zero_query,
                 q_lens=q_lens)


# ---------------------------------------------------------------------------
# multi-token (extend) workloads: each sequence appends a chunk of new tokens
# after its cached ones and attends causally over both.  Prefix caching
# ("vLLM 0.5 deep dive: PagedAttention architecture", chenxutan.com, s4.4:
# requests share a cached system prompt and compute only what follows it)
# and chunked prefill (same page, s5.2: long prompts enter in chunks, with a
# budget of 8192 batched tokens per step) both run this operation.

EXTEND_SEED_BASE = 26800

EXTEND_NAMES = ("chunked_prefill_bf16", "prefix_extend_bf16", "extend_fp8_window")


def extend_config(name: str, **overrides) -> Workload:
    """The named extend workloads, drawn from seed 26800 + their index."""
    rng = np.random.default_rng(EXTEND_SEED_BASE + EXTEND_NAMES.index(name))
    if name == "chunked_prefill_bf16":
        prior = rng.integers(0, 3072, size=8, endpoint=True)
        chunk = np.full(8, 1024)
        return build(name, rng, prior + chunk, q_lens=chunk, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                     description="8 seqs x 1024-token chunks (8192 batched tokens) after "
                                 "U[0,3072] cached tokens, 32/8 heads, D 128, bs 16, bf16",
                     **overrides)
    if name == "prefix_extend_bf16":
        new = rng.integers(32, 256, size=32, endpoint=True)
        return build(name, rng, 2048 + new, q_lens=new, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                     shared_prefix=2048,
                     description="32 requests sharing a cached 2048-token prompt, each adding "
                                 "U[32,256] new tokens, 32/8 heads, D 128, bs 16, bf16",
                     **overrides)
    if name == "extend_fp8_window":
        prior = rng.integers(1024, 8192, size=16, endpoint=True)
        chunk = np.full(16, 256)
        return build(name, rng, prior + chunk, q_lens=chunk, num_q_heads=32, num_kv_heads=8,
                     head_dim=128, block_size=16, q_dtype="bf16", kv_dtype="fp8_e4m3",
                     sliding_window=4096,
                     description="16 seqs x 256-token chunks after U[1024,8192] cached tokens, "
                                 "32/8 heads, D 128, bs 16, fp8 e4m3 KV, window 4096",
                     **overrides)
    raise ValueError(f"no extend workload {name}")
