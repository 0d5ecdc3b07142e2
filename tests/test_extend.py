"""Multi-token (extend) paged attention: oracle pins and GPU parity.

Each sequence brings a chunk of new query tokens, the last ones of its keys;
token i of a chunk of n sits at position p = L - n + i and attends causally to
keys up to p (within its own window).  Prefix caching ("vLLM 0.5 deep dive:
PagedAttention architecture", chenxutan.com, s4.4) and chunked prefill (same
page, s5.2) both reduce to this operation over the paged cache.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_267_amd import workloads as W
from tests.helpers import err_stats, half_ulp_bf16, oracle_caches, widen
from tests.test_oracle_pins import encode, paged_identity


def oracle_extend(wl, kc, vc, rows=None, **over):
    kw = dict(block_size=wl.block_size, scale=wl.scale, num_kv_heads=wl.num_kv_heads,
              q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype, sliding_window=wl.sliding_window,
              k_scale=wl.k_scale, v_scale=wl.v_scale, rows=rows)
    kw.update(over)
    return oracle.extend(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                         **kw)


# ---------------------------------------------------------------------------
# pins of the oracle (CPU)

def sdpa_causal(q64, k64, v64, lens, qsl, scale, window):
    """torch SDPA in float64 per sequence with an explicit mask: query i of a
    chunk of n sees key j iff j <= p and (window == 0 or j > p - window),
    p = L - n + i.  q64 [T, Hq, D]; k64, v64 [S, Hkv, Lmax, D]."""
    T, Hq, D = q64.shape
    S, Hkv, Lm, _ = k64.shape
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(S):
        a, b, L = int(qsl[s]), int(qsl[s + 1]), int(lens[s])
        n = b - a
        if n == 0:
            continue
        q = torch.from_numpy(q64[a:b]).permute(1, 0, 2)                  # [Hq, n, D]
        k = torch.from_numpy(k64[s]).repeat_interleave(G, dim=0)[:, :L]  # [Hq, L, D]
        v = torch.from_numpy(v64[s]).repeat_interleave(G, dim=0)[:, :L]
        p = torch.arange(L - n, L)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= p
        if window > 0:
            mask &= j > p - window
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                             scale=scale)
        out[a:b] = o.permute(1, 0, 2).numpy()
    return out


EXT_DENSE_CASES = [
    # (Hq, Hkv, D, bs, q_dtype, kv_dtype, window)
    (4, 2, 64, 16, "bf16", "bf16", 0),
    (8, 2, 128, 32, "bf16", "bf16", 0),
    (4, 4, 128, 16, "bf16", "fp8_e4m3", 0),
    (8, 1, 64, 64, "bf16", "bf16", 21),
    (4, 2, 128, 16, "bf16", "bf16", 40),
    (16, 1, 64, 32, "bf16", "fp8_e4m3", 33),
]


@pytest.mark.parametrize("case", EXT_DENSE_CASES)
def test_extend_identity_layout_matches_causal_sdpa(case):
    Hq, Hkv, D, bs, qdt, kvdt, window = case
    rng = np.random.default_rng(4321 + D + bs + Hq + window)
    lens = np.array([1, 9, 40, bs + 3, 70, 5], dtype=np.int64)
    qlen = np.array([1, 9, 17, 1, 33, 2], dtype=np.int64)    # 9 = L: no cached keys before
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    S, Lm, T = len(lens), int(lens.max()), int(qlen.sum())
    qf = rng.standard_normal((T, Hq, D), dtype=np.float32)
    kf = rng.standard_normal((S, Hkv, Lm, D), dtype=np.float32)
    vf = rng.standard_normal((S, Hkv, Lm, D), dtype=np.float32)
    ks = vs = 1.0
    if kvdt == "fp8_e4m3":
        ks = float(np.float32(np.abs(kf).max() / 448.0))
        vs = float(np.float32(np.abs(vf).max() / 448.0))
    q_raw, k_raw, v_raw = encode(qf, qdt), encode(kf, kvdt, ks), encode(vf, kvdt, vs)
    kc, vc, tables, _ = paged_identity(k_raw, v_raw, lens, bs, kvdt)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = oracle.extend(q_raw, kc, vc, tables, lens.astype(np.int32), qsl, block_size=bs,
                        scale=scale, num_kv_heads=Hkv, q_dtype=qdt, kv_dtype=kvdt,
                        sliding_window=window, k_scale=ks, v_scale=vs)
    ref = sdpa_causal(widen(q_raw, qdt), widen(k_raw, kvdt) * ks, widen(v_raw, kvdt) * vs,
                      lens, qsl, scale, window)
    np.testing.assert_allclose(got.reshape(T, Hq, D), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 30])
def test_extend_with_one_token_is_decode(window):
    kw = dict(seq_lens=[1, 2, 17, 40, 100], num_q_heads=8, num_kv_heads=2, head_dim=64,
              block_size=16, q_dtype="bf16", kv_dtype="bf16", sliding_window=window)
    dec = W.random_case(91, **kw)
    ext = W.random_case(91, q_lens=[1] * 5, **kw)
    assert np.array_equal(dec.query, ext.query)          # the same draws
    kc, vc = oracle_caches(ext)
    got = oracle_extend(ext, kc, vc)
    ref = oracle.decode(dec.query, kc, vc, dec.block_tables, dec.seq_lens,
                        block_size=16, scale=dec.scale, num_kv_heads=2, q_dtype="bf16",
                        kv_dtype="bf16", sliding_window=window)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("window", [0, 19])
def test_extend_token_is_decode_of_the_cut_sequence(window):
    """Token i of a chunk equals one-query decode over the sequence cut after
    its position: its row, seq_len p + 1, the same block table."""
    wl = W.random_case(92, seq_lens=[30, 64, 7], q_lens=[12, 40, 7], num_q_heads=4,
                       num_kv_heads=2, head_dim=64, block_size=16, sliding_window=window)
    kc, vc = oracle_caches(wl)
    got = oracle_extend(wl, kc, vc).reshape(wl.num_tokens, wl.num_q_heads, -1)
    qsl = wl.query_start_loc
    for s in range(wl.num_seqs):
        L, n = int(wl.seq_lens[s]), int(qsl[s + 1] - qsl[s])
        for i in range(n):
            row = int(qsl[s]) + i
            ref = oracle.decode(wl.query[row:row + 1], kc, vc, wl.block_tables[s:s + 1],
                                np.array([L - n + i + 1], np.int32), block_size=16,
                                scale=wl.scale, num_kv_heads=2, q_dtype="bf16",
                                kv_dtype="bf16", sliding_window=window)
            assert np.array_equal(got[row], ref.reshape(wl.num_q_heads, -1)), (s, i)


def test_extend_token_before_position_zero_is_zero():
    """A chunk longer than the sequence: its first tokens have no position."""
    rng = np.random.default_rng(5)
    D, bs = 64, 16
    lens = np.array([3], np.int64)
    kf = rng.standard_normal((1, 1, 3, D), dtype=np.float32)
    k_raw, v_raw = encode(kf, "bf16"), encode(kf[..., ::-1].copy(), "bf16")
    kc, vc, tables, _ = paged_identity(k_raw, v_raw, lens, bs, "bf16")
    q = encode(rng.standard_normal((5, 2, D), dtype=np.float32), "bf16")
    out = oracle.extend(q, kc, vc, tables, lens.astype(np.int32), np.array([0, 5], np.int32),
                        block_size=bs, scale=0.125, num_kv_heads=1, q_dtype="bf16",
                        kv_dtype="bf16").reshape(5, 2, D)
    assert not out[:2].any()
    v = widen(v_raw, "bf16")[0, 0]
    np.testing.assert_allclose(out[2], np.broadcast_to(v[0], (2, D)), rtol=0, atol=0)
    assert np.abs(out[3:]).sum() > 0


def test_extend_workloads_shapes():
    for name in W.EXTEND_NAMES:
        wl = W.extend_config(name)
        qsl = wl.query_start_loc
        assert qsl[0] == 0 and qsl[-1] == wl.num_tokens
        assert wl.new_key.shape[0] == wl.num_tokens == wl.new_slots.shape[0]
        assert (wl.q_lens <= wl.seq_lens).all()
    wl = W.extend_config("chunked_prefill_bf16")
    assert wl.num_tokens == 8192 and wl.max_query_len == 1024


# ---------------------------------------------------------------------------
# GPU parity: the HIP kernel through the C ABI against the oracle

TOL = {"bf16": (1e-2, 1e-3), "fp8_e4m3": (2e-2, 2e-3)}


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _assert_close(got, ref, kv_dtype, what):
    """The bf16 output is within the tolerance of the fp64 oracle once its own
    rounding (half a bf16 ulp of the exact value) is set aside; mean as is."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = err_stats(got, ref)
    tmax, tmean = TOL[kv_dtype]
    excess = np.abs(got - ref) - half_ulp_bf16(ref)
    at = np.unravel_index(int(np.argmax(excess)), got.shape)
    mx_ex = float(max(excess.max(), 0.0))
    print(f"    {what}: max abs {mx:.3e}, beyond bf16 rounding {mx_ex:.3e} (row {at[0]}, "
          f"dim {at[1]}, ref {ref[at]:.4f}), mean abs {mean:.3e}", flush=True)
    assert mx_ex <= tmax and mean <= tmean, f"{what}: max {mx_ex:.3e} mean {mean:.3e}"


def _gpu_extend(wl):
    from paged_kv_cache_267_amd.harness import DeviceWorkload
    dw = DeviceWorkload(wl)
    dw.fill_history()
    dw.step_extend()
    torch.cuda.synchronize()
    return dw


# lens / chunk lengths: a chunk that is the whole sequence, single tokens, a
# chunk spanning several column blocks, chunks not a multiple of 16, and long
# cached histories (several 32-key steps before the chunk)
SMALL_LENS = [40, 1, 70, 300, 129, 33]
SMALL_QLENS = [40, 1, 45, 100, 3, 17]


@pytest.mark.gpu
@pytest.mark.parametrize("kvdt", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64])
@pytest.mark.parametrize("G", [1, 4, 16])
@pytest.mark.parametrize("window", [0, 50])
def test_extend_small_parity(kvdt, D, bs, G, window):
    Hkv = 2 if G < 16 else 1
    _announce(f"extend small kv={kvdt} D={D} bs={bs} G={G} W={window}")
    wl = W.random_case(700 + D + bs + G + window, seq_lens=SMALL_LENS, q_lens=SMALL_QLENS,
                       num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                       kv_dtype=kvdt, sliding_window=window, poison_out_of_window=window > 0)
    kc, vc = oracle_caches(wl)
    ref = oracle_extend(wl, kc, vc)
    dw = _gpu_extend(wl)
    _assert_close(dw.out_f64(), ref, kvdt, f"extend kv={kvdt} D={D} bs={bs} G={G} W={window}")


def extend_sweep_cases(n, seed=4242):
    """Seeded random extend shapes: cache dtype, G 1..16, head_dim, block size,
    KV heads, 1-6 sequences whose cached part and chunk are drawn from edge
    values (block and 32-key step boundaries) or at random, and a window that
    is off, 1, random or wider than every sequence."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kvdt = ["bf16", "fp8_e4m3"][i % 2]
        G = [1, 2, 4, 8, 16][(i // 2) % 5]
        D = int(rng.choice([64, 128]))
        bs = int(rng.choice([16, 32, 64]))
        Hkv = int(rng.integers(1, 4)) if G < 16 else int(rng.integers(1, 3))
        S = int(rng.integers(1, 7))
        edge_c = [0, 1, bs - 1, bs, bs + 1, 31, 32, 33, 2 * bs + 3]
        edge_n = [1, 2, 15, 16, 17, 31, 32, 33, 64]
        cached = [int(rng.choice(edge_c)) if rng.random() < 0.4 else int(rng.integers(0, 400))
                  for _ in range(S)]
        chunk = [int(rng.choice(edge_n)) if rng.random() < 0.4 else int(rng.integers(1, 121))
                 for _ in range(S)]
        window = {0: 0, 1: 1, 2: int(rng.integers(2, 300)), 3: 100000}[(i // 10) % 4]
        cases.append(dict(i=i, kvdt=kvdt, G=G, D=D, bs=bs, Hkv=Hkv, window=window,
                          lens=[c + q for c, q in zip(cached, chunk)], q_lens=chunk,
                          seed=seed * 100 + i))
    return cases


def test_extend_sweep_cases_cover_the_grid():
    cases = extend_sweep_cases(40)
    assert {c["G"] for c in cases if c["window"] not in (0, 100000)} == {1, 2, 4, 8, 16}
    assert {(c["kvdt"], c["D"]) for c in cases} == {(k, d) for k in ("bf16", "fp8_e4m3")
                                                    for d in (64, 128)}
    assert {c["bs"] for c in cases} == {16, 32, 64}
    assert all(1 <= q <= L for c in cases for q, L in zip(c["q_lens"], c["lens"]))


@pytest.mark.gpu
def test_extend_random_shape_sweep():
    """40 seeded cases against the oracle; the first failing case stops the
    sweep and is named."""
    for c in extend_sweep_cases(40):
        what = (f"extend case {c['i']}: {c['kvdt']} D{c['D']} bs{c['bs']} G{c['G']} "
                f"Hkv{c['Hkv']} lens {c['lens']} chunks {c['q_lens']} W{c['window']}")
        _announce(what)
        wl = W.random_case(c["seed"], seq_lens=c["lens"], q_lens=c["q_lens"],
                           num_q_heads=c["G"] * c["Hkv"], num_kv_heads=c["Hkv"],
                           head_dim=c["D"], block_size=c["bs"], kv_dtype=c["kvdt"],
                           sliding_window=c["window"])
        kc, vc = oracle_caches(wl)
        ref = oracle_extend(wl, kc, vc)
        dw = _gpu_extend(wl)
        _assert_close(dw.out_f64(), ref, c["kvdt"], what)


@pytest.mark.gpu
@pytest.mark.parametrize("nseq,kvdt,window", [(64, "bf16", 0), (65, "bf16", 0),
                                              (64, "fp8_e4m3", 90), (65, "fp8_e4m3", 90)])
def test_extend_dealing_orders(nseq, kvdt, window):
    """Batches of up to 64 sequences are dealt by work (one lane per sequence
    ranks them); larger batches in sequence order.  64 and 65 sequences run
    both paths; equal (length, chunk) pairs make ties, broken by index."""
    rng = np.random.default_rng(900 + nseq)
    q = rng.integers(1, 40, size=nseq)
    lens = q + rng.integers(0, 260, size=nseq)
    lens[1::7], q[1::7] = lens[0], q[0]          # ties in work
    q[2::11] = 1                                 # one-token chunks
    _announce(f"extend dealing order: {nseq} sequences kv={kvdt} W={window}")
    wl = W.random_case(950 + nseq, seq_lens=lens.tolist(), q_lens=q.tolist(), num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, kv_dtype=kvdt,
                       sliding_window=window)
    kc, vc = oracle_caches(wl)
    ref = oracle_extend(wl, kc, vc)
    dw = _gpu_extend(wl)
    _assert_close(dw.out_f64(), ref, kvdt, f"extend {nseq} sequences kv={kvdt} W={window}")


def _sample_rows(wl, n, seed):
    total = wl.num_tokens * wl.num_q_heads
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    # every head of the first and last token of the longest sequence
    s = int(np.argmax(wl.seq_lens))
    for t in (int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1]) - 1):
        rows |= set(range(t * wl.num_q_heads, (t + 1) * wl.num_q_heads))
    return np.array(sorted(rows), dtype=np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("name", W.EXTEND_NAMES)
def test_extend_named_workload_parity(name):
    _announce(f"extend workload {name}: generating")
    wl = W.extend_config(name)
    rows = _sample_rows(wl, 2048, seed=3)
    kc, vc = oracle_caches(wl)
    _announce(f"extend workload {name}: oracle on {rows.size} rows")
    ref = oracle_extend(wl, kc, vc, rows=rows)
    _announce(f"extend workload {name}: gpu")
    dw = _gpu_extend(wl)
    _assert_close(dw.out_f64()[rows], ref, wl.kv_dtype, f"extend {name}")


@pytest.mark.gpu
@pytest.mark.parametrize("kvdt", ["bf16", "fp8_e4m3"])
def test_extend_blocks_past_4gib_of_cache(kvdt):
    """Chunks over blocks at the top of a pool whose caches span more than
    4 GiB (block b at N - 1 - b, NaN poison elsewhere), against the oracle of
    the original layout."""
    from paged_kv_cache_267_amd.harness import DeviceWorkload
    from tests.helpers import relocate_far
    wl = W.random_case(4444, seq_lens=[300, 2000, 129, 1500], q_lens=[300, 200, 17, 64],
                       num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       kv_dtype=kvdt, sliding_window=1000 if kvdt == "fp8_e4m3" else 0)
    _announce(f"extend pool past 4 GiB {kvdt}")
    kc, vc = oracle_caches(wl)
    ref = oracle_extend(wl, kc, vc)
    dw = DeviceWorkload(wl)
    dw.fill_history()
    dw.append_new()
    relocate_far(dw)
    assert dw.key_cache.numel() * dw.key_cache.element_size() > (1 << 32)
    dw.extend()
    torch.cuda.synchronize()
    _assert_close(dw.out_f64(), ref, kvdt, f"extend pool past 4 GiB {kvdt}")


@pytest.mark.gpu
@pytest.mark.parametrize("name", W.EXTEND_NAMES)
def test_extend_repeat_runs_bit_identical(name):
    """Each output column is computed by one wave in a fixed key order, so
    every run gives the same bits (the LDS ring's reuse is race-free)."""
    wl = W.extend_config(name)
    _announce(f"extend repeat runs {name}")
    dw = _gpu_extend(wl)
    first = dw.out.clone()
    for _ in range(6):
        dw.extend()
        torch.cuda.synchronize()
        assert torch.equal(dw.out.view(torch.int16), first.view(torch.int16))


@pytest.mark.gpu
def test_extend_window_poison_variant():
    _announce("extend fp8 window with out-of-window blocks pointing at a NaN block")
    wl = W.extend_config("extend_fp8_window", poison_out_of_window=True)
    rows = _sample_rows(wl, 1024, seed=4)
    kc, vc = oracle_caches(wl)
    ref = oracle_extend(wl, kc, vc, rows=rows)
    dw = _gpu_extend(wl)
    _assert_close(dw.out_f64()[rows], ref, wl.kv_dtype, "extend fp8 window poison")


@pytest.mark.gpu
def test_extend_edge_metadata():
    """Chunks longer than their sequence (tokens at negative positions get
    zero rows) and an empty chunk, checked against the oracle on the same
    (modified) metadata."""
    import paged_kv_cache_267_amd as pa
    _announce("extend edge metadata")
    wl = W.random_case(811, seq_lens=[50, 20, 64, 9], q_lens=[10, 20, 30, 9], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16)
    kc, vc = oracle_caches(wl)
    dw = _gpu_extend(wl)
    # sequence 1 keeps its rows but only 12 keys (8 tokens before position 0);
    # sequence 2's chunk becomes empty, its 30 rows going to sequence 3 (39 tokens, 9 keys)
    lens = np.array([50, 12, 64, 9], np.int32)
    qsl = np.array([0, 10, 30, 30, 69], np.int32)
    ref = oracle.extend(wl.query, kc, vc, wl.block_tables, lens, qsl, block_size=16,
                        scale=wl.scale, num_kv_heads=2, q_dtype="bf16", kv_dtype="bf16")
    out = torch.full_like(dw.out, float("nan"))
    pa.pa_extend(dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                 torch.from_numpy(lens).cuda(), torch.from_numpy(qsl).cuda(), block_size=16,
                 scale=wl.scale, out=out, num_kv_heads=2, max_query_len=39)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy().reshape(-1, 128)
    _assert_close(got, ref, "bf16", "edge metadata")
    zero_rows = ref.reshape(69, 8, 128)
    assert not zero_rows[10:18].any() and not zero_rows[30:60].any()
    assert not got.reshape(69, 8, 128)[10:18].any() and not got.reshape(69, 8, 128)[30:60].any()
    # nothing to do: no sequences, or no tokens
    pa.pa_extend(dw.query[:0], dw.key_cache, dw.value_cache, dw.block_tables,
                 torch.zeros(4, dtype=torch.int32, device="cuda"),
                 torch.zeros(5, dtype=torch.int32, device="cuda"), block_size=16,
                 scale=wl.scale, out=out, num_kv_heads=2, max_query_len=0)
    torch.cuda.synchronize()
