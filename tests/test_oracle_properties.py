"""Property-based pins of the CPU oracle over random small shapes.

Shapes are drawn with hypothesis (derandomized, so every run draws the same
examples): sequence lengths 1-300, GQA groups 1, 2, 4 and 8, block sizes 16
and 32, head_dim 64 and 128, f32 / bf16 / E4M3 caches, and windows off, 1 or
random.  For each draw the oracle, reading a paged cache written through the
documented layouts, must equal float64 torch SDPA on the dense tensors; and
relabelling the physical blocks must leave its output bit-identical.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tests.helpers import widen
from tests.test_oracle_pins import encode, paged_identity, sdpa_dense


@st.composite
def shapes(draw):
    kvdt = draw(st.sampled_from(["f32", "bf16", "fp8_e4m3"]))
    G = draw(st.sampled_from([1, 2, 4, 8]))
    Hkv = draw(st.integers(1, 2))
    D = draw(st.sampled_from([64, 128]))
    bs = draw(st.sampled_from([16, 32]))
    lens = draw(st.lists(st.integers(1, 300), min_size=1, max_size=4))
    window = draw(st.one_of(st.just(0), st.just(1), st.integers(2, 320)))
    seed = draw(st.integers(0, 2**31 - 1))
    return kvdt, G, Hkv, D, bs, lens, window, seed


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(shapes())
def test_oracle_equals_dense_sdpa_and_ignores_placement(shape):
    kvdt, G, Hkv, D, bs, lens, window, seed = shape
    qdt = "f32" if kvdt == "f32" else "bf16"
    Hq = G * Hkv
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    S, Lm = len(lens), int(lens.max())
    qf = rng.standard_normal((S, Hq, D), dtype=np.float32)
    kf = rng.standard_normal((S, Hkv, Lm, D), dtype=np.float32)
    vf = rng.standard_normal((S, Hkv, Lm, D), dtype=np.float32)
    ks = vs = 1.0
    if kvdt == "fp8_e4m3":
        ks = float(np.float32(np.abs(kf).max() / 448.0))
        vs = float(np.float32(np.abs(vf).max() / 448.0))
    q_raw, k_raw, v_raw = encode(qf, qdt), encode(kf, kvdt, ks), encode(vf, kvdt, vs)
    kc, vc, tables, NB = paged_identity(k_raw, v_raw, lens, bs, kvdt)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    kw = dict(block_size=bs, scale=scale, num_kv_heads=Hkv, q_dtype=qdt, kv_dtype=kvdt,
              sliding_window=window, k_scale=ks, v_scale=vs)
    got = oracle.decode(q_raw, kc, vc, tables, lens.astype(np.int32), **kw)
    ref = sdpa_dense(widen(q_raw, qdt), widen(k_raw, kvdt) * ks, widen(v_raw, kvdt) * vs,
                     lens, scale, window)
    np.testing.assert_allclose(got.reshape(S, Hq, D), ref, rtol=0, atol=1e-12)

    # the same cache with its physical blocks relabelled: bit-identical
    pi = rng.permutation(NB)
    per_block = kc.size // NB
    kc2 = np.empty_like(kc).reshape(NB, per_block)
    vc2 = np.empty_like(vc).reshape(NB, per_block)
    kc2[pi] = kc.reshape(NB, per_block)
    vc2[pi] = vc.reshape(NB, per_block)
    got2 = oracle.decode(q_raw, kc2.ravel(), vc2.ravel(), pi[tables].astype(np.int32),
                         lens.astype(np.int32), **kw)
    assert np.array_equal(got2, got)
