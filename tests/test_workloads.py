"""Intent checks of the seeded generators (CPU only).

The configurations describe concentrated attention (a few needles) and diffuse
topics; these checks confirm, through the oracle's indexer and top-p, that the
drawn inputs land in those regimes (the pages report a needle answered by a
couple of tokens and a diffuse topic needing thousands: techwalker article,
section 4; budgets three orders of magnitude apart: RTPurboV2 article, finding 4).
"""
import numpy as np
import pytest

import workloads as W
from oracle import rtp_oracle as O


def _sets(wl, b, kv_i, p, idx_rows=None):
    G = wl.G
    kv = wl.ret_kv_heads[kv_i]
    idx = idx_rows if idx_rows is not None else O.f64_to_bf16(
        O.bf16_to_f64(wl.k_pre[b, kv]) @ O.bf16_to_f64(wl.w_k[kv_i]))
    out = {}
    for g in range(G):
        h = kv * G + g
        s = O.scores(O.query_index(wl.q_pre[b, h], wl.w_q[kv_i * G + g]), idx)
        out[h] = (s, O.top_p_set(s, p))
    return out


def test_bf16_generation_is_deterministic_and_rne():
    a = W.make(1)
    b = W.make(1)
    assert np.array_equal(a.k_pre, b.k_pre) and np.array_equal(a.q_pre, b.q_pre)
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5], dtype=np.float32)
    assert W.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0xC020]


def test_tiny_needles_hold_the_mass():
    wl = W.make(1)
    res = _sets(wl, 0, 0, 0.9)
    for h, (s, tp) in res.items():
        mine = [p for p, o in zip(wl.meta["needles"], wl.meta["needle_owner"]) if o == h]
        w = np.exp(s.astype(np.float64) - s.max())
        assert w[mine].sum() / w.sum() >= 0.9
        assert set(mine) <= set(tp["set"].tolist())


def test_variable_budget_spans_orders_of_magnitude():
    wl = W.variable_budget_decode(B=1)
    needle, diffuse = [], []
    for kv_i in range(wl.n_ret):
        for h, (s, tp) in _sets(wl, 0, kv_i, 0.9).items():
            kind = wl.meta["kinds"][(0, h)][0]
            (needle if kind == "needle" else diffuse).append(len(tp["set"]))
    assert max(needle) <= 10
    assert min(diffuse) >= 1000


def test_qwen3_8b_clusters_are_sparse():
    wl = W.qwen3_8b_decode(B=1)
    sizes = [len(tp["set"]) for kv_i in range(wl.n_ret)
             for _, (_, tp) in _sets(wl, 0, kv_i, 0.9).items()]
    assert np.median(sizes) <= 0.02 * wl.N


@pytest.mark.slow
def test_million_clusters_are_sparse():
    wl = W.million_decode()
    sizes = [len(tp["set"]) for _, (_, tp) in _sets(wl, 0, 0, 0.9).items()]
    assert np.median(sizes) <= 0.02 * wl.N


@pytest.mark.slow
def test_million_prefill_shape_and_density():
    """The 1M chunk: 4096 rows at the end of 2^20 keys, C5's head layout, clusters at
    C5's density (about three quarters of the keys clustered), rows aligned to
    clusters select a small fraction of the keys."""
    wl = W.make(6)
    assert (wl.N, wl.Tq, wl.q_start, wl.Hq, wl.Hkv) == (1 << 20, 4096, (1 << 20) - 4096, 32, 8)
    assert wl.ret_kv_heads == [0, 5] and wl.q_pre.shape == (1, 32, 4096, 128)
    kv = wl.ret_kv_heads[0]
    idx = O.f64_to_bf16(O.bf16_to_f64(wl.k_pre[0, kv]) @ O.bf16_to_f64(wl.w_k[0]))
    sizes = []
    for t in (0, 2047, 4095):
        s = O.scores(O.query_index(wl.q_pre[0, 0, t], wl.w_q[0]), idx[:wl.q_start + t + 1])
        sizes.append(len(O.top_p_set(s, 0.9)["set"]))
    assert np.median(sizes) <= 0.02 * wl.N, sizes
