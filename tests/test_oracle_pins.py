"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than its own formula: a
library routine (torch's bf16 conversion, torch's scaled-dot-product attention
in fp64), a closed form, a brute-force enumeration, or an invariant that any
correct implementation must satisfy.  A planted mistake in the oracle (a dropped
term, a wrong sign, a transposed operand, an off-by-one in the top-p scan)
fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import rtp_oracle as O

D = 128


def _bits_from_f32(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _f32_from_bits(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    assert np.array_equal(O.f64_to_bf16(x.astype(np.float64)), _bits_from_f32(x))


def test_bf16_round_ties_to_even_and_no_double_rounding():
    one = 0x3F80
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: tie goes to the even mantissa (1.0)
    assert O.f64_to_bf16(np.array([1 + 2.0 ** -8]))[0] == one
    # 1 + 3*2^-8 is the midpoint of 1+2^-7 (odd) and 1+2^-6 (even): rounds up
    assert O.f64_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == one + 2
    # slightly above a midpoint in fp64 but equal to it after fp32 rounding: must go up
    assert O.f64_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == one + 1
    assert O.f64_to_bf16(np.array([-(1 + 2.0 ** -8 + 2.0 ** -40)]))[0] == (one + 1) | 0x8000
    assert O.f64_to_bf16(np.array([0.0]))[0] == 0


# ------------------------------------------------------------------ RoPE

def _rope_complex(x, pos, base=1e6):
    """Textbook RoPE as complex multiplication: (x_i + i x_{i+D/2}) * exp(i pos theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    d2 = x.shape[-1] // 2
    theta = np.array([base ** (-(2.0 * i) / x.shape[-1]) for i in range(d2)])
    z = (x[..., :d2] + 1j * x[..., d2:]) * np.exp(1j * np.asarray(pos, float)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, D))
    pos = rng.integers(0, 1 << 20, 64)
    # theta_i may differ by an ulp between the two pow evaluations: pos * 1 ulp ~ 2e-10
    assert np.allclose(O.rope(x, pos), _rope_complex(x, pos), rtol=0, atol=1e-9)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    assert np.allclose(O.rope(q, 0), q, atol=0)
    for p in (1, 77, 65535, 1048575):
        assert abs(np.linalg.norm(O.rope(q, p)) - np.linalg.norm(q)) < 1e-12
    d1 = O.rope(q, 1000) @ O.rope(k, 10)
    d2 = O.rope(q, 5990) @ O.rope(k, 5000)
    assert abs(d1 - d2) < 1e-10
    # highest-frequency pair (theta_0 = 1): e_0 -> cos(p) e_0 + sin(p) e_64
    e0 = np.zeros(D); e0[0] = 1
    r = O.rope(e0, 3)
    assert abs(r[0] - math.cos(3)) < 1e-15 and abs(r[64] - math.sin(3)) < 1e-15
    e64 = np.zeros(D); e64[64] = 1
    r = O.rope(e64, 3)
    assert abs(r[0] + math.sin(3)) < 1e-15 and abs(r[64] - math.cos(3)) < 1e-15


# ------------------------------------------------------------------ top-p

def _brute_min_set(w, p):
    n = len(w)
    Z = w.sum()
    for size in range(1, n + 1):
        best = None
        for U in itertools.combinations(range(n), size):
            m = w[list(U)].sum()
            if m >= p * Z and (best is None or m > best[0]):
                best = (m, set(U))
        if best is not None:
            return best[1]
    return set(range(n))


@pytest.mark.parametrize("seed", range(12))
def test_top_p_brute_force_small(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 13))
    s = (rng.standard_normal(n) * 3).astype(np.float32)
    for p in (1e-6, 0.3, 0.5, 0.9, 0.999):
        got = set(O.top_p_set(s, p)["set"].tolist())
        w = np.exp(s.astype(np.float64) - s.max())
        assert got == _brute_min_set(w, p), (n, p)


def test_top_p_geometric_closed_form():
    n = 20
    s = (-np.arange(n) * math.log(2)).astype(np.float32)
    for p, k in ((0.6, 2), (0.9, 4), (0.97, 6), (0.2, 1)):
        assert math.ceil(-math.log2(1 - p * (1 - 2.0 ** -n))) == k
        assert O.top_p_set(s, p)["set"].tolist() == list(range(k))


def test_top_p_needles_closed_form():
    N, n = 4096, 3
    for L in (5.0, 8.0, 12.0):
        s = np.zeros(N, dtype=np.float32)
        pos = [10, 999, 3000]
        s[pos] = L
        E = math.exp(L)
        share = n * E / (n * E + N - n)
        T = O.top_p_set(s, 0.9)["set"].tolist()
        if share >= 0.9:
            assert T == pos
        else:
            assert T == list(range(N))  # the rest are tied zeros: all of them join


def test_top_p_ties_and_p_one():
    s = np.full(50, 1.5, dtype=np.float32)
    assert len(O.top_p_set(s, 0.5)["set"]) == 50
    r = np.random.default_rng(3).standard_normal(50).astype(np.float32)
    t = O.top_p_set(r, 1.0)
    assert len(t["set"]) == 50 and t["tau"] == -np.inf


@pytest.mark.parametrize("seed", range(5))
def test_top_p_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    s = (rng.standard_normal(5000) * rng.uniform(0.5, 6)).astype(np.float32)
    for p in (0.5, 0.8, 0.9, 0.95, 0.999):
        t = O.top_p_set(s, p)
        w = np.exp(s.astype(np.float64) - s.max())
        Z = w.sum()
        T = t["set"]
        assert w[T].sum() >= p * Z                       # reaches p
        above = s > np.float32(t["tau"])
        assert w[above].sum() < p * Z                    # minimal threshold
        assert s[T].min() >= np.float32(t["tau"])         # upward closed
        assert (s[~np.isin(np.arange(len(s)), T)] < np.float32(t["tau"])).all()


# ------------------------------------------------------------------ attention

def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    K = _bits_from_f32(rng.standard_normal((40, D)))
    vrow = _bits_from_f32(rng.standard_normal(D))
    V = np.tile(vrow, (40, 1))
    q = rng.standard_normal(D)
    assert np.allclose(O.attention(q, K, V, 0.1), _f32_from_bits(vrow), atol=1e-12)
    V2 = _bits_from_f32(rng.standard_normal((40, D)))
    assert np.allclose(O.attention(np.zeros(D), K, V2, 0.1),
                       _f32_from_bits(V2).astype(np.float64).mean(0), atol=1e-12)
    assert np.allclose(O.attention(q, K[7:8], V2[7:8], 0.1), _f32_from_bits(V2[7]), atol=0)


def _sdpa64(q, K, V, scale, mask=None):
    qt = torch.from_numpy(np.asarray(q, np.float64)).view(1, 1, 1, -1)
    kt = torch.from_numpy(np.asarray(K, np.float64)).view(1, 1, K.shape[0], -1)
    vt = torch.from_numpy(np.asarray(V, np.float64)).view(1, 1, V.shape[0], -1)
    m = None if mask is None else torch.from_numpy(mask).view(1, 1, 1, -1)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, scale=scale).view(-1).numpy()


def _small_wl(seed=5, N=700, window=128):
    import workloads
    return workloads.random_decode(seed, B=1, Hq=4, Hkv=2, N=N, ret_kv=[0], window=window,
                                   n_sink=4, n_needles=3)


def test_p_one_equals_dense_attention():
    wl = _small_wl()
    kc, vc, idx = O.caches_for(wl)
    res = O.decode(wl, kc, vc, idx, top_p=1.0, heads=[0, 1])
    pos = wl.N - 1
    for h in (0, 1):
        q = _rope_complex(O.bf16_to_f64(wl.q_pre[0, h]), pos)
        K = _rope_complex(O.bf16_to_f64(wl.k_pre[0, 0]), np.arange(wl.N))
        # the cache holds bf16(RoPE(k)); use the same rounded rows for the reference
        K = O.bf16_to_f64(O.f64_to_bf16(K))
        ref = _sdpa64(q, K, O.bf16_to_f64(wl.v[0, 0]), wl.attn_scale)
        assert len(res[(0, h)]["S"]) == wl.N
        assert np.allclose(res[(0, h)]["out"], ref, rtol=0, atol=1e-12)


def test_swa_equals_masked_dense_attention():
    wl = _small_wl(seed=6, N=900, window=200)
    kc, vc, idx = O.caches_for(wl)
    res = O.decode(wl, kc, vc, idx, top_p=0.9, heads=[2, 3])
    pos = wl.N - 1
    j = np.arange(wl.N)
    mask = ((j > pos - wl.window) & (j <= pos)) | (j < wl.n_sink)
    assert mask.sum() == wl.window + wl.n_sink
    for h in (2, 3):
        q = _rope_complex(O.bf16_to_f64(wl.q_pre[0, h]), pos)
        K = O.bf16_to_f64(O.f64_to_bf16(_rope_complex(O.bf16_to_f64(wl.k_pre[0, 1]), j)))
        ref = _sdpa64(q, K, O.bf16_to_f64(wl.v[0, 1]), wl.attn_scale, mask)
        assert np.allclose(res[(0, h)]["out"], ref, rtol=0, atol=1e-12)


def test_swa_window_covers_sinks_when_short():
    L = O.swa_keys(pos=5, window=8192, n_sink=4)
    assert L.tolist() == list(range(6))
    L = O.swa_keys(pos=100, window=10, n_sink=4)
    assert L.tolist() == [0, 1, 2, 3] + list(range(91, 101))


def test_sinks_added_after_top_p():
    wl = _small_wl(seed=7)
    kc, vc, idx = O.caches_for(wl)
    r = O.decode(wl, kc, vc, idx, top_p=0.5, heads=[0])[(0, 0)]
    assert set(range(4)) <= set(r["S"].tolist())
    assert set(r["T"].tolist()) <= set(r["S"].tolist())
    assert set(r["S"].tolist()) == set(r["T"].tolist()) | {0, 1, 2, 3}


# ------------------------------------------------------------------ append / index

def test_index_matches_library_matmul():
    wl = _small_wl(seed=8, N=2048)
    _, _, idx = O.caches_for(wl)
    k = torch.from_numpy(O.bf16_to_f64(wl.k_pre[0, 0]))
    W = torch.from_numpy(O.bf16_to_f64(wl.w_k[0]))
    exact = (k @ W).numpy()                     # products of bf16 are exact in fp64
    f32 = exact.astype(np.float32)
    lib = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = idx[0, 0]
    diff = ours != lib
    # the library path rounds twice (fp64 -> fp32 -> bf16); it may differ only where
    # the fp32 image sits exactly on a bf16 midpoint
    u = f32.view(np.uint32)
    assert np.all((u[diff] & 0xFFFF) == 0x8000)
    assert diff.mean() < 1e-3


def test_scores_use_pre_rope_index():
    wl = _small_wl(seed=9, N=300)
    kc, vc, idx = O.caches_for(wl)
    r = O.decode(wl, kc, vc, idx, top_p=0.9, heads=[1])[(0, 1)]
    qi = O.bf16_to_f64(wl.q_pre[0, 1]) @ O.bf16_to_f64(wl.w_q[1])
    s_ref = O.bf16_to_f64(idx[0, 0]) @ qi.astype(np.float32).astype(np.float64)
    assert np.allclose(r["scores"], s_ref, rtol=1e-6, atol=1e-6)
    # the index is not the projection of the rotated key
    rot = O.bf16_to_f64(kc[0, 0]) @ O.bf16_to_f64(wl.w_k[0])
    assert not np.allclose(O.bf16_to_f64(idx[0, 0]), rot, atol=1e-2)


def test_prefill_row_p_one_is_causal_dense():
    import workloads
    wl = workloads.random_prefill(11, B=1, Hq=4, Hkv=2, N=400, Tq=16, ret_kv=[0], window=64)
    kc, vc, idx = O.caches_for(wl)
    for t in (0, 7, 15):
        pos = wl.q_start + t
        r = O.prefill_row(wl, kc, vc, idx, 0, 1, t, 1.0)
        q = _rope_complex(O.bf16_to_f64(wl.q_pre[0, 1, t]), pos)
        K = O.bf16_to_f64(kc[0, 0, :pos + 1])
        ref = _sdpa64(q, K, O.bf16_to_f64(wl.v[0, 0, :pos + 1]), wl.attn_scale)
        assert np.allclose(r["out"], ref, atol=1e-12)
        assert len(r["S"]) == pos + 1


# ---------------------------------------------------------------- fixed top-k budget

@pytest.mark.parametrize("seed", range(6))
def test_top_k_is_the_k_largest(seed):
    """Distinct scores: the set is exactly the k largest, by an independent sort."""
    rng = np.random.default_rng(300 + seed)
    s = rng.permutation(np.arange(40, dtype=np.float32) * np.float32(0.37) - np.float32(5))
    for k in (1, 2, 7, 39, 40, 55):
        got = np.sort(O.top_k_set(s, k)["set"])
        want = np.sort(sorted(range(len(s)), key=lambda j: -float(s[j]))[:min(k, len(s))])
        assert np.array_equal(got, want), k


def test_top_k_ties_and_budget_past_n():
    s = np.array([3, 1, 3, 3, 2, 0], dtype=np.float32)
    assert np.array_equal(np.sort(O.top_k_set(s, 2)["set"]), [0, 2, 3])  # ties at tau kept
    assert np.array_equal(np.sort(O.top_k_set(s, 4)["set"]), [0, 2, 3, 4])
    assert np.array_equal(O.top_k_set(s, 6)["set"], np.arange(6))
    assert O.top_k_set(s, 9)["tau"] == -np.inf


# ------------------------------------------------------------------ V2 cluster index

def _rand_index_bits(rng, n, scale=1.0):
    return O.f64_to_bf16(rng.standard_normal((n, 16)) * scale)


def test_kmeans_assign_is_nearest_centre():
    """Against scipy's fp64 distances: equal except where the two nearest centres are
    within fp32 rounding of each other."""
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(400)
    x = O.bf16_to_f64(_rand_index_bits(rng, 3000)).astype(np.float32)
    c = rng.standard_normal((37, 16)).astype(np.float32)
    got = O.kmeans_assign(x, c)
    d = cdist(x.astype(np.float64), c.astype(np.float64), "sqeuclidean")
    want = d.argmin(axis=1)
    two = np.sort(d, axis=1)[:, :2]
    near_tie = (two[:, 1] - two[:, 0]) <= 1e-5 * two[:, 1]
    assert np.array_equal(got[~near_tie], want[~near_tie])
    assert near_tie.mean() < 0.01


def test_kmeans_ties_go_to_lowest_centre():
    x = np.zeros((3, 16), dtype=np.float32)
    x[1, 0] = 1.0
    c = np.zeros((4, 16), dtype=np.float32)
    c[0, 0], c[1, 0], c[2, 0], c[3, 0] = 2.0, 0.0, 0.0, 1.0   # rows 1 and 2 are identical
    a = O.kmeans_assign(x, c)
    assert a[0] == 1           # equal distance to centres 1 and 2 -> 1
    assert a[1] == 3           # exactly on centre 3
    assert a[2] == 1


def test_kmeans_single_cluster_is_the_mean():
    rng = np.random.default_rng(401)
    bits = _rand_index_bits(rng, 5000, 3.0)
    r = O.kmeans_index(bits, [17], iters=2)
    mean = O.bf16_to_f64(bits).mean(axis=0)
    assert np.all(np.abs(r["centroids"][0] - mean) <= 2.0 ** -22 * np.maximum(np.abs(mean), 1))
    assert np.array_equal(r["assign"], np.zeros(5000))
    assert np.array_equal(r["members"], np.arange(5000))
    assert list(r["offsets"]) == [0, 5000]


def test_kmeans_tiny_values_truncation_bound():
    """Index values below 2^-17 are not whole multiples of 2^-24, so the centre sums
    truncate them (the cluster-index reading).  Each row then loses less than one
    2^-24 unit per dimension, so a centre of n rows is within 2^-24 of the exact
    fp64 mean (plus the fp32 rounding of the result); rows and centres of size
    2^-20 and below are assigned exactly as scipy's fp64 distances say."""
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(402)
    x = rng.standard_normal((4000, 16)) * 2.0 ** -19            # |x| mostly below 2^-17
    bits = O.f64_to_bf16(x)
    xv = O.bf16_to_f64(bits)
    assert (np.abs(xv) < 2.0 ** -17).mean() > 0.9
    frac = np.abs(xv * 2.0 ** 24 - np.trunc(xv * 2.0 ** 24))
    assert (frac > 0).mean() > 0.5                                # truncation really occurs
    assign = np.arange(4000) % 5
    c = O.kmeans_centres(bits, assign, np.zeros((5, 16), np.float32))
    for k in range(5):
        mean = xv[assign == k].mean(axis=0)
        err = np.abs(c[k].astype(np.float64) - mean)
        assert np.all(err <= 2.0 ** -24 + 2.0 ** -24 * np.abs(mean)), (k, err.max())
    x32 = xv.astype(np.float32)
    cen = (rng.standard_normal((9, 16)) * 2.0 ** -20).astype(np.float32)
    got = O.kmeans_assign(x32, cen)
    d = cdist(x32.astype(np.float64), cen.astype(np.float64), "sqeuclidean")
    two = np.sort(d, axis=1)[:, :2]
    far = (two[:, 1] - two[:, 0]) > 1e-5 * two[:, 1]
    assert far.mean() > 0.98
    assert np.array_equal(got[far], d.argmin(axis=1)[far])


def test_kmeans_recovers_planted_clusters():
    """Well-separated clusters seeded with one row of each: the partition is the planted
    one and the centres are the members' means."""
    rng = np.random.default_rng(402)
    centres = rng.standard_normal((6, 16)) * 20.0
    label = rng.integers(0, 6, 900)
    bits = O.f64_to_bf16(centres[label] + 0.1 * rng.standard_normal((900, 16)))
    seeds = [int(np.nonzero(label == t)[0][0]) for t in (3, 0, 5, 1, 4, 2)]
    r = O.kmeans_index(bits, seeds, iters=3)
    order = [3, 0, 5, 1, 4, 2]               # cluster c was seeded from planted order[c]
    assert np.array_equal(np.asarray(order)[r["assign"]], label)
    x = O.bf16_to_f64(bits)
    for c, t in enumerate(order):
        assert np.allclose(r["centroids"][c], x[label == t].mean(axis=0), atol=1e-5)


def test_kmeans_objective_never_increases():
    rng = np.random.default_rng(403)
    bits = _rand_index_bits(rng, 4000)
    x = O.bf16_to_f64(bits)
    init = rng.choice(4000, 24, replace=False)
    prev = np.inf
    for it in range(6):
        r = O.kmeans_index(bits, init, iters=it)
        obj = ((x - r["centroids"][r["assign"]].astype(np.float64)) ** 2).sum()
        assert obj <= prev * (1 + 1e-9), (it, obj, prev)
        prev = obj


def test_kmeans_empty_cluster_keeps_its_centre():
    """Centre 2 duplicates centre 0, so the first assignment gives it no rows (ties go
    to the lower centre) and the first update leaves it where it was."""
    rng = np.random.default_rng(404)
    bits = _rand_index_bits(rng, 300)
    x32 = O.bf16_to_f64(bits).astype(np.float32)
    assert 2 not in set(O.kmeans_assign(x32, x32[[5, 9, 5]]).tolist())
    r = O.kmeans_index(bits, [5, 9, 5], iters=1)
    assert np.array_equal(r["centroids"][2], x32[5])
    assert not np.array_equal(r["centroids"][0], x32[5])


def test_kmeans_members_grouped_by_cluster_ascending():
    rng = np.random.default_rng(405)
    bits = _rand_index_bits(rng, 2000)
    r = O.kmeans_index(bits, rng.choice(2000, 16, replace=False), iters=2)
    want = [j for _, j in sorted((int(r["assign"][j]), j) for j in range(2000))]
    assert np.array_equal(r["members"], want)
    assert np.array_equal(np.diff(r["offsets"]), np.bincount(r["assign"], minlength=16))


def _select_brute(sigma, counts, p):
    """Largest threshold t among the live sigmas whose set {sigma >= t} holds p of the
    size-weighted mass (enumeration over thresholds)."""
    live = [c for c in range(len(sigma)) if counts[c] > 0]
    m = max(float(sigma[c]) for c in live)
    w = {c: counts[c] * math.exp(float(sigma[c]) - m) for c in live}
    W = sum(w.values())
    best = None
    for t in sorted({float(sigma[c]) for c in live}):
        mass = sum(w[c] for c in live if float(sigma[c]) >= t)
        if mass >= p * W:
            best = t
    return sorted(c for c in live if float(sigma[c]) >= best)


@pytest.mark.parametrize("seed", range(6))
def test_cluster_select_brute_force(seed):
    rng = np.random.default_rng(410 + seed)
    K = 7
    cen = rng.standard_normal((K, 16)).astype(np.float32)
    qi = rng.standard_normal(16).astype(np.float32)
    counts = rng.integers(0, 50, K)
    counts[0] = max(counts[0], 1)
    if seed % 2:
        cen[3] = cen[5]                           # a tie between two clusters
    for p in (0.05, 0.3, 0.6, 0.9, 0.999):
        r = O.cluster_select(qi, cen, counts, p)
        assert list(np.sort(r["hit"])) == _select_brute(r["sigma"], counts, p), p


def test_cluster_select_p_one_and_dominant_cluster():
    cen = np.zeros((5, 16), dtype=np.float32)
    cen[2, 0] = 30.0
    qi = np.zeros(16, dtype=np.float32)
    qi[0] = 1.0
    counts = np.array([10, 0, 3, 40, 7])
    assert list(O.cluster_select(qi, cen, counts, 1.0)["hit"]) == [0, 2, 3, 4]
    assert list(O.cluster_select(qi, cen, counts, 0.99)["hit"]) == [2]


def test_cluster_head_p_one_is_dense_and_keeps_tail_and_sinks():
    wl = _small_wl(N=600)
    kc, vc, idx = O.caches_for(wl)
    n_tok = 520
    rng = np.random.default_rng(420)
    cl = O.kmeans_index(idx[0, 0, :n_tok], rng.choice(n_tok, 8, replace=False), iters=3)
    pos = wl.N - 1
    q = _rope_complex(O.bf16_to_f64(wl.q_pre[0, 0]), pos)
    K = O.bf16_to_f64(O.f64_to_bf16(_rope_complex(O.bf16_to_f64(wl.k_pre[0, 0]), np.arange(wl.N))))
    r = O.cluster_head(wl.q_pre[0, 0], wl.w_q[0], kc[0, 0], vc[0, 0], cl, n_tok, pos, 1.0,
                       wl.n_sink, 1.0, wl.attn_scale, wl.rope_base)
    assert np.array_equal(r["S"], np.arange(wl.N))
    ref = _sdpa64(q, K, O.bf16_to_f64(wl.v[0, 0]), wl.attn_scale)
    assert np.allclose(r["out"], ref, rtol=0, atol=1e-12)
    r = O.cluster_head(wl.q_pre[0, 0], wl.w_q[0], kc[0, 0], vc[0, 0], cl, n_tok, pos, 1e-6,
                       wl.n_sink, 1.0, wl.attn_scale, wl.rope_base)
    assert len(r["hit"]) >= 1
    members = np.concatenate([cl["members"][cl["offsets"][c]:cl["offsets"][c + 1]]
                              for c in r["hit"]])
    assert set(range(wl.n_sink)) <= set(r["S"].tolist())
    assert set(range(n_tok, wl.N)) <= set(r["S"].tolist())
    assert set(r["S"].tolist()) == set(members.tolist()) | set(range(wl.n_sink)) | set(range(n_tok, wl.N))
