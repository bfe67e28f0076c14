"""GPU parity of the V2 cluster index (rtp_cluster_build, rtp_decode_cluster_attn).

The build takes its nearest-centre decisions in fp32 with a fixed operation order
and sums the centres exactly, so the GPU's centres, members and offsets must equal
the oracle's bit for bit.  The decode selects clusters by a top-p cut over fp64
masses of fp32 centre scores: sets are compared like token sets (clusters whose
score lies within the band of the oracle's threshold may differ; a cut that
differs outside it must still be a valid top-p cut under the oracle's masses), and
outputs are always checked against the oracle's attention over the GPU's own set.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_long_retrieval_amd as R  # noqa: E402
import workloads as W  # noqa: E402
from oracle import rtp_oracle as O  # noqa: E402
from tests import _parity as P  # noqa: E402


def _build(layer, idx_dev, B, n_ret, n_tok, K, iters, init):
    Pn = B * n_ret
    cen = torch.zeros((Pn, K, 16), dtype=torch.float32, device="cuda")
    mem = torch.zeros((Pn, n_tok), dtype=torch.int32, device="cuda")
    off = torch.zeros((Pn, K + 1), dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(256, R.workspace_size(layer, R.OP_CLUSTER_BUILD, n_tok, Tq=K)),
                     dtype=torch.uint8, device="cuda")
    init_dev = torch.from_numpy(np.ascontiguousarray(init, dtype=np.int32)).to("cuda")
    R.cluster_build(layer, idx_dev, n_tok, K, iters, init_dev, cen, mem, off, ws)
    torch.cuda.synchronize()
    return cen, mem, off


def _index_of(wl):
    _, _, idx = O.caches_for(wl, rows_needed={kv: np.arange(1) for kv in range(wl.Hkv)})
    return idx


BUILD_CASES = [
    # (seed, B, Hkv, ret, N, n_tok, K, iters, duplicated seeds)
    (81, 1, 1, [0], 3000, 3000, 1, 2, False),
    (82, 1, 2, [1], 5000, 4321, 7, 0, False),       # no update, ragged n_tok
    (83, 2, 4, [0, 3], 9000, 9000, 128, 3, False),  # four pairs
    (84, 1, 1, [0], 20000, 19999, 256, 5, False),   # the largest K, several blocks
    (85, 1, 1, [0], 3000, 3000, 16, 3, True),       # empty clusters from repeated seeds
]


@pytest.mark.parametrize("case", BUILD_CASES, ids=[f"s{c[0]}" for c in BUILD_CASES])
def test_cluster_build_matches_oracle_bit_exact(case):
    seed, B, Hkv, ret, N, n_tok, K, iters, dup = case
    wl = W.random_decode(seed, B, 4 * Hkv, Hkv, N, ret, 256, n_needles=3)
    idx = _index_of(wl)
    layer = R.Layer(B, wl.Hq, Hkv, N, ret, wl.n_sink, wl.window, wl.rope_base)
    rng = np.random.default_rng(seed + 1000)
    n_ret = len(ret)
    init = np.stack([rng.choice(n_tok, K, replace=K > n_tok) for _ in range(B * n_ret)])
    if dup:
        init[:, K // 2:] = init[:, :K - K // 2][:, :K // 2]
    cen, mem, off = _build(layer, P.to_dev(idx), B, n_ret, n_tok, K, iters, init)
    cen, mem, off = cen.cpu().numpy(), mem.cpu().numpy(), off.cpu().numpy()
    for b in range(B):
        for i in range(n_ret):
            pr = b * n_ret + i
            r = O.kmeans_index(idx[b, i, :n_tok], init[pr], iters)
            assert np.array_equal(off[pr], r["offsets"]), f"offsets pair {pr}"
            assert np.array_equal(mem[pr], r["members"]), f"members pair {pr}"
            assert np.array_equal(cen[pr].view(np.uint32), r["centroids"].view(np.uint32)), \
                f"centroids pair {pr}"
    if dup:
        # the case exercises the update of clusters left without rows: the first
        # assignment (to the seeds) gives the repeated centres nothing
        x32 = O.bf16_to_f64(idx[0, 0, :n_tok]).astype(np.float32)
        first = set(O.kmeans_assign(x32, x32[init[0]]).tolist())
        assert len(set(range(K)) - first) > 0


def _check_clusters(hit_gpu, r, counts, p, neutral):
    """Hit sets equal, or differing only in clusters at the threshold (band), or a
    valid top-p cut under the oracle's masses.  Clusters made of sinks only
    (`neutral`) cannot be seen in a set and are left out of the comparison."""
    st = P.stats()
    hit_o = set(r["hit"].tolist()) - neutral
    hit_g = set(hit_gpu)
    if hit_g == hit_o:
        st["exact"] += 1
        return "exact"
    sig = r["sigma"].astype(np.float64)
    tau = float(r["tau"])
    diff = hit_g ^ hit_o
    if all(abs(sig[c] - tau) <= P.BAND_REL * max(abs(tau), 1.0) for c in diff):
        st["band"] += 1
        st["band_tokens"] += len(diff)
        return "band"
    assert p > P.STRICT_P, f"p={p}: cluster cut differs outside the band: {sorted(diff)[:8]}"
    live = np.nonzero(counts > 0)[0]
    m = sig[live].max()
    w = {int(c): counts[c] * np.exp(sig[c] - m) for c in live}
    W_ = sum(w.values())
    hit_full = hit_g | (set(r["hit"].tolist()) & neutral)
    mass = sum(w[c] for c in hit_full)
    lowest = min(sig[c] for c in hit_full)
    below = sum(w[c] for c in hit_full if sig[c] > lowest)
    assert mass >= p * W_ * (1 - P.MASS_TOL) and below < p * W_ * (1 + P.MASS_TOL), \
        f"cluster cut differs outside the band: {sorted(diff)[:8]}"
    st["valid-alt"] += 1
    st["alt_tokens"] += len(diff)
    st["max_mass_slack"] = max(st["max_mass_slack"], abs(mass / (p * W_) - 1.0))
    return "valid-alt"


def _decode(layer, wl, dev_q, dev_wq, kc, vc, cen, mem, off, K, n_tok, p, cap):
    out = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.int16, device="cuda")
    ws = torch.zeros(max(256, R.workspace_size(layer, R.OP_CLUSTER_DECODE, wl.N, Tq=K)),
                     dtype=torch.uint8, device="cuda")
    dbg = R.Debug(wl.B * wl.n_ret * wl.G, cap)
    R.decode_cluster_attn(layer, dev_q, dev_wq, kc, vc, cen, mem, off, K, n_tok, wl.N, p, out,
                          ws, debug=dbg)
    torch.cuda.synchronize()
    return {"out": P.from_dev(out), "cnt": dbg.sel_count.cpu().numpy(),
            "idx": dbg.sel_idx.cpu().numpy(), "tau": dbg.tau.cpu().numpy()}


def _compare_decode(wl, kc, vc, cl_np, n_tok, p, res, K):
    """Every retrieval q-head: set (via its clusters) and output against the oracle."""
    kinds = {}
    cen, mem, off = cl_np
    for b in range(wl.B):
        for i, kv in enumerate(wl.ret_kv_heads):
            pr = b * wl.n_ret + i
            cl = {"centroids": cen[pr], "members": mem[pr], "offsets": off[pr]}
            counts = np.diff(off[pr].astype(np.int64))
            assign = np.empty(n_tok, dtype=np.int64)
            neutral = set()
            for c in range(K):
                mc = mem[pr][off[pr][c]:off[pr][c + 1]]
                assign[mc] = c
                if len(mc) and mc.max() < wl.n_sink:
                    neutral.add(c)
            for g in range(wl.G):
                h = kv * wl.G + g
                unit = pr * wl.G + g
                r = O.cluster_head(wl.q_pre[b, h], wl.w_q[i * wl.G + g], kc[b, kv], vc[b, kv],
                                   cl, n_tok, wl.N - 1, p, wl.n_sink, wl.idx_scale,
                                   wl.attn_scale, wl.rope_base)
                S = P.gpu_set(res, unit)
                assert len(S) == len(np.unique(S)), "a token attended twice"
                extra = S[(S >= wl.n_sink) & (S < n_tok)]
                hit_gpu = sorted(set(assign[extra].tolist()))
                if p < 1.0:
                    kind = _check_clusters(hit_gpu, r, counts, p, neutral)
                else:
                    assert set(hit_gpu) == set(np.nonzero(counts)[0].tolist()) - neutral
                    kind = "exact"
                    P.stats()["exact"] += 1
                # the set is exactly: members of its clusters, appended tokens, sinks
                want = set(range(min(wl.n_sink, wl.N))) | set(range(n_tok, wl.N))
                for c in hit_gpu:
                    want |= set(mem[pr][off[pr][c]:off[pr][c + 1]].tolist())
                assert set(S.tolist()) == want, f"b{b} h{h}: set is not whole clusters"
                kinds[kind] = kinds.get(kind, 0) + 1
                qr = O.rope(P.bf16_f64(wl.q_pre[b, h]), wl.N - 1, wl.rope_base)
                own = O.attention(qr, kc[b, kv][S], vc[b, kv][S], wl.attn_scale)
                P.check_out(res["out"][b, h], own, f"own set b{b} h{h}")
                if kind == "exact":
                    assert np.array_equal(S, r["S"])
                P.check_out(res["out"][b, h], r["out"], f"b{b} h{h} ({kind})")
    return kinds


DECODE_CASES = [
    # (seed, B, Hq, Hkv, N, ret, n_tok, K, iters, n_sink)
    (91, 1, 8, 1, 6000, [0], 6000, 32, 3, 4),       # G = 8
    (92, 2, 8, 2, 5000, [1], 4500, 16, 2, 4),       # G = 4, B = 2, 500 appended tokens
    (93, 1, 4, 4, 4000, [0, 2], 3900, 64, 4, 0),    # G = 1, two retrieval heads, no sinks
    (94, 1, 4, 2, 3000, [0], 2990, 7, 1, 7),        # G = 2, 7 sinks
]


@pytest.mark.parametrize("p", [0.3, 0.9, 0.999, 1.0])
@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"s{c[0]}" for c in DECODE_CASES])
def test_cluster_decode_matches_oracle(case, p):
    seed, B, Hq, Hkv, N, ret, n_tok, K, iters, n_sink = case
    wl = W.random_decode(seed, B, Hq, Hkv, N, ret, 256, n_sink=n_sink, n_needles=4,
                         q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    layer = R.Layer(B, Hq, Hkv, N, ret, n_sink, wl.window, wl.rope_base)
    rng = np.random.default_rng(seed + 2000)
    init = np.stack([rng.choice(n_tok, K, replace=False) for _ in range(B * len(ret))])
    cen, mem, off = _build(layer, P.to_dev(idx), B, len(ret), n_tok, K, iters, init)
    res = _decode(layer, wl, P.to_dev(wl.q_pre), P.to_dev(wl.w_q), P.to_dev(kc), P.to_dev(vc),
                  cen, mem, off, K, n_tok, p, N)
    kinds = _compare_decode(wl, kc, vc, (cen.cpu().numpy(), mem.cpu().numpy(),
                                         off.cpu().numpy()), n_tok, p, res, K)
    print(f"{wl.name} p={p}: {kinds}")


def test_cluster_build_and_decode_deterministic():
    wl = W.random_decode(95, 1, 8, 1, 7000, [0], 256, n_needles=4, q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    layer = R.Layer(1, 8, 1, 7000, [0], wl.n_sink, wl.window, wl.rope_base)
    init = np.random.default_rng(7).choice(7000, 64, replace=False)[None]
    outs = []
    for _ in range(2):
        cen, mem, off = _build(layer, P.to_dev(idx), 1, 1, 6800, 64, 3, init)
        res = _decode(layer, wl, P.to_dev(wl.q_pre), P.to_dev(wl.w_q), P.to_dev(kc),
                      P.to_dev(vc), cen, mem, off, 64, 6800, 0.9, 7000)
        outs.append((cen.cpu().numpy().tobytes(), mem.cpu().numpy().tobytes(),
                     off.cpu().numpy().tobytes(), res["out"].tobytes()))
    assert outs[0] == outs[1]


def test_cluster_million():
    """1M context, K = 128 (the article's example), 3 updates: the index bit-exact
    against the oracle, then every retrieval q-head's set and output."""
    wl = W.make(4)
    rows = {kv: np.union1d(np.arange(wl.N - wl.window, wl.N), np.arange(wl.n_sink))
            for kv in range(wl.Hkv) if kv not in wl.ret_kv_heads}
    kc, vc, idx = O.caches_for(wl, rows_needed=rows)
    layer = R.Layer(wl.B, wl.Hq, wl.Hkv, wl.N, wl.ret_kv_heads, wl.n_sink, wl.window,
                    wl.rope_base)
    K, iters, n_tok = 128, 3, wl.N
    init = np.random.default_rng(1004).choice(n_tok, K, replace=False)[None]
    cen, mem, off = _build(layer, P.to_dev(idx), 1, 1, n_tok, K, iters, init)
    cl_np = (cen.cpu().numpy(), mem.cpu().numpy(), off.cpu().numpy())
    r = O.kmeans_index(idx[0, 0], init[0], iters)
    assert np.array_equal(cl_np[2][0], r["offsets"])
    assert np.array_equal(cl_np[1][0], r["members"])
    assert np.array_equal(cl_np[0][0].view(np.uint32), r["centroids"].view(np.uint32))
    res = _decode(layer, wl, P.to_dev(wl.q_pre), P.to_dev(wl.w_q), P.to_dev(kc), P.to_dev(vc),
                  cen, mem, off, K, n_tok, 0.9, wl.N)
    kinds = _compare_decode(wl, kc, vc, cl_np, n_tok, 0.9, res, K)
    print(f"1M cluster decode: {kinds}; set sizes {[int(c) for c in res['cnt']]}")
