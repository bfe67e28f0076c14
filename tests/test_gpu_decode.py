"""GPU parity of the decode path (append, retrieval decode, SWA) against the oracle.

All cases are seeded; each runs the C ABI on cuda:0 and compares with the CPU
oracle on the same bytes (caches and index produced by the oracle's append).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rtp_oracle as O
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _run(wl, top_p, cap=None, max_seq=None, idx_scale=1.0):
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx, max_seq=max_seq)
    res = dev.decode(top_p, debug_cap=cap or wl.N, idx_scale=idx_scale)
    return kc, vc, idx, res


def test_append_matches_oracle():
    wl = W.random_decode(21, B=2, Hq=8, Hkv=4, N=300, ret_kv=[1, 3], window=64)
    layer = P.R.Layer(wl.B, wl.Hq, wl.Hkv, 400, wl.ret_kv_heads, 4, 64)
    kc = torch.zeros((2, 4, 400, 128), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    idx = torch.zeros((2, 2, 400, 16), dtype=torch.int16, device="cuda")
    start = 37
    P.R.index_append(layer, P.to_dev(wl.k_pre), P.to_dev(wl.v), P.to_dev(wl.w_k), start,
                     kc, vc, idx)
    # a one-token append right after (the decode-step shape)
    one_k = wl.k_pre[:, :, :1].copy()
    one_v = wl.v[:, :, :1].copy()
    P.R.index_append(layer, P.to_dev(one_k), P.to_dev(one_v), P.to_dev(wl.w_k), start + 300,
                     kc, vc, idx)
    torch.cuda.synchronize()
    ok, ov, oi = O.append(wl.k_pre, wl.v, wl.w_k, wl.ret_kv_heads, start)
    gk = P.from_dev(kc)[:, :, start:start + 300]
    gi = P.from_dev(idx)[:, :, start:start + 300]
    assert np.array_equal(P.from_dev(vc)[:, :, start:start + 300], ov)
    assert np.array_equal(gi, oi), "index rows must be the exact bf16 of the fp64 projection"
    d = np.abs(gk.astype(np.int32) - ok.astype(np.int32))
    assert d.max() <= 1 and (d != 0).mean() < 1e-4, (d.max(), (d != 0).mean())
    k1, _, i1 = O.append(one_k, one_v, wl.w_k, wl.ret_kv_heads, start + 300)
    assert np.array_equal(P.from_dev(idx)[:, :, start + 300:start + 301], i1)
    d1 = np.abs(P.from_dev(kc)[:, :, start + 300:start + 301].astype(np.int32) - k1.astype(np.int32))
    assert d1.max() <= 1
    # rows outside the appended range stay untouched
    assert not P.from_dev(kc)[:, :, :start].any() and not P.from_dev(kc)[:, :, start + 301:].any()


@pytest.mark.parametrize("top_p", [0.9, 1e-6, 0.5, 0.999, 1.0])
def test_tiny_decode(top_p):
    wl = W.make(1)
    kc, vc, idx, res = _run(wl, top_p)
    summ = P.compare_decode(wl, kc, vc, idx, res, top_p)
    print("tiny", top_p, summ)
    if top_p == 0.9:
        # the needles of each head are selected
        for h in (0, 1):
            mine = [pp for pp, o in zip(wl.meta["needles"], wl.meta["needle_owner"]) if o == h]
            assert set(mine) <= set(P.gpu_set(res, h).tolist())


CASES = [
    # seed, B, Hq, Hkv, N, ret, window, needles, q_scale
    (31, 1, 2, 1, 1, [0], 16, 0, 1.0),
    (32, 1, 2, 2, 3, [1], 2, 0, 1.0),
    (33, 1, 4, 1, 4, [0], 8, 0, 1.0),
    (34, 2, 4, 2, 5, [0], 3, 0, 1.0),
    (35, 1, 8, 1, 17, [0], 5, 1, 1.0),
    (36, 1, 8, 2, 511, [0, 1], 100, 3, 1.0),
    (37, 2, 16, 4, 4099, [1, 2], 300, 4, 1.0),
    (38, 1, 8, 8, 6149, [0, 3, 7], 2048, 2, 2.0),
    (39, 1, 32, 4, 2 * 2048 + 1, [0], 1024, 0, 3.0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_N{c[4]}_G{c[2] // c[3]}" for c in CASES])
@pytest.mark.parametrize("top_p", [1e-6, 0.5, 0.9, 0.999, 1.0])
def test_random_shapes(case, top_p):
    seed, B, Hq, Hkv, N, ret, window, needles, qs = case
    wl = W.random_decode(seed, B, Hq, Hkv, N, ret, window, n_needles=needles, q_scale=qs)
    kc, vc, idx, res = _run(wl, top_p, max_seq=N + 7)
    summ = P.compare_decode(wl, kc, vc, idx, res, top_p)
    print(case, top_p, summ)


def test_all_scores_tied():
    """q = 0 on every head: all indexer scores are 0, every key joins (ties), and
    the output is the mean of V over all keys."""
    wl = W.random_decode(41, 1, 4, 2, 700, [0], 64)
    wl.q_pre[:] = 0
    kc, vc, idx, res = _run(wl, 0.5)
    for h in (0, 1):
        assert len(P.gpu_set(res, h)) == wl.N
    P.compare_decode(wl, kc, vc, idx, res, 0.5)


def test_boundary_below_histogram_window():
    """One key 17.5 above a flat background and p close to 1: the needle alone does
    not reach p, so the threshold falls 17.5 below the max, beyond the 16-unit
    histogram window; the tail of the window becomes the candidate set."""
    wl = W.random_decode(42, 1, 8, 1, 9000, [0], 512)
    kc, vc, idx = O.caches_for(wl)
    rng = np.random.default_rng(7)
    qi0 = O.query_index(wl.q_pre[0, 0], wl.w_q[0]).astype(np.float64)
    rows = 0.01 * rng.standard_normal((wl.N, 16))
    rows[1234] = 17.5 * qi0 / (qi0 @ qi0)
    idx = idx.copy()
    idx[0, 0] = O.f64_to_bf16(rows)
    res = P.Device(wl, kc, vc, idx).decode(0.9999, debug_cap=wl.N)
    r0 = O.decode(wl, kc, vc, idx, 0.9999, heads=[0])[(0, 0)]
    assert r0["m"] - r0["tau"] > 16 and len(r0["T"]) > 100, (r0["m"], r0["tau"], len(r0["T"]))
    print(P.compare_decode(wl, kc, vc, idx, res, 0.9999))


def test_idx_scale():
    wl = W.random_decode(43, 1, 4, 1, 3000, [0], 256, n_needles=2)
    kc, vc, idx, res = _run(wl, 0.9, idx_scale=0.25)
    wl.idx_scale = 0.25
    print(P.compare_decode(wl, kc, vc, idx, res, 0.9))


def test_deterministic_repeat():
    wl = W.random_decode(44, 2, 8, 2, 20000, [0], 1000, n_needles=3, q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    a = dev.decode(0.9, debug_cap=wl.N)
    b = dev.decode(0.9, debug_cap=wl.N)
    assert np.array_equal(a["cnt"], b["cnt"]) and np.array_equal(a["tau"], b["tau"])
    for u in range(len(a["cnt"])):
        assert np.array_equal(P.gpu_set(a, u), P.gpu_set(b, u))


def test_workspace_reuse_across_shapes():
    """One workspace, zero-filled once, serves consecutive calls of different
    lengths and top-p values; each result equals the one from a fresh workspace
    (the kernels leave their counters at zero)."""
    wls = [W.random_decode(46, 1, 8, 2, n, [0], 256, n_needles=2, q_scale=1.5)
           for n in (5000, 300, 70000)]
    devs = []
    for wl in wls:
        kc, vc, idx = O.caches_for(wl)
        devs.append(P.Device(wl, kc, vc, idx))
    big = max(P.R.workspace_size(d.layer, P.R.OP_DECODE, d.wl.N) for d in devs)
    bigs = max(P.R.workspace_size(d.layer, P.R.OP_SWA, d.wl.N) for d in devs)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    wss = torch.zeros(bigs, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for d, p in zip(devs, (0.9, 0.5, 0.95)):
            a = d.decode(p, debug_cap=d.wl.N, ws=ws, wss=wss)
            b = d.decode(p, debug_cap=d.wl.N)
            assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["cnt"], b["cnt"])
            assert np.array_equal(a["tau"], b["tau"])


@pytest.mark.parametrize("window,n_sink", [(1, 4), (5000, 4), (64, 0), (8, 30)])
def test_swa_edges(window, n_sink):
    wl = W.random_decode(45, 1, 8, 2, 1000, [0], window, n_sink=n_sink)
    kc, vc, idx, res = _run(wl, 0.9)
    print(P.compare_decode(wl, kc, vc, idx, res, 0.9))


def test_graph_replay_matches_eager():
    """The whole decode step (append of the newest token, local-head SWA on a second
    stream, retrieval decode) captured in a HIP graph gives the eager step's output on
    every replay, with unrelated eager work and synchronizations between replays."""
    import sparse_attention_long_retrieval_amd as R
    wl = W.random_decode(46, 1, 16, 4, 30000, [0, 2], 2048, n_needles=2, q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    N = wl.N
    new_k = P.to_dev(wl.k_pre[:, :, N - 1:N])
    new_v = P.to_dev(wl.v[:, :, N - 1:N])
    w_k = P.to_dev(wl.w_k)
    out = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.int16, device="cuda")
    ws = torch.zeros(R.workspace_size(dev.layer, R.OP_DECODE, N), dtype=torch.uint8,
                     device="cuda")
    wss = torch.zeros(R.workspace_size(dev.layer, R.OP_SWA, N), dtype=torch.uint8,
                      device="cuda")
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def step():
        cur = torch.cuda.current_stream()
        R.index_append(dev.layer, new_k, new_v, w_k, N - 1, dev.kc, dev.vc, dev.idx)
        fork.record(cur)
        side.wait_event(fork)
        R.swa_attn(dev.layer, dev.q, N - 1, 1, dev.kc, dev.vc, out, wss, stream=side)
        join.record(side)
        R.decode_sparse_attn(dev.layer, dev.q, dev.w_q, dev.kc, dev.vc, dev.idx, N, 0.9, out,
                             ws)
        cur.wait_event(join)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    other = torch.zeros_like(out)
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
        # eager work between replays: another decode into another buffer, torch ops
        R.decode_sparse_attn(dev.layer, dev.q, dev.w_q, dev.kc, dev.vc, dev.idx, N, 0.5,
                             other, ws)
        torch.cuda.synchronize()
        _ = (other.float() * 2).sum().item()
    # the eager result itself is the oracle's (parity of the step)
    res = {"out": P.from_dev(out)}
    ref = O.decode(wl, kc, vc, idx, 0.9)
    for (b, h), r in ref.items():
        P.check_out(res["out"][b, h], r["out"], f"graph b{b} h{h}")


TOPK_CASES = [
    # (seed, B, Hq, Hkv, N, ret_kv, window)
    (51, 1, 4, 2, 4096, [0], 512),
    (52, 2, 16, 2, 20000, [1], 1000),       # G = 8, B = 2
    (53, 1, 8, 4, 9000, [0, 3], 700),       # two retrieval heads, G = 2
]


@pytest.mark.parametrize("top_k", [1, 7, 300, 4096, 10 ** 6])
@pytest.mark.parametrize("case", TOPK_CASES, ids=[f"s{c[0]}" for c in TOPK_CASES])
def test_decode_topk(case, top_k):
    """Fixed budget decode: the top_k highest scores plus sinks, against the oracle."""
    seed, B, Hq, Hkv, N, ret, window = case
    wl = W.random_decode(seed, B, Hq, Hkv, N, ret, window, n_needles=2, q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    res = P.Device(wl, kc, vc, idx).decode(0.9, debug_cap=N, top_k=top_k)
    ref = O.decode(wl, kc, vc, idx, 0.9, top_k=top_k)
    kinds = {}
    for (b, h), r in ref.items():
        kv = h // wl.G
        if kv not in wl.ret_kv_heads:
            continue
        i = wl.ret_kv_heads.index(kv)
        unit = (b * wl.n_ret + i) * wl.G + h % wl.G
        S = P.gpu_set(res, unit)
        kind = P.check_set_topk(S, r, top_k, wl.n_sink)
        kinds[kind] = kinds.get(kind, 0) + 1
        qr = O.rope(P.bf16_f64(wl.q_pre[b, h]), N - 1, wl.rope_base)
        own = O.attention(qr, kc[b, kv][S], vc[b, kv][S], wl.attn_scale)
        P.check_out(res["out"][b, h], own, f"own set b{b} h{h}")
        P.check_out(res["out"][b, h], r["out"], f"b{b} h{h} ({kind})")
    print(f"{wl.name} top-{top_k}: {kinds}")


def test_decode_topk_million_budgets():
    """1M-context decode (512 clusters, 8 retrieval q-heads) with the pages' ablation
    budgets 4096 and 16384: every set and output against the oracle."""
    wl = W.make(4)
    rows = {kv: np.union1d(np.arange(wl.N - wl.window, wl.N), np.arange(wl.n_sink))
            for kv in range(wl.Hkv) if kv not in wl.ret_kv_heads}
    kc, vc, idx = O.caches_for(wl, rows_needed=rows)
    dev = P.Device(wl, kc, vc, idx)
    for k in (4096, 16384):
        res = dev.decode(0.9, debug_cap=2 * k, top_k=k)
        ref = O.decode(wl, kc, vc, idx, 0.9, heads=wl.ret_q_heads(), top_k=k)
        for (b, h), r in ref.items():
            unit = (b * wl.n_ret + wl.ret_kv_heads.index(h // wl.G)) * wl.G + h % wl.G
            S = P.gpu_set(res, unit)
            kind = P.check_set_topk(S, r, k, wl.n_sink)
            qr = O.rope(P.bf16_f64(wl.q_pre[b, h]), wl.N - 1, wl.rope_base)
            own = O.attention(qr, kc[b, h // wl.G][S], vc[b, h // wl.G][S], wl.attn_scale)
            P.check_out(res["out"][b, h], own, f"top-{k} own set h{h}")
            P.check_out(res["out"][b, h], r["out"], f"top-{k} h{h} ({kind})")


# (needle score, background half-width, N, top_k, candidate range the case is built for)
FAR_BUDGET_CASES = [
    (25.0, 4.0, 3000, 100, (1, 8192)),           # 1-unit grid
    (60.0, 4.0, 3000, 100, (1, 8192)),           # 2-unit grid, keys and tokens in LDS
    (60.0, 4.0, 48000, 100, (8193, 16384)),      # keys alone in LDS
    (60.0, 4.0, 100000, 100, (16385, 10 ** 9)),  # candidates read in place
    (300.0, 4.0, 9000, 100, (8193, 16384)),      # beyond the coarsest window too
]


def _far_candidates(s: np.ndarray, k: int) -> int:
    """Size of the candidate list the grids leave: the boundary bin of the finest
    grid (widths 0.5, 1, 2, 4, 8; 32 bins below the top) that reaches the k-th
    score, else everything below the coarsest window."""
    kth = np.sort(s)[::-1][k - 1]
    for w in (0.5, 1.0, 2.0, 4.0, 8.0):
        if np.floor(s.max() / w) - np.floor(kth / w) < 32:
            return int((np.floor(s / w) == np.floor(kth / w)).sum())
    return int((np.floor(s / 8.0) <= np.floor(s.max() / 8.0) - 32).sum())


@pytest.mark.parametrize("case", FAR_BUDGET_CASES, ids=[f"n{c[0]:.0f}_N{c[2]}" for c in FAR_BUDGET_CASES])
def test_decode_topk_far_boundary(case):
    """A fixed budget whose k-th score lies far below the max: one needle high above
    a background of scores spread evenly over [-a, a].  The fine 16-unit window
    misses the boundary, the coarse one (or, past 128 units, its tail) holds the
    candidates; the sizes put the candidate list in each resolver path."""
    needle, a, N, k, (c_lo, c_hi) = case
    wl = W.random_decode(71, 1, 8, 1, N, [0], 512)
    kc, vc, idx = O.caches_for(wl)
    rng = np.random.default_rng(72)
    qi0 = O.query_index(wl.q_pre[0, 0], wl.w_q[0]).astype(np.float64)
    u = qi0 / (qi0 @ qi0)
    target = rng.uniform(-a, a, wl.N)
    target[N // 3] = needle
    rows = target[:, None] * u[None, :] + 1e-3 * rng.standard_normal((wl.N, 16))
    idx = idx.copy()
    idx[0, 0] = O.f64_to_bf16(rows)
    s0 = O.scores(O.query_index(wl.q_pre[0, 0], wl.w_q[0]), idx[0, 0]).astype(np.float64)
    kth = np.sort(s0)[::-1][k - 1]
    assert s0.max() - kth > 16
    n_cand = _far_candidates(s0, k)
    assert c_lo <= n_cand <= c_hi, n_cand
    res = P.Device(wl, kc, vc, idx).decode(0.9, debug_cap=wl.N, top_k=k)
    ref = O.decode(wl, kc, vc, idx, 0.9, top_k=k)
    kinds = {}
    for (b, h), r in ref.items():
        S = P.gpu_set(res, h)
        kind = P.check_set_topk(S, r, k, wl.n_sink)
        kinds[kind] = kinds.get(kind, 0) + 1
        qr = O.rope(P.bf16_f64(wl.q_pre[b, h]), N - 1, wl.rope_base)
        own = O.attention(qr, kc[b, 0][S], vc[b, 0][S], wl.attn_scale)
        P.check_out(res["out"][b, h], own, f"own set h{h}")
        P.check_out(res["out"][b, h], r["out"], f"h{h} ({kind})")
    print(f"needle {needle} N {N} top-{k}: head-0 candidates {n_cand}, {kinds}")


@pytest.mark.parametrize("case", [CASES[5], CASES[6], CASES[8]],
                         ids=[f"s{c[0]}_N{c[4]}_G{c[2] // c[3]}" for c in (CASES[5], CASES[6], CASES[8])])
@pytest.mark.parametrize("top_p", [0.5, 0.9, 0.999, 1.0])
def test_three_launch_path_matches_fused(case, top_p, monkeypatch):
    """The scan, threshold and select kernels in turn (the path for grids that do not
    fit the GPU at once) give the fused pass's sets and outputs bit for bit, and both
    meet the oracle."""
    seed, B, Hq, Hkv, N, ret, window, needles, qs = case
    wl = W.random_decode(seed, B, Hq, Hkv, N, ret, window, n_needles=needles, q_scale=qs)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx, max_seq=N + 7)
    fused = dev.decode(top_p, debug_cap=N)
    monkeypatch.setenv("RTP_DECODE_PASSES", "3")
    three = dev.decode(top_p, debug_cap=N)
    assert np.array_equal(fused["out"], three["out"])
    assert np.array_equal(fused["cnt"], three["cnt"]) and np.array_equal(fused["tau"], three["tau"])
    for u in range(len(fused["cnt"])):
        assert np.array_equal(P.gpu_set(fused, u), P.gpu_set(three, u))
    P.compare_decode(wl, kc, vc, idx, three, top_p)


def test_fused_pass_leaves_no_error_and_counters_at_rest():
    """After fused decodes of several shapes on one workspace, the give-up word is zero
    and every counter of the counter region is back at zero."""
    import sparse_attention_long_retrieval_amd as R
    wls = [W.random_decode(47, 1, 8, 2, n, [0], 256, n_needles=2, q_scale=1.5)
           for n in (40000, 2049, 300000)]
    ws = None
    for wl in wls:
        kc, vc, idx = O.caches_for(wl)
        dev = P.Device(wl, kc, vc, idx)
        need = R.workspace_size(dev.layer, R.OP_DECODE, wl.N)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device="cuda")
        res = dev.decode(0.9, debug_cap=wl.N, ws=ws)
        P.compare_decode(wl, kc, vc, idx, res, 0.9)
        counters = ws[:65536].view(torch.int32).cpu().numpy()
        assert not counters.any(), np.nonzero(counters)[0][:8]


def test_fused_wait_give_up_raises_the_error_word(monkeypatch):
    """Capped at one poll (RTP_DECODE_SPIN_LIMIT, a test hook), the blocks that do not
    see their threshold at once give up: every kernel ends, the call's give-up word is
    set, and after the documented zero-fill of the counter region the same workspace
    gives the oracle's results again."""
    import sparse_attention_long_retrieval_amd as R
    wl = W.random_decode(71, 1, 8, 2, 300000, [0], 256, n_needles=2, q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    ws = torch.zeros(R.workspace_size(dev.layer, R.OP_DECODE, wl.N), dtype=torch.uint8,
                     device="cuda")
    monkeypatch.setenv("RTP_DECODE_SPIN_LIMIT", "1")
    dev.decode(0.9, ws=ws)
    err = ws[65532:65536].view(torch.int32).item()
    assert err == 1, "no wait gave up at one poll"
    monkeypatch.delenv("RTP_DECODE_SPIN_LIMIT")
    ws[:65536].zero_()
    res = dev.decode(0.9, debug_cap=wl.N, ws=ws)
    assert ws[65532:65536].view(torch.int32).item() == 0
    assert not ws[:65536].view(torch.int32).cpu().numpy().any()
    P.compare_decode(wl, kc, vc, idx, res, 0.9)
