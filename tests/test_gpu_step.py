"""GPU parity of the whole-layer decode step (rtp_decode_step): retrieval q-heads by
dynamic top-p and local q-heads over sinks + window, in one call.

Retrieval outputs and sets must equal the separate retrieval decode bit for bit;
local outputs meet the oracle (their window segments differ from the local-head
kernel's, so only rounding may differ from it).  Rings and the full cache give the
same bits, and so does the path that runs the index passes as separate launches.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rtp_oracle as O
from tests import _parity as P

pytestmark = pytest.mark.gpu
R = P.R

CASES = [
    # seed, B, Hq, Hkv, N, ret, window, needles, q_scale, n_sink
    (61, 1, 2, 2, 3, [1], 2, 0, 1.0, 4),
    (62, 2, 4, 2, 5, [0], 3, 0, 1.0, 4),
    (63, 1, 8, 2, 511, [0], 100, 3, 1.0, 4),
    (64, 2, 16, 4, 4099, [1, 2], 300, 4, 1.0, 4),
    (65, 1, 8, 8, 6149, [0, 3, 7], 2048, 2, 2.0, 4),
    (66, 1, 32, 4, 40000, [0], 8192, 2, 1.5, 4),
    (67, 3, 16, 4, 9000, [2], 700, 1, 1.0, 0),
]


def _rings(wl, kc, vc, ring_len):
    """Local heads' rings filled from the cache rows of the window and the sinks."""
    loc = [h for h in range(wl.Hkv) if h not in wl.ret_kv_heads]
    kr = np.zeros((wl.B, len(loc), wl.n_sink + ring_len, 128), dtype=np.uint16)
    vr = np.zeros_like(kr)
    lo = max(0, wl.N - ring_len)
    for li, kv in enumerate(loc):
        for j in list(range(min(wl.n_sink, wl.N))) + list(range(max(lo, wl.n_sink), wl.N)):
            r = j if j < wl.n_sink else wl.n_sink + (j - wl.n_sink) % ring_len
            kr[:, li, r] = kc[:, kv, j]
            vr[:, li, r] = vc[:, kv, j]
    return P.to_dev(kr), P.to_dev(vr)


def _step(dev, wl, top_p, ring=None, debug_cap=0):
    out = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.int16, device="cuda")
    ws = torch.zeros(max(256, R.workspace_size(dev.layer, R.OP_DECODE_STEP, wl.N)),
                     dtype=torch.uint8, device="cuda")
    dbg = R.Debug(wl.B * wl.n_ret * wl.G, debug_cap) if debug_cap else None
    if ring is None:
        R.decode_step(dev.layer, dev.q, dev.w_q, dev.kc, dev.vc, dev.idx, wl.N, top_p, out, ws,
                      debug=dbg)
    else:
        ring_len, kr, vr = ring
        R.decode_step(dev.layer, dev.q, dev.w_q, dev.kc, dev.vc, dev.idx, wl.N, top_p, out, ws,
                      ring_len=ring_len, k_ring=kr, v_ring=vr, debug=dbg)
    torch.cuda.synchronize()
    res = {"out": P.from_dev(out)}
    if dbg is not None:
        res["cnt"] = dbg.sel_count.cpu().numpy()
        res["idx"] = dbg.sel_idx.cpu().numpy()
        res["tau"] = dbg.tau.cpu().numpy()
    counters = ws[:65536].view(torch.int32).cpu().numpy()
    assert not counters.any(), f"counters not at rest: {np.nonzero(counters)[0][:8]}"
    return res


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_N{c[4]}_G{c[2] // c[3]}" for c in CASES])
@pytest.mark.parametrize("top_p", [0.5, 0.9, 1.0])
def test_step_matches_separate_calls_and_oracle(case, top_p, monkeypatch):
    seed, B, Hq, Hkv, N, ret, window, needles, qs, n_sink = case
    wl = W.random_decode(seed, B, Hq, Hkv, N, ret, window, n_needles=needles, q_scale=qs,
                         n_sink=n_sink)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    sep = dev.decode(top_p, debug_cap=N)
    step = _step(dev, wl, top_p, debug_cap=N)
    rq = wl.ret_q_heads()
    assert np.array_equal(step["out"][:, rq], sep["out"][:, rq]), "retrieval rows differ"
    assert np.array_equal(step["cnt"], sep["cnt"]) and np.array_equal(step["tau"], sep["tau"])
    for u in range(len(sep["cnt"])):
        assert np.array_equal(P.gpu_set(step, u), P.gpu_set(sep, u))
    summ = P.compare_decode(wl, kc, vc, idx, step, top_p)
    print(case, top_p, summ)
    # local heads from rings of the window: the same bits
    ring = (window,) + _rings(wl, kc, vc, window)
    ring_res = _step(dev, wl, top_p, ring=ring)
    assert np.array_equal(ring_res["out"], step["out"]), "ring step differs from full-cache step"
    # the index passes as separate launches (local-head kernel after them): the same bits
    monkeypatch.setenv("RTP_DECODE_PASSES", "3")
    three = _step(dev, wl, top_p)
    bad = sorted({int(h) for h in np.nonzero((three["out"] != step["out"]).any(-1))[1]})
    assert not bad, f"three-launch step differs on q-heads {bad} (retrieval {rq})"


def test_step_million_shaped_layer():
    """A 2^17-token layer shaped like the 1M configuration (32 q / 4 KV heads, one
    retrieval head, rings of the 8192 window): local rows against the oracle on sampled
    heads, retrieval rows equal to the separate decode."""
    wl = W.clustered_decode("step_131k", 1007, 1, 32, 4, 1 << 17, [0], 64)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    sep = dev.decode(0.9, debug_cap=wl.N)
    ring = (wl.window,) + _rings(wl, kc, vc, wl.window)
    step = _step(dev, wl, 0.9, ring=ring, debug_cap=wl.N)
    rq = wl.ret_q_heads()
    assert np.array_equal(step["out"][:, rq], sep["out"][:, rq])
    heads = [8, 13, 21, 31]
    ref = O.decode(wl, kc, vc, idx, 0.9, heads=heads)
    for (b, h), r in ref.items():
        P.check_out(step["out"][b, h], r["out"], f"local b{b} h{h}")


@pytest.mark.parametrize("ret", [[], [0, 1, 2, 3]], ids=["local_only", "retrieval_only"])
def test_step_with_one_kind_of_head(ret):
    """A layer of local heads only runs the local-head kernel; a layer of retrieval heads
    only gives the retrieval decode's bits."""
    wl = W.random_decode(68, 2, 16, 4, 3000, ret, 500, n_needles=2 if ret else 0, n_sink=4)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    step = _step(dev, wl, 0.9, debug_cap=wl.N if ret else 0)
    if ret:
        sep = dev.decode(0.9, debug_cap=wl.N)
        assert np.array_equal(step["out"], sep["out"])
    else:
        ring = (wl.window,) + _rings(wl, kc, vc, wl.window)
        assert np.array_equal(_step(dev, wl, 0.9, ring=ring)["out"], step["out"])
    P.compare_decode(wl, kc, vc, idx, step, 0.9)


def test_step_graph_replay_matches_eager():
    """Append + rtp_decode_step captured in one HIP graph gives the eager step's bits on
    every replay, with other decode steps and torch work between the replays."""
    wl = W.random_decode(69, 1, 32, 4, 60000, [0], 8192, n_needles=2, q_scale=1.5)
    kc, vc, idx = O.caches_for(wl)
    dev = P.Device(wl, kc, vc, idx)
    N = wl.N
    new_k = P.to_dev(wl.k_pre[:, :, N - 1:N])
    new_v = P.to_dev(wl.v[:, :, N - 1:N])
    w_k = P.to_dev(wl.w_k)
    out = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.int16, device="cuda")
    ws = torch.zeros(R.workspace_size(dev.layer, R.OP_DECODE_STEP, N), dtype=torch.uint8,
                     device="cuda")

    def step(p=0.9, o=out):
        R.index_append(dev.layer, new_k, new_v, w_k, N - 1, dev.kc, dev.vc, dev.idx)
        R.decode_step(dev.layer, dev.q, dev.w_q, dev.kc, dev.vc, dev.idx, N, p, o, ws)

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
        step(0.5, other)
        torch.cuda.synchronize()
        _ = (other.float() * 2).sum().item()
    assert not ws[:65536].view(torch.int32).cpu().numpy().any()
    ref = O.decode(wl, kc, vc, idx, 0.9)
    got = P.from_dev(out)
    for (b, h), r in ref.items():
        P.check_out(got[b, h], r["out"], f"graph b{b} h{h}")
