"""GPU parity of the chunked-prefill local-head attention (causal window + sinks,
MFMA flash tiles) against the oracle, on the oracle's own cache bytes.

Outputs are compared element by element with the tolerance of tests/_parity.py
(max-abs 1e-2, bf16 output, fp32 accumulation; the kernel also rounds q and the
probabilities to bf16 for the matrix cores, which moves logits by ~1e-3).
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




def _local_rows_needed(wl, rows):
    """KV rows the oracle needs for local heads at the given chunk rows."""
    pos = wl.q_start + np.asarray(rows)
    need = [np.arange(max(0, p - wl.window + 1), p + 1) for p in pos]
    need.append(np.arange(min(wl.n_sink, wl.N)))
    u = np.unique(np.concatenate(need))
    return {kv: u for kv in range(wl.Hkv) if kv not in wl.ret_kv_heads}


def _swa_chunk(wl, kc, vc, max_seq=None):
    dev = P.Device(wl, kc, vc, np.zeros((wl.B, max(1, wl.n_ret), wl.N, 16), np.uint16),
                   max_seq=max_seq)
    out = torch.zeros((wl.B, wl.Hq, wl.Tq, 128), dtype=torch.int16, device="cuda")
    assert R.workspace_size(dev.layer, R.OP_SWA, wl.N, Tq=wl.Tq) == 0
    R.swa_attn(dev.layer, dev.q, wl.q_start, wl.Tq, dev.kc, dev.vc, out)
    torch.cuda.synchronize()
    return P.from_dev(out)


def _check_rows(wl, kc, vc, out_bits, rows):
    worst = 0.0
    for b in range(wl.B):
        for h in wl.local_q_heads():
            kv = h // wl.G
            for t in rows:
                ref = O.local_head(wl.q_pre[b, h, t], kc[b, kv], vc[b, kv], wl.q_start + t,
                                   wl.window, wl.n_sink, wl.attn_scale, wl.rope_base)["out"]
                err = P.check_out(out_bits[b, h, t], ref, f"b{b} h{h} row {t}")
                worst = max(worst, err)
    return worst


CASES = [
    # (seed, B, Hq, Hkv, N, Tq, ret_kv, window, n_sink)
    (11, 1, 4, 2, 1500, 300, [0], 256, 4),        # ragged tail, window inside the chunk
    (12, 1, 8, 2, 900, 200, [1], 4096, 4),        # window longer than the context: causal
    (13, 1, 4, 1, 200, 200, [], 64, 4),           # first chunk: rows near 0, sinks in window
    (14, 2, 16, 2, 700, 129, [], 100, 0),         # no sinks, G = 8, B = 2, one spill row
    (15, 1, 2, 2, 600, 130, [0], 1, 4),           # window 1: self + sinks
    (16, 1, 4, 4, 3000, 640, [0, 2], 512, 7),     # more sinks than 4, several row blocks
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_swa_prefill_small(case):
    seed, B, Hq, Hkv, N, Tq, ret, window, n_sink = case
    wl = W.random_prefill(seed, B, Hq, Hkv, N, Tq, ret, window, n_sink=n_sink)
    kc, vc, _ = O.caches_for(wl)
    out = _swa_chunk(wl, kc, vc)
    worst = _check_rows(wl, kc, vc, out, range(Tq))
    print(f"{wl.name}: worst |err| {worst:.3g}")


def test_swa_prefill_max_seq_padding():
    """Caches longer than the context (max_seq > N): keys past the chunk are never read."""
    wl = W.random_prefill(17, 1, 4, 2, 800, 150, [0], 300)
    kc, vc, _ = O.caches_for(wl)
    out = _swa_chunk(wl, kc, vc, max_seq=wl.N + 77)
    _check_rows(wl, kc, vc, out, range(wl.Tq))


def test_swa_prefill_deterministic():
    wl = W.random_prefill(18, 1, 4, 2, 1200, 256, [0], 333)
    kc, vc, _ = O.caches_for(wl)
    a = _swa_chunk(wl, kc, vc)
    b = _swa_chunk(wl, kc, vc)
    assert np.array_equal(a, b)


def test_swa_prefill_chunked_256k_sampled():
    """Chunked prefill at 256K (4096-row chunk at the end of 262,144 keys, 24 local
    q-heads, window 8192 + 4 sinks): the full chunk on the GPU, sampled rows checked."""
    wl = W.make(5)
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 31, 32, 127, 128, 2047, 4094, 4095] +
                      rng.integers(0, wl.Tq, 7).tolist()))
    kc, vc, _ = O.caches_for(wl, rows_needed=_local_rows_needed(wl, rows))
    out = _swa_chunk(wl, kc, vc)
    worst = _check_rows(wl, kc, vc, out, rows)
    print(f"chunked_prefill_256k local heads: worst |err| {worst:.3g}")


# ---------------------------------------------------------------- retrieval heads

def _prefill_retrieval(wl, kc, vc, idx, top_p, cap, idx_scale=1.0, max_seq=None, units=None):
    dev = P.Device(wl, kc, vc, idx, max_seq=max_seq)
    out = torch.zeros((wl.B, wl.Hq, wl.Tq, 128), dtype=torch.int16, device="cuda")
    nbytes = R.workspace_size(dev.layer, R.OP_PREFILL, wl.N, Tq=wl.Tq)
    ws = torch.empty(max(256, nbytes), dtype=torch.uint8, device="cuda")
    V = wl.B * wl.n_ret * wl.G * wl.Tq
    dbg = R.Debug(V, cap, pairs=wl.B * wl.n_ret)
    R.prefill_chunk(dev.layer, dev.q, wl.q_start, dev.w_q, dev.kc, dev.vc, dev.idx, top_p, out,
                    ws, idx_scale=idx_scale, debug=dbg)
    torch.cuda.synchronize()
    if units is None:
        # the union count of each (batch, retrieval KV head) pair is the number of
        # distinct keys in the sets of all its rows and q-heads
        cnt = dbg.sel_count.cpu().numpy()
        sel = dbg.sel_idx.cpu().numpy()
        per = wl.G * wl.Tq
        for pr, u in enumerate(dbg.union_count.cpu().numpy()):
            keys = np.concatenate([sel[v, :min(cnt[v], cap)] for v in range(pr * per, (pr + 1) * per)])
            assert int(u) == len(np.unique(keys)), (pr, int(u), len(np.unique(keys)))
    if units is None:
        sel = dbg.sel_idx.cpu().numpy()
    else:  # only the sampled entries come back to the host
        u = torch.tensor(sorted(units), dtype=torch.long, device="cuda")
        rows = dbg.sel_idx.index_select(0, u).cpu().numpy()
        sel = {int(k): rows[n] for n, k in enumerate(sorted(units))}
    res = {"idx": sel, "cnt": dbg.sel_count.cpu().numpy(),
           "tau": dbg.tau.cpu().numpy(), "out": P.from_dev(out), "cap": cap}
    return res


def _gpu_set(res, unit):
    c = int(res["cnt"][unit])
    assert c <= res["cap"], f"debug capacity {res['cap']} < set size {c}"
    return np.sort(np.asarray(res["idx"][unit][:c], dtype=np.int64))


def _check_retrieval(wl, kc, vc, idx, res, top_p, rows, idx_scale=1.0):
    kinds = {}
    worst = 0.0
    for b in range(wl.B):
        for i, kv in enumerate(wl.ret_kv_heads):
            for g in range(wl.G):
                h = kv * wl.G + g
                for t in rows:
                    unit = ((b * wl.n_ret + i) * wl.G + g) * wl.Tq + t
                    r = O.retrieval_head(wl.q_pre[b, h, t], wl.w_q[i * wl.G + g], kc[b, kv],
                                         vc[b, kv], idx[b, i], wl.q_start + t, top_p,
                                         wl.n_sink, idx_scale, wl.attn_scale, wl.rope_base)
                    S = _gpu_set(res, unit)
                    kind = P.check_set(S, res["tau"][unit], r, top_p, wl.n_sink)
                    kinds[kind] = kinds.get(kind, 0) + 1
                    # attention over the GPU's own set (the attention step alone), and
                    # the output end to end against the oracle's, whatever the set kind
                    qr = O.rope(O.bf16_to_f64(wl.q_pre[b, h, t]), wl.q_start + t, wl.rope_base)
                    own = O.attention(qr, kc[b, kv][S], vc[b, kv][S], wl.attn_scale)
                    err = P.check_out(res["out"][b, h, t], own, f"own set b{b} h{h} t{t}")
                    err = max(err, P.check_out(res["out"][b, h, t], r["out"],
                                               f"b{b} h{h} row {t} ({kind})"))
                    worst = max(worst, err)
    return kinds, worst


RCASES = [
    # (seed, B, Hq, Hkv, N, Tq, ret_kv, n_sink)
    (31, 1, 4, 2, 2500, 200, [0], 4),        # G = 2, ragged row blocks
    (32, 1, 8, 2, 1200, 1200, [1], 4),       # first chunk (q_start = 0), G = 4
    (33, 2, 16, 2, 3000, 96, [0, 1], 4),     # B = 2, G = 8, two retrieval heads
    (34, 1, 4, 4, 5000, 130, [2], 0),        # no sinks, G = 1
    (35, 1, 4, 1, 700, 300, [0], 40),        # many sinks (a whole 32-key block and more)
]


@pytest.mark.parametrize("top_p", [0.9, 0.5, 0.999, 1e-6, 1.0])
@pytest.mark.parametrize("case", RCASES, ids=[f"s{c[0]}" for c in RCASES])
def test_prefill_retrieval_small(case, top_p):
    seed, B, Hq, Hkv, N, Tq, ret, n_sink = case
    wl = W.random_prefill(seed, B, Hq, Hkv, N, Tq, ret, 256, n_sink=n_sink)
    kc, vc, idx = O.caches_for(wl)
    res = _prefill_retrieval(wl, kc, vc, idx, top_p, cap=N)
    kinds, worst = _check_retrieval(wl, kc, vc, idx, res, top_p, range(Tq))
    print(f"{wl.name} p={top_p}: {kinds} worst |err| {worst:.3g}")


def _same_result(a, b, V):
    """Two runs of one chunk select the same sets and write the same output bits."""
    assert np.array_equal(a["cnt"], b["cnt"])
    assert np.array_equal(a["tau"], b["tau"])
    for v in range(V):
        c = int(a["cnt"][v])
        assert np.array_equal(np.sort(a["idx"][v][:c]), np.sort(b["idx"][v][:c])), v
    assert np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("slots", ["0", "1000"])
@pytest.mark.parametrize("top_p", [0.9, 0.999])
@pytest.mark.parametrize("case", RCASES[1:3], ids=[f"s{c[0]}" for c in RCASES[1:3]])
def test_prefill_retrieval_recomputed_scores(monkeypatch, case, top_p, slots):
    """Vectors past the resolver's score slots compute their candidates' scores again in
    every pass (RTP_PREFILL_SCORE_SLOTS caps the slots: 0 sends every vector that way,
    1000 the vectors after the first few): the same thresholds, sets and output bits as
    with every vector in the slots, and parity with the oracle."""
    seed, B, Hq, Hkv, N, Tq, ret, n_sink = case
    wl = W.random_prefill(seed, B, Hq, Hkv, N, Tq, ret, 256, n_sink=n_sink)
    kc, vc, idx = O.caches_for(wl)
    base = _prefill_retrieval(wl, kc, vc, idx, top_p, cap=N)
    monkeypatch.setenv("RTP_PREFILL_SCORE_SLOTS", slots)
    res = _prefill_retrieval(wl, kc, vc, idx, top_p, cap=N)
    _same_result(base, res, wl.B * wl.n_ret * wl.G * wl.Tq)
    kinds, worst = _check_retrieval(wl, kc, vc, idx, res, top_p, range(Tq))
    print(f"{wl.name} p={top_p} slots={slots}: {kinds} worst |err| {worst:.3g}")


def test_prefill_retrieval_ties():
    """q = 0 gives qi = 0: every score ties at 0, so every key is selected (ties at the
    threshold are included).  The boundary bin holds every key: each candidate word is
    full, and the resolver's range collapses to one key."""
    wl = W.random_prefill(36, 1, 4, 2, 3000, 64, [0], 256)
    wl.q_pre[:] = 0
    kc, vc, idx = O.caches_for(wl)
    res = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=wl.N)
    kinds, _ = _check_retrieval(wl, kc, vc, idx, res, 0.9, range(wl.Tq))
    assert set(kinds) == {"exact"}


def test_prefill_retrieval_idx_scale_and_padding():
    wl = W.random_prefill(37, 1, 4, 2, 1500, 100, [0], 256)
    kc, vc, idx = O.caches_for(wl)
    res = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=wl.N, idx_scale=0.25, max_seq=wl.N + 40)
    _check_retrieval(wl, kc, vc, idx, res, 0.9, range(wl.Tq), idx_scale=0.25)


def test_prefill_retrieval_deterministic():
    wl = W.random_prefill(38, 1, 4, 2, 2000, 128, [0], 256)
    kc, vc, idx = O.caches_for(wl)
    a = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=wl.N)
    b = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=wl.N)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["cnt"], b["cnt"])


def test_prefill_retrieval_split_items():
    """Near-flat scores (q scaled by 1/32) select most of 40K keys: those vectors have far
    more than 256 words (definite and candidate: the scores span little more than a
    boundary bin), so the attend cuts them into work items and merges the partial
    results.  Two rows keep their clustered queries (smaller sets) in the same call."""
    wl = W.random_prefill(39, 1, 4, 2, 40000, 8, [0], 256)
    q = W.bf16_bits_to_f32(wl.q_pre)
    q[:, :, :6] *= np.float32(1.0 / 32.0)
    wl.q_pre = W.f32_to_bf16_bits(q)
    kc, vc, idx = O.caches_for(wl)
    res = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=wl.N)
    kinds, _ = _check_retrieval(wl, kc, vc, idx, res, 0.9, range(wl.Tq))
    cnt = res["cnt"].reshape(wl.B * wl.n_ret * wl.G, wl.Tq)
    # more rows than 256 full words of 32 keys: more than 256 words, so cut
    assert (cnt[:, :6] > 256 * 32 + wl.n_sink).all(), cnt
    print(f"split items: {kinds}, set sizes {cnt.tolist()}")


def test_prefill_retrieval_chunked_256k_sampled():
    """Chunked prefill at 256K: the whole 4096-row chunk of both retrieval KV heads (8
    retrieval q-heads) on the GPU, sets and outputs of sampled rows against the oracle."""
    wl = W.make(5)
    rng = np.random.default_rng(55)
    rows = sorted(set([0, 1, 63, 64, 2048, 4095] + rng.integers(0, wl.Tq, 4).tolist()))
    kc, vc, idx = O.caches_for(wl, rows_needed={kv: np.arange(0) for kv in range(wl.Hkv)
                                                 if kv not in wl.ret_kv_heads})
    units = [((b * wl.n_ret + i) * wl.G + g) * wl.Tq + t for b in range(wl.B)
             for i in range(wl.n_ret) for g in range(wl.G) for t in rows]
    res = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=65536, units=units)
    kinds, worst = _check_retrieval(wl, kc, vc, idx, res, 0.9, rows)
    sizes = [int(res["cnt"][u]) for u in range(0, len(res["cnt"]), 997)]
    print(f"chunked_prefill_256k retrieval: {kinds} worst |err| {worst:.3g} "
          f"sample set sizes {sizes[:12]}")


@pytest.fixture(scope="module")
def million_chunk():
    """The 1M-context chunk and the oracle caches its sampled rows need."""
    wl = W.make(6)
    rng = np.random.default_rng(66)
    rows = sorted(set([0, 1, 2048, 4095] + rng.integers(0, wl.Tq, 2).tolist()))
    kc, vc, idx = O.caches_for(wl, rows_needed=_local_rows_needed(wl, rows))
    return wl, rows, kc, vc, idx


@pytest.mark.timeout(900)
def test_prefill_retrieval_chunked_1m_sampled(million_chunk):
    """Chunked prefill at 1M context (a 4096-row chunk at the end of 2^20 keys, 8
    retrieval q-heads): the workspace the call asks for fits the GPU with room to
    spare (below 24 GiB of 288 GB: mostly the definite and candidate word lists, each
    able to hold every 32-key block of an index wave's range, 8 GiB apiece), the whole
    chunk runs, and the sets and outputs of sampled rows of every retrieval q-head
    match the oracle."""
    wl, rows, kc, vc, idx = million_chunk
    layer = R.Layer(wl.B, wl.Hq, wl.Hkv, wl.N, wl.ret_kv_heads, wl.n_sink, wl.window)
    nbytes = R.workspace_size(layer, R.OP_PREFILL, wl.N, Tq=wl.Tq)
    assert nbytes < 24 << 30, nbytes
    units = [((b * wl.n_ret + i) * wl.G + g) * wl.Tq + t for b in range(wl.B)
             for i in range(wl.n_ret) for g in range(wl.G) for t in rows]
    res = _prefill_retrieval(wl, kc, vc, idx, 0.9, cap=1 << 18, units=units)
    kinds, worst = _check_retrieval(wl, kc, vc, idx, res, 0.9, rows)
    assert kinds.get("valid-alt", 0) == 0
    print(f"chunked_prefill_1m retrieval: workspace {nbytes / 2**30:.2f} GiB, {kinds}, "
          f"worst |err| {worst:.3g}, sampled set sizes {[int(res['cnt'][u]) for u in units]}")


@pytest.mark.timeout(600)
def test_swa_prefill_chunked_1m_sampled(million_chunk):
    """The local heads of the same 1M-context chunk (24 q-heads, window 8192 + 4
    sinks): the full chunk on the GPU, sampled rows against the oracle."""
    wl, rows, kc, vc, _ = million_chunk
    out = _swa_chunk(wl, kc, vc)
    worst = _check_rows(wl, kc, vc, out, rows)
    print(f"chunked_prefill_1m local heads: worst |err| {worst:.3g}")
