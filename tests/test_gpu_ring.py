"""GPU parity of the local-head ring caches (rtp_ring_append / rtp_swa_attn_ring).

The ring is storage only: attention through it must be bit-identical to the same
kernels over a full cache holding the same rows, and match the oracle's sliding
window + sink attention (tolerance of tests/_parity.py).  The rings here wrap
around several times before the measured rows.
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

CASES = [
    # (seed, B, Hq, Hkv, N, Tq, ret_kv, window, n_sink)
    (61, 1, 8, 4, 3000, 300, [1], 256, 4),
    (62, 2, 16, 2, 2500, 129, [0], 300, 0),     # G = 8, B = 2, no sinks
    (63, 1, 4, 4, 4000, 64, [0, 3], 1000, 7),   # two retrieval heads, more sinks
]


def _fill(wl, layer, ring_len, step):
    """Full caches (rtp_index_append) and rings (rtp_ring_append) fed the same tokens in
    chunks of `step`, then the query chunk."""
    B, Hkv, N = wl.B, wl.Hkv, wl.N
    n_loc = Hkv - wl.n_ret
    k_pre, v = P.to_dev(wl.k_pre), P.to_dev(wl.v)
    w_k = P.to_dev(wl.w_k)
    kc = torch.zeros((B, Hkv, N, 128), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    idx = torch.zeros((B, max(1, wl.n_ret), N, 16), dtype=torch.int16, device="cuda")
    kr = torch.zeros((B, n_loc, wl.n_sink + ring_len, 128), dtype=torch.int16, device="cuda")
    vr = torch.zeros_like(kr)
    bounds = list(range(0, wl.q_start, step)) + [wl.q_start, N]
    for a, c in zip(bounds[:-1], bounds[1:]):
        if c <= a:
            continue
        kp, vp = k_pre[:, :, a:c].contiguous(), v[:, :, a:c].contiguous()
        R.index_append(layer, kp, vp, w_k, a, kc, vc, idx)
        R.ring_append(layer, kp, vp, a, ring_len, kr, vr)
    return kc, vc, kr, vr


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_ring_matches_full_cache_and_oracle(case):
    seed, B, Hq, Hkv, N, Tq, ret, window, n_sink = case
    wl = W.random_prefill(seed, B, Hq, Hkv, N, Tq, ret, window, n_sink=n_sink)
    layer = R.Layer(B, Hq, Hkv, N, ret, n_sink, window, wl.rope_base)
    ring_len = window + Tq - 1
    kc, vc, kr, vr = _fill(wl, layer, ring_len, step=min(ring_len, 500))
    q = P.to_dev(wl.q_pre)
    loc = wl.local_q_heads()
    # the chunk (causal window attention over Tq rows)
    out_f = torch.zeros((B, Hq, Tq, 128), dtype=torch.int16, device="cuda")
    out_r = torch.zeros_like(out_f)
    R.swa_attn(layer, q, wl.q_start, Tq, kc, vc, out_f)
    R.swa_attn_ring(layer, q, wl.q_start, Tq, ring_len, kr, vr, out_r)
    # decode at the last position
    qd = q[:, :, Tq - 1].contiguous()
    ws = torch.zeros(R.workspace_size(layer, R.OP_SWA, N), dtype=torch.uint8, device="cuda")
    dec_f = torch.zeros((B, Hq, 128), dtype=torch.int16, device="cuda")
    dec_r = torch.zeros_like(dec_f)
    R.swa_attn(layer, qd, N - 1, 1, kc, vc, dec_f, ws)
    R.swa_attn_ring(layer, qd, N - 1, 1, ring_len, kr, vr, dec_r, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_f[:, loc], out_r[:, loc]), "ring chunk differs from the full cache"
    assert torch.equal(dec_f[:, loc], dec_r[:, loc]), "ring decode differs from the full cache"
    # against the oracle, on the GPU's own cache rows
    kc_h, vc_h = P.from_dev(kc), P.from_dev(vc)
    got = P.from_dev(out_r)
    for b in range(B):
        for h in loc:
            kv = h // wl.G
            for t in range(Tq):
                ref = O.local_head(wl.q_pre[b, h, t], kc_h[b, kv], vc_h[b, kv], wl.q_start + t,
                                   window, n_sink, wl.attn_scale, wl.rope_base)["out"]
                P.check_out(got[b, h, t], ref, f"ring b{b} h{h} row {t}")


def test_ring_rows_hold_the_window():
    """After a wrap-around, every ring row holds exactly the token the mapping names."""
    wl = W.random_prefill(64, 1, 4, 2, 1500, 100, [0], 200, n_sink=4)
    layer = R.Layer(1, 4, 2, wl.N, [0], 4, 200, wl.rope_base)
    ring_len = 299
    kc, _, kr, _ = _fill(wl, layer, ring_len, step=150)
    kc_h, kr_h = P.from_dev(kc), P.from_dev(kr)
    last = wl.N - 1
    for row in range(4 + ring_len):
        if row < 4:
            tok = row
        else:  # the newest token j >= 4 with 4 + (j - 4) % ring_len == row
            tok = last - ((last - 4 - (row - 4)) % ring_len)
        assert np.array_equal(kr_h[0, 0, row], kc_h[0, 1, tok]), row
