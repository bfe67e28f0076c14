"""The allocation-free decode (rtp_decode_sparse_attn_noalloc) against the decode with
a caller workspace, through the C ABI: two calls in a row, the second on a smaller
input, then the first shape again (the shared scratch keeps the last call's contents),
each bit-identical to the workspace call and within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

import sparse_attention_long_retrieval_amd as R
import workloads as W
from oracle import rtp_oracle as O
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _noalloc(dev, top_p, cap):
    wl = dev.wl
    out = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.int16, device="cuda")
    dbg = R.Debug(wl.B * wl.n_ret * wl.G, cap)
    R.decode_sparse_attn_noalloc(dev.layer, dev.q, dev.w_q, dev.kc, dev.vc, dev.idx, wl.N,
                                 top_p, out, debug=dbg)
    return out, dbg


def test_noalloc_matches_workspace_decode():
    big = W.random_decode(71, 1, 16, 2, 70000, [0], 1024, n_needles=3, q_scale=1.5)
    small = W.random_decode(72, 2, 8, 2, 3000, [1], 256, n_needles=2, q_scale=2.0)
    cases = []
    for wl, p in ((big, 0.9), (small, 0.95)):
        kc, vc, idx = O.caches_for(wl)
        dev = P.Device(wl, kc, vc, idx)
        ref = dev.decode(p, debug_cap=wl.N)          # rtp_decode_sparse_attn + workspace
        cases.append((wl, p, kc, vc, idx, dev, ref))
    torch.cuda.synchronize()
    # the allocation-free calls back to back: big, then small, then big again
    runs = [(c, _noalloc(c[5], c[1], c[0].N)) for c in (cases[0], cases[1], cases[0])]
    torch.cuda.synchronize()
    for (wl, p, kc, vc, idx, dev, ref), (out, dbg) in runs:
        o = P.from_dev(out)
        G = wl.G
        ret_heads = [kv * G + g for kv in wl.ret_kv_heads for g in range(G)]
        assert np.array_equal(o[:, ret_heads], ref["out"][:, ret_heads]), wl.name
        res = {"out": o, "cnt": dbg.sel_count.cpu().numpy(), "idx": dbg.sel_idx.cpu().numpy(),
               "tau": dbg.tau.cpu().numpy()}
        assert np.array_equal(res["cnt"], ref["cnt"]) and np.array_equal(res["tau"], ref["tau"])
        for u in range(len(res["cnt"])):
            assert np.array_equal(P.gpu_set(res, u), P.gpu_set(ref, u))
        summ = P.compare_decode(wl, kc, vc, idx, res, p, heads=ret_heads, ret_only=True)
        print(wl.name, p, summ)
