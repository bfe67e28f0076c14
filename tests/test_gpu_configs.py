"""GPU parity at the full sizes of the decode workloads (the launch configuration
bench.py times): every retrieval q-head's selected set and output, and every
local head's output, against the oracle on the same bytes."""
import numpy as np
import pytest

import workloads as W
from oracle import rtp_oracle as O
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _caches(wl):
    N = wl.N
    lo = max(0, N - wl.window)
    win = np.union1d(np.arange(lo, N), np.arange(min(wl.n_sink, N)))
    rows = {kv: (None if kv in wl.ret_kv_heads else win) for kv in range(wl.Hkv)}
    return O.caches_for(wl, rows_needed=rows)


def _check(wl, ps):
    kc, vc, idx = _caches(wl)
    dev = P.Device(wl, kc, vc, idx)
    for p in ps:
        res = dev.decode(p, debug_cap=1 << 16)
        summ = P.compare_decode(wl, kc, vc, idx, res, p)
        sizes = res["cnt"].tolist()
        print(wl.name, "p", p, summ, "set sizes", sizes)


def test_million_decode():
    _check(W.make(4), [0.9])


def test_qwen3_8b_decode_64k():
    _check(W.make(2), [0.9])


def test_variable_budget_128k():
    wl = W.make(3)
    _check(wl, wl.top_p)
