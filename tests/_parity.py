"""Helpers of the GPU parity tests: upload seeded inputs, run the C ABI, compare
against the oracle.

Tolerances (stated once here, used by every GPU test):
  * selected sets: bit-exact except tokens whose oracle fp32 score lies within
    BAND_REL * max(|tau|, 1) of the oracle threshold tau ("band").
  * Beyond the band, a set may differ from the oracle's only by the run of
    rank-adjacent tokens between the two thresholds ("valid-alt"), and only for
    p > STRICT_P.  Such a set must be a threshold set (every key above its own
    threshold is in it, nothing below it is) whose oracle fp64 mass satisfies the
    top-p conditions within MASS_TOL relative:  mass(set) >= p Z (1 - MASS_TOL) and
    mass(keys strictly above its threshold) < p Z (1 + MASS_TOL).
    Where MASS_TOL comes from: qi is the fp32 rounding of the exact dot product on
    both sides, so the scores differ only by the fp32 accumulation of the matrix
    cores (one ulp on about a third of the keys, random sign, measured); the decode
    histogram rounds each key's weight to 2^-20 of its bin edge (at most 2^-21 of
    the weight) and exp2 adds about 1e-7.  The slack of a crossing is the weighted
    sum of these per-key errors: the rounding terms are bounded by 2^-21 + 2.4e-7 =
    7.2e-7 of the mass whatever the rows (reached when one key holds nearly all of
    it), and the score term is a sum of independent signed errors of order
    2e-6 / sqrt(n_eff), n_eff = Z^2 / sum(w^2), which is what lets a diffuse row at
    p close to 1 end one or two keys earlier or later.  MASS_TOL = 1e-6 covers the
    first bound and several standard deviations of the second for n_eff >= 100.
    Observed: slack 7.5e-7 for a needle over a flat background at p = 0.9999 (the
    bin rounding of the needle), about 1e-8 for diffuse prefill rows at p = 0.999,
    and no differing boundary at p <= 0.95.
  * outputs: |o_gpu - o_oracle| <= OUT_TOL (bf16 output, fp32 accumulation); for
    |o| >= 4, where half a bf16 ulp alone exceeds it, OUT_TOL + half an ulp; the
    outputs accepted only through that allowance are counted.
Every retrieval output is compared twice: against oracle attention over the GPU's
own set (the attention step alone) and end to end against the oracle's output.

Each test's counts (exact / band / valid-alt sets, tokens in the differences, the
largest mass slack, half-ulp acceptances) are collected in STATS and printed in the
pytest terminal summary (tests/conftest.py), also under -q.
"""
from __future__ import annotations

import math
import os
from typing import Dict, Optional

import numpy as np
import torch

import sparse_attention_long_retrieval_amd as R
from oracle import rtp_oracle as O

BAND_REL = 1e-5
MASS_TOL = 1e-6
STRICT_P = 0.95
OUT_TOL = 1e-2

# per test: counts of the set kinds and output acceptances
STATS: Dict[str, Dict[str, float]] = {}


def stats() -> Dict[str, float]:
    name = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    return STATS.setdefault(name, {"exact": 0, "band": 0, "valid-alt": 0, "band_tokens": 0,
                                   "alt_tokens": 0, "max_mass_slack": 0.0, "outputs": 0,
                                   "half_ulp_outputs": 0, "max_out_err": 0.0})


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_f64(bits):
    return O.bf16_to_f64(bits)


class Device:
    """One workload's caches and index resident on the GPU (oracle append output)."""

    def __init__(self, wl, kc: np.ndarray, vc: np.ndarray, idx: np.ndarray,
                 max_seq: Optional[int] = None):
        self.wl = wl
        self.max_seq = max_seq or wl.N
        B, Hkv, N, D = kc.shape
        self.layer = R.Layer(wl.B, wl.Hq, wl.Hkv, self.max_seq, wl.ret_kv_heads, wl.n_sink,
                             wl.window, wl.rope_base)
        if self.max_seq == N:
            self.kc, self.vc = to_dev(kc), to_dev(vc)
            self.idx = to_dev(idx) if wl.n_ret else torch.zeros(16, dtype=torch.int16,
                                                                 device="cuda")
        else:
            self.kc = torch.zeros((B, Hkv, self.max_seq, D), dtype=torch.int16, device="cuda")
            self.vc = torch.zeros_like(self.kc)
            self.kc[:, :, :N] = to_dev(kc)
            self.vc[:, :, :N] = to_dev(vc)
            self.idx = torch.zeros((B, max(1, wl.n_ret), self.max_seq, 16), dtype=torch.int16,
                                   device="cuda")
            if wl.n_ret:
                self.idx[:, :, :N] = to_dev(idx)
        self.q = to_dev(wl.q_pre)
        self.w_q = to_dev(wl.w_q) if wl.n_ret else torch.zeros(16, dtype=torch.int16,
                                                                 device="cuda")

    def decode(self, top_p: float, debug_cap: int = 0, idx_scale: float = 1.0, ws=None,
               wss=None, top_k: Optional[int] = None):
        wl = self.wl
        out = torch.zeros((wl.B, wl.Hq, 128), dtype=torch.int16, device="cuda")
        if ws is None:
            ws = torch.zeros(max(256, R.workspace_size(self.layer, R.OP_DECODE, wl.N)),
                             dtype=torch.uint8, device="cuda")
        dbg = R.Debug(wl.B * wl.n_ret * wl.G, debug_cap) if debug_cap else None
        if top_k is None:
            R.decode_sparse_attn(self.layer, self.q, self.w_q, self.kc, self.vc, self.idx, wl.N,
                                 top_p, out, ws, idx_scale=idx_scale, debug=dbg)
        else:
            R.decode_topk(self.layer, self.q, self.w_q, self.kc, self.vc, self.idx, wl.N,
                          top_k, out, ws, idx_scale=idx_scale, debug=dbg)
        if wss is None:
            wss = torch.zeros(max(256, R.workspace_size(self.layer, R.OP_SWA, wl.N)),
                              dtype=torch.uint8, device="cuda")
        R.swa_attn(self.layer, self.q, wl.N - 1, 1, self.kc, self.vc, out, wss)
        torch.cuda.synchronize()
        res = {"out": from_dev(out)}
        if dbg is not None:
            res["cnt"] = dbg.sel_count.cpu().numpy()
            res["idx"] = dbg.sel_idx.cpu().numpy()
            res["tau"] = dbg.tau.cpu().numpy()
        return res


def gpu_set(res, unit: int) -> np.ndarray:
    c = int(res["cnt"][unit])
    cap = res["idx"].shape[1]
    assert c <= cap, f"debug capacity {cap} < set size {c}"
    return np.sort(res["idx"][unit, :c].astype(np.int64))


def check_set(S_gpu: np.ndarray, tau_gpu: float, r: Dict, p: float, n_sink: int) -> str:
    """Compare a GPU set with the oracle's; return 'exact', 'band' or 'valid-alt'
    (see the module docstring for the rule) and count the outcome."""
    st = stats()
    n = len(r["scores"])
    if p >= 1.0:
        assert np.array_equal(S_gpu, np.arange(n)), "p=1 must keep every key"
        st["exact"] += 1
        return "exact"
    S_o = r["S"]
    if np.array_equal(S_gpu, S_o):
        st["exact"] += 1
        return "exact"
    s = r["scores"].astype(np.float64)
    tau = float(r["tau"])
    band = BAND_REL * max(abs(tau), 1.0)
    diff = np.setxor1d(S_gpu, S_o)
    if np.all(np.abs(s[diff] - tau) <= band):
        st["band"] += 1
        st["band_tokens"] += len(diff)
        return "band"
    # a different rank boundary: allowed only close to p = 1, as the run of
    # rank-adjacent keys between the two thresholds, under the mass tolerance
    outside = diff[np.abs(s[diff] - tau) > band]
    assert p > STRICT_P, (f"p={p}: set differs outside the band at {outside[:8]} "
                          f"(scores {s[outside[:4]]}, tau {tau})")
    mm = O.mass(r["scores"])
    w, Z = mm["w"], mm["Z"]
    tg = float(tau_gpu)
    bandg = BAND_REL * max(abs(tg), 1.0)
    T_g = np.nonzero(s >= tg - bandg)[0]
    strict = s > tg + bandg
    core = np.union1d(np.nonzero(strict)[0], np.arange(min(n_sink, n)))
    assert np.all(np.isin(core, S_gpu)), "GPU set misses keys above its threshold"
    allowed = np.union1d(T_g, np.arange(min(n_sink, n)))
    assert np.all(np.isin(S_gpu, allowed)), "GPU set holds keys below its threshold"
    # every differing key lies between the two thresholds: one run of adjacent ranks
    lo, hi = min(tau, tg) - max(band, bandg), max(tau, tg) + max(band, bandg)
    assert np.all((s[diff] >= lo) & (s[diff] <= hi)), "differing keys outside the threshold run"
    reach = w[T_g].sum() / (p * Z)
    above = w[strict].sum() / (p * Z)
    slack = max(1.0 - reach, above - 1.0, 0.0)
    assert reach >= 1.0 - MASS_TOL, f"GPU set reaches only {reach:.9f} of p*Z"
    assert above < 1.0 + MASS_TOL, f"GPU threshold is not minimal: {above:.9f} of p*Z above it"
    st["valid-alt"] += 1
    st["alt_tokens"] += len(diff)
    st["max_mass_slack"] = max(st["max_mass_slack"], slack)
    return "valid-alt"


def check_set_topk(S_gpu: np.ndarray, r: Dict, top_k: int, n_sink: int) -> str:
    """Fixed budget: the GPU set equals the oracle's except for keys in the band
    around the oracle's threshold (a count decides, so no mass tolerance applies)."""
    st = stats()
    n = len(r["scores"])
    if top_k >= n:
        assert np.array_equal(S_gpu, np.arange(n)), "a budget >= n must keep every key"
        st["exact"] += 1
        return "exact"
    if np.array_equal(S_gpu, r["S"]):
        st["exact"] += 1
        return "exact"
    s = r["scores"].astype(np.float64)
    tau = float(r["tau"])
    diff = np.setxor1d(S_gpu, r["S"])
    assert np.all(np.abs(s[diff] - tau) <= BAND_REL * max(abs(tau), 1.0)), \
        f"top-{top_k} set differs outside the band: {diff[:8]}"
    st["band"] += 1
    st["band_tokens"] += len(diff)
    return "band"


def check_out(o_gpu_bits: np.ndarray, o_ref: np.ndarray, what: str = "") -> float:
    o = bf16_f64(o_gpu_bits)
    err = np.abs(o - o_ref)
    ulp_half = np.where(np.abs(o_ref) >= 4.0,
                        np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-30))) - 8), 0.0)
    bad = err > OUT_TOL + ulp_half
    assert not bad.any(), f"{what}: max err {err.max():.3g} at {np.argmax(err)}"
    st = stats()
    st["outputs"] += 1
    st["half_ulp_outputs"] += int((err > OUT_TOL).any())
    st["max_out_err"] = max(st["max_out_err"], float(err.max()))
    return float(err.max())


def compare_decode(wl, kc, vc, idx, res, top_p: float, heads=None, batches=None,
                   ret_only: bool = False):
    """Oracle decode vs GPU result; returns a summary dict.  Retrieval q-heads: the
    set (check_set), oracle attention over the GPU's own set, and the output end to
    end; local q-heads: the output."""
    G = wl.G
    ref = O.decode(wl, kc, vc, idx, top_p, heads=heads, batches=batches)
    kinds = {"exact": 0, "band": 0, "valid-alt": 0}
    worst = 0.0
    for (b, h), r in ref.items():
        kv = h // G
        is_ret = kv in wl.ret_kv_heads
        if ret_only and not is_ret:
            continue
        if is_ret and "cnt" in res:
            i = wl.ret_kv_heads.index(kv)
            unit = (b * wl.n_ret + i) * G + h % G
            S_g = gpu_set(res, unit)
            kinds[check_set(S_g, res["tau"][unit], r, top_p, wl.n_sink)] += 1
            # the attention step alone: oracle attention over the GPU's own set
            qr = O.rope(bf16_f64(wl.q_pre[b, h]), wl.N - 1, wl.rope_base)
            o_own = O.attention(qr, kc[b, kv][S_g], vc[b, kv][S_g], wl.attn_scale)
            check_out(res["out"][b, h], o_own, f"attention over GPU set b{b} h{h}")
        worst = max(worst, check_out(res["out"][b, h], r["out"], f"b{b} h{h}"))
    kinds["max_err"] = worst
    return kinds
