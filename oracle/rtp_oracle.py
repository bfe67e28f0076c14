"""CPU oracle for RTPurbo's head-wise sparse attention step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the graft
entry point and the cpu_baseline leg of the benchmark may import this module.
The product path (the HIP library and its Python binding) never calls it and
shares no code with it.

It is a plain, slow, obviously correct NumPy implementation of what the step
computes, in fp64 except where the method fixes fp32 (the indexer scores that
decide the selected set are rounded to fp32, the precision of the kernel that
takes the same decision).  Inputs are the bf16 bit patterns (uint16 arrays) the
GPU consumes.

Sources (the pages about arXiv 2605.16928, "Full Attention Strikes Back"):
  [zhichai]   zhichai.net blog, sections 02-03 (three insights, three steps)
  [techwalker] techwalker article, sections 2 (head roles), 3 (16-dim indexer),
              4 (dynamic top-p budget), 6 (GPU kernels), 8 (window/sink settings)
  [v2]        aitntnews RTPurboV2 article, findings 1-4
  [ngjoo]     ngjoo paper digest, abstract and core-method summary

Steps, in the order the step performs them:
  append        index row = bf16(k_pre . W_k) from the pre-RoPE key; K cache row
                = bf16(RoPE(k_pre, j)); V row stored as is
                ([techwalker] §3: 128 -> 16 projection per retrieval head;
                [ngjoo] core method: low-dimensional pre-RoPE projections)
  query_prep    qi = q_pre . W_q (fp32 result), q_rope = RoPE(q_pre, pos)
  scores        s_j = fp32(idx_scale * <qi, index_j>) for every cached key j <= pos
                ([techwalker] §3: the 16-dim "radar" scores every token first)
  top_p_set     softmax-normalised mass; smallest highest-scoring set whose mass
                reaches p ([techwalker] §4; [zhichai] 02 insight three;
                [v2] finding 4)
  top_k_set     the fixed-budget baseline: the k highest scores ([techwalker] §4, §7)
  with_sinks    union with the first n_sink tokens ([techwalker] §2 attention
                sinks, §8: 4 sinks)
  attention     exact 128-dim softmax attention over the chosen rows only
                ([techwalker] §3: full 128-dim computation on the selected words)
  swa_keys      local heads: sliding window of W tokens ending at the query,
                plus the sinks ([techwalker] §2, §8: window 8192 + 4 sinks)
  prefill_row   the decode computation for query row t with keys j <= t
  kmeans_index  the V2 cluster index: k-means over the index rows ([v2] finding 3)
  cluster_head  decode through it: coarse match of the centres, top-p over clusters,
                exact attention over the hit clusters' tokens ([v2] finding 3)

Readings where the pages are silent (each repeated at the function):
  * idx_scale multiplies the dot product; 1.0 in every workload.
  * top-p: the set is {j : s_j >= tau}, where tau is the score at which the
    descending cumulative mass first reaches p * Z; ties at tau are included.
    p >= 1 selects every key without summing.
  * sinks are added after top-p; their mass counts toward p like any token's.
  * softmax over the selected rows is renormalised over those rows.
  * RoPE pairs dimension i with i + D/2 (rotate-half), theta_i = base^(-2i/D),
    angle pos * theta_i evaluated in fp64.
  * the decode query sits at position N - 1 and sees itself; the SWA window is
    (pos - W, pos].
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

HEAD_DIM = 128
IDX_RANK = 16


# ---------------------------------------------------------------- bf16 bits

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value, ties to the even mantissa; returns uint16 bits.

    The two bf16 neighbours of x are found from its fp32 image (which lies within
    half an fp32 ulp of x, so it never leaves the bf16 interval that holds x); the
    choice between them compares |x| with their midpoint exactly in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    lo_bits = f.view(np.uint32).astype(np.int64) >> 16          # truncated toward zero
    lo = (lo_bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    hi = ((lo_bits + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    amid = np.abs(0.5 * (lo + hi))
    ax = np.abs(x)
    up = (ax > amid) | ((ax == amid) & ((lo_bits & 1) == 1))
    return (np.where(up, lo_bits + 1, lo_bits) & 0xFFFF).astype(np.uint16)


# ---------------------------------------------------------------- RoPE

def rope_angles(pos: np.ndarray, dim: int = HEAD_DIM, base: float = 1e6) -> np.ndarray:
    """Angles pos * theta_i with theta_i = base^(-2i/dim), i < dim/2, in fp64.

    [techwalker] §3 and [v2] finding 2 describe RoPE as a per-dimension rotation
    whose speed falls with the dimension index; the pages' formula was lost, so
    the standard rotate-half form with these frequencies is the reading.
    """
    i = np.arange(dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rope(x: np.ndarray, pos, base: float = 1e6) -> np.ndarray:
    """Rotate x[..., D] at positions pos[...]: pairs (i, i + D/2) turn by pos*theta_i."""
    x = np.asarray(x, dtype=np.float64)
    d2 = x.shape[-1] // 2
    ang = rope_angles(np.asarray(pos), x.shape[-1], base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :d2], x[..., d2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------- append

def append(k_pre: np.ndarray, v: np.ndarray, w_k: np.ndarray, ret_kv_heads: Sequence[int],
           start_pos: int, rope_base: float = 1e6, rows: Optional[np.ndarray] = None):
    """Cache append for tokens start_pos .. start_pos+T-1.

    k_pre, v: [B][Hkv][T][D] bf16 bits; w_k: [n_ret][D][r] bf16 bits.
    Returns (k_cache_rows [B][Hkv][T][D], v_rows, index_rows [B][n_ret][T][r]) as bf16 bits.
    The index is computed from the pre-RoPE key ([ngjoo] core method: pre-RoPE
    projections), the cache row from the rotated key.  When `rows` is given, RoPE
    is evaluated only for those token offsets (others are returned as zero bits).
    """
    k = np.asarray(k_pre)
    B, Hkv, T, D = k.shape
    kc = np.zeros_like(k, dtype=np.uint16)
    sel = np.arange(T) if rows is None else np.asarray(rows)
    pos = start_pos + sel
    for b in range(B):
        for h in range(Hkv):
            kc[b, h, sel] = f64_to_bf16(rope(bf16_to_f64(k[b, h, sel]), pos, rope_base))
    idx = np.zeros((B, len(ret_kv_heads), T, w_k.shape[-1]), dtype=np.uint16)
    for b in range(B):
        for i, h in enumerate(ret_kv_heads):
            idx[b, i] = f64_to_bf16(bf16_to_f64(k[b, h]) @ bf16_to_f64(w_k[i]))
    return kc, np.array(v, dtype=np.uint16, copy=True), idx


# ---------------------------------------------------------------- query side

def query_index(q_pre_row: np.ndarray, w_q_head: np.ndarray) -> np.ndarray:
    """qi = q_pre . W_q for one head, as an fp32 vector ([techwalker] §3)."""
    return (bf16_to_f64(q_pre_row) @ bf16_to_f64(w_q_head)).astype(np.float32)


def scores(qi: np.ndarray, index_rows: np.ndarray, idx_scale: float = 1.0) -> np.ndarray:
    """s_j = fp32(idx_scale * <qi, index_j>) for all rows given (fp64 sum, one rounding)."""
    s = bf16_to_f64(index_rows) @ np.asarray(qi, dtype=np.float64)
    return (np.float64(idx_scale) * s).astype(np.float32)


def mass(s: np.ndarray) -> Dict[str, object]:
    """Softmax masses of fp32 scores in fp64: m = max s, w = exp(s - m), Z = sum w."""
    s64 = np.asarray(s, dtype=np.float64)
    m = float(s64.max())
    w = np.exp(s64 - m)
    return {"m": m, "w": w, "Z": float(w.sum())}


def top_p_set(s: np.ndarray, p: float) -> Dict[str, object]:
    """Dynamic top-p ([techwalker] §4; [zhichai] 02 insight three; [v2] finding 4).

    Keeps the smallest highest-scoring set whose softmax mass reaches p.  Keys are
    ordered by score, descending; tau is the score at the first position where the
    running mass is >= p * Z; the set is {j : s_j >= tau}, ties included.
    p >= 1 keeps every key and tau = -inf.
    """
    s = np.asarray(s, dtype=np.float32)
    if p >= 1.0:
        return {"set": np.arange(len(s)), "tau": -np.inf, "m": float(s.max()),
                "Z": mass(s)["Z"]}
    mm = mass(s)
    order = np.argsort(-s.astype(np.float64), kind="stable")
    cum = np.cumsum(mm["w"][order])
    k = int(np.searchsorted(cum, p * mm["Z"], side="left"))
    k = min(k, len(s) - 1)
    tau = float(s[order[k]])
    chosen = np.nonzero(s >= np.float32(tau))[0]
    return {"set": chosen, "tau": tau, "m": mm["m"], "Z": mm["Z"]}


def top_k_set(s: np.ndarray, k: int) -> Dict[str, object]:
    """Fixed top-k budget, the baseline the pages set dynamic top-p against
    ([techwalker] §4 and §7: a fixed token budget per head; [v2] finding 4).

    Keeps the k highest-scoring keys: tau is the k-th largest score and the set is
    {j : s_j >= tau}, ties included (the same threshold form as top_p_set).
    k >= number of keys keeps every key and tau = -inf.
    """
    s = np.asarray(s, dtype=np.float32)
    if k >= len(s):
        return {"set": np.arange(len(s)), "tau": -np.inf, "m": float(s.max())}
    order = np.argsort(-s.astype(np.float64), kind="stable")
    tau = float(s[order[k - 1]])
    chosen = np.nonzero(s >= np.float32(tau))[0]
    return {"set": chosen, "tau": tau, "m": float(s.max())}


def with_sinks(chosen: np.ndarray, n_sink: int, n_keys: int) -> np.ndarray:
    """S = T u {j < n_sink}, sorted ([techwalker] §2, §8: first tokens always kept)."""
    sinks = np.arange(min(n_sink, n_keys))
    return np.union1d(np.asarray(chosen, dtype=np.int64), sinks)


def attention(q_rope: np.ndarray, k_rows_bits: np.ndarray, v_rows_bits: np.ndarray,
              attn_scale: float) -> np.ndarray:
    """Softmax attention of one query over the given rows, fp64 throughout."""
    k = bf16_to_f64(k_rows_bits)
    v = bf16_to_f64(v_rows_bits)
    logits = attn_scale * (k @ np.asarray(q_rope, dtype=np.float64))
    logits -= logits.max()
    e = np.exp(logits)
    return (e[:, None] * v).sum(axis=0) / e.sum()


def swa_keys(pos: int, window: int, n_sink: int) -> np.ndarray:
    """Local-head keys: (pos - W, pos] u {j < n_sink} ([techwalker] §2, §8)."""
    lo = max(0, pos - window + 1)
    return np.union1d(np.arange(lo, pos + 1), np.arange(min(n_sink, pos + 1)))


# ---------------------------------------------------------------- whole step

def retrieval_head(q_pre_row, w_q_head, k_cache_head, v_cache_head, index_head, pos: int,
                   top_p: float, n_sink: int, idx_scale: float, attn_scale: float,
                   rope_base: float = 1e6, top_k: Optional[int] = None) -> Dict[str, object]:
    """One retrieval q-head at query position pos over keys 0..pos (top-p, or a fixed
    top-k budget when top_k is given)."""
    n = pos + 1
    qi = query_index(q_pre_row, w_q_head)
    s = scores(qi, index_head[:n], idx_scale)
    tp = top_p_set(s, top_p) if top_k is None else top_k_set(s, top_k)
    S = with_sinks(tp["set"], n_sink, n)
    qr = rope(bf16_to_f64(q_pre_row), pos, rope_base)
    o = attention(qr, k_cache_head[S], v_cache_head[S], attn_scale)
    return {"out": o, "scores": s, "qi": qi, "T": tp["set"], "S": S, "tau": tp["tau"],
            "m": tp["m"], "Z": tp.get("Z")}


def local_head(q_pre_row, k_cache_head, v_cache_head, pos: int, window: int, n_sink: int,
               attn_scale: float, rope_base: float = 1e6) -> Dict[str, object]:
    L = swa_keys(pos, window, n_sink)
    qr = rope(bf16_to_f64(q_pre_row), pos, rope_base)
    return {"out": attention(qr, k_cache_head[L], v_cache_head[L], attn_scale), "L": L}


def decode(wl, k_cache, v_cache, index, top_p: float, heads: Optional[Iterable] = None,
           batches: Optional[Iterable] = None, top_k: Optional[int] = None) -> Dict:
    """Decode step for a workload: query at position N-1 of every batch row.

    Returns {(b, h): head result} for the requested heads (default: all).  With top_k
    the retrieval heads keep a fixed budget of the top_k highest scores instead of
    the top-p set.
    """
    G = wl.Hq // wl.Hkv
    pos = wl.N - 1
    ret = list(wl.ret_kv_heads)
    res = {}
    for b in (range(wl.B) if batches is None else batches):
        for h in (range(wl.Hq) if heads is None else heads):
            kv = h // G
            if kv in ret:
                i = ret.index(kv)
                res[(b, h)] = retrieval_head(
                    wl.q_pre[b, h], wl.w_q[i * G + h % G], k_cache[b, kv], v_cache[b, kv],
                    index[b, i], pos, top_p, wl.n_sink, wl.idx_scale, wl.attn_scale,
                    wl.rope_base, top_k=top_k)
            else:
                res[(b, h)] = local_head(wl.q_pre[b, h], k_cache[b, kv], v_cache[b, kv], pos,
                                         wl.window, wl.n_sink, wl.attn_scale, wl.rope_base)
    return res


def prefill_row(wl, k_cache, v_cache, index, b: int, h: int, t: int, top_p: float) -> Dict:
    """Query row t of the chunk (absolute position q_start + t), keys j <= position."""
    G = wl.Hq // wl.Hkv
    pos = wl.q_start + t
    kv = h // G
    ret = list(wl.ret_kv_heads)
    q = wl.q_pre[b, h, t]
    if kv in ret:
        i = ret.index(kv)
        return retrieval_head(q, wl.w_q[i * G + h % G], k_cache[b, kv], v_cache[b, kv],
                              index[b, i], pos, top_p, wl.n_sink, wl.idx_scale,
                              wl.attn_scale, wl.rope_base)
    return local_head(q, k_cache[b, kv], v_cache[b, kv], pos, wl.window, wl.n_sink,
                      wl.attn_scale, wl.rope_base)


def caches_for(wl, rows_needed: Optional[Dict[int, np.ndarray]] = None):
    """Oracle append of the whole workload context (start_pos 0).

    rows_needed maps a KV head to the token rows whose rotated key is needed;
    heads not listed get every row.
    """
    B, Hkv, N, D = wl.k_pre.shape
    kc = np.zeros((B, Hkv, N, D), dtype=np.uint16)
    idx = np.zeros((B, wl.n_ret, N, wl.w_k.shape[-1]), dtype=np.uint16)
    for b in range(B):
        for h in range(Hkv):
            rows = None if rows_needed is None else rows_needed.get(h)
            sel = np.arange(N) if rows is None else np.asarray(rows)
            for s0 in range(0, len(sel), 1 << 16):
                part = sel[s0:s0 + (1 << 16)]
                kc[b, h, part] = f64_to_bf16(rope(bf16_to_f64(wl.k_pre[b, h, part]), part,
                                                  wl.rope_base))
        for i, h in enumerate(wl.ret_kv_heads):
            for s0 in range(0, N, 1 << 16):
                idx[b, i, s0:s0 + (1 << 16)] = f64_to_bf16(
                    bf16_to_f64(wl.k_pre[b, h, s0:s0 + (1 << 16)]) @ bf16_to_f64(wl.w_k[i]))
    return kc, wl.v, idx


# ---------------------------------------------------------------- V2 cluster index
#
# [v2] finding 3: the low-rank index rows of the cached tokens are grouped into K
# semantic clusters (K = 128 in the article's example); a query first matches the K
# cluster centres (coarse), and full attention then runs only over the tokens of the
# clusters it hits (fine).  The retrieval heads of the V2 recipe combine the low-rank
# projection, this cluster index and dynamic top-p ([v2] summary of the recipe).
#
# Readings where the pages give only the outline:
#  * clustering is Lloyd's k-means on the 16-dim index rows with squared Euclidean
#    distance, seeded with the index rows of K caller-chosen tokens and run for a
#    caller-chosen number of iterations; a final assignment to the last centres
#    defines the clusters;
#  * the nearest-centre decision is taken in fp32, the precision of the kernel that
#    takes it: the distance accumulates (x_d - c_d)^2 over d = 0..15 in order, each
#    subtraction, square and addition rounded to fp32; ties go to the lowest centre;
#  * a centre is the mean of its rows: every bf16 value becomes an integer multiple of
#    2^-24 (truncated toward zero; exact for |x| >= 2^-17), the integers are summed,
#    and the sum is divided in fp64 and rounded to fp32; an empty cluster keeps its
#    centre;
#  * the coarse match scores a cluster by sigma_c = fp32(idx_scale <qi, centre_c>) and
#    weighs it by its size: w_c = n_c exp(sigma_c - max sigma), the softmax mass its
#    tokens would have if each scored sigma_c; the clusters hit are the top-p set of
#    these masses (same threshold rule as tokens, ties included; p >= 1 takes every
#    non-empty cluster);
#  * the tokens attended are the members of the hit clusters, the tokens appended
#    after the build (n_tokens .. pos), and the sinks.

FX_CENTRE = 16777216.0   # 2^-24 units of the centre sums


def kmeans_assign(x32: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """Nearest centre of every row (reading: fp32 distance in dimension order,
    ties to the lowest centre)."""
    x32 = np.asarray(x32, dtype=np.float32)
    c32 = np.asarray(c32, dtype=np.float32)
    n, r = x32.shape
    best = np.full(n, np.inf, dtype=np.float32)
    arg = np.zeros(n, dtype=np.int64)
    for k in range(c32.shape[0]):
        acc = np.zeros(n, dtype=np.float32)
        for d in range(r):
            t = x32[:, d] - c32[k, d]
            acc = acc + t * t
        better = acc < best
        best = np.where(better, acc, best)
        arg = np.where(better, k, arg)
    return arg


def kmeans_centres(x_bits: np.ndarray, assign: np.ndarray, prev_c32: np.ndarray) -> np.ndarray:
    """Means of the clusters' rows from exact integer sums (reading above); an empty
    cluster keeps its previous centre."""
    K, r = prev_c32.shape
    fx = np.trunc(bf16_to_f64(x_bits) * FX_CENTRE).astype(np.int64)
    sums = np.zeros((K, r), dtype=np.int64)
    np.add.at(sums, np.asarray(assign, dtype=np.int64), fx)
    cnt = np.bincount(assign, minlength=K)
    c = np.array(prev_c32, dtype=np.float32, copy=True)
    nz = cnt > 0
    c[nz] = (sums[nz].astype(np.float64) /
             (cnt[nz, None].astype(np.float64) * FX_CENTRE)).astype(np.float32)
    return c


def kmeans_index(index_bits: np.ndarray, init: Sequence[int], iters: int) -> Dict[str, object]:
    """The cluster index of one retrieval KV head ([v2] finding 3): Lloyd's k-means on
    the index rows (N, 16) seeded with the rows of tokens `init`, `iters` updates,
    then the final assignment.  members lists the tokens grouped by cluster, in
    ascending token order within a cluster; cluster c holds
    members[offsets[c]:offsets[c + 1]]."""
    index_bits = np.asarray(index_bits, dtype=np.uint16)
    x32 = bf16_to_f64(index_bits).astype(np.float32)
    c32 = x32[np.asarray(init, dtype=np.int64)].copy()
    for _ in range(iters):
        c32 = kmeans_centres(index_bits, kmeans_assign(x32, c32), c32)
    assign = kmeans_assign(x32, c32)
    K = c32.shape[0]
    members = np.argsort(assign, kind="stable")
    offsets = np.concatenate([[0], np.cumsum(np.bincount(assign, minlength=K))]).astype(np.int64)
    return {"centroids": c32, "assign": assign, "members": members, "offsets": offsets}


def cluster_select(qi: np.ndarray, centroids: np.ndarray, counts: np.ndarray, p: float,
                   idx_scale: float = 1.0) -> Dict[str, object]:
    """Coarse match and dynamic top-p over clusters (reading above): sigma_c, the
    size-weighted masses w_c, and the hit clusters {c : n_c > 0, sigma_c >= tau_c}."""
    sigma = (np.float64(idx_scale) * (np.asarray(centroids, dtype=np.float64) @
                                      np.asarray(qi, dtype=np.float64))).astype(np.float32)
    counts = np.asarray(counts, dtype=np.int64)
    live = np.nonzero(counts > 0)[0]
    if p >= 1.0:
        return {"sigma": sigma, "hit": live, "tau": -np.inf}
    s = sigma[live].astype(np.float64)
    w = counts[live].astype(np.float64) * np.exp(s - s.max())
    order = np.argsort(-s, kind="stable")
    cum = np.cumsum(w[order])
    i = int(np.searchsorted(cum, p * w.sum(), side="left"))
    i = min(i, len(order) - 1)
    tau = float(sigma[live][order[i]])
    hit = live[sigma[live] >= np.float32(tau)]
    return {"sigma": sigma, "hit": hit, "tau": tau, "W": float(w.sum())}


def cluster_head(q_pre_row, w_q_head, k_cache_head, v_cache_head, cl: Dict[str, object],
                 n_tokens: int, pos: int, top_p: float, n_sink: int, idx_scale: float,
                 attn_scale: float, rope_base: float = 1e6) -> Dict[str, object]:
    """One retrieval q-head decoding through the cluster index built over tokens
    0 .. n_tokens-1: S = members of the hit clusters u (n_tokens .. pos) u sinks, then
    exact attention over S."""
    qi = query_index(q_pre_row, w_q_head)
    counts = np.diff(np.asarray(cl["offsets"], dtype=np.int64))
    sel = cluster_select(qi, cl["centroids"], counts, top_p, idx_scale)
    off = np.asarray(cl["offsets"], dtype=np.int64)
    parts = [np.asarray(cl["members"][off[c]:off[c + 1]], dtype=np.int64) for c in sel["hit"]]
    parts.append(np.arange(n_tokens, pos + 1, dtype=np.int64))
    S = with_sinks(np.concatenate(parts) if parts else np.zeros(0, np.int64), n_sink, pos + 1)
    qr = rope(bf16_to_f64(q_pre_row), pos, rope_base)
    o = attention(qr, k_cache_head[S], v_cache_head[S], attn_scale)
    return {"out": o, "S": S, "hit": sel["hit"], "sigma": sel["sigma"], "tau": sel["tau"],
            "qi": qi}
