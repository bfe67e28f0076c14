"""Seeded synthetic workloads for RTPurbo's head-wise sparse attention step.

This module draws the inputs that both the CPU oracle and the HIP path consume.
It holds none of the method's arithmetic: no RoPE, no indexer projection, no
top-p selection and no attention.  It only draws Gaussian tensors with NumPy's
PCG64 generator, plants keys aligned to a direction, and rounds fp32 draws to
bf16 bit patterns (round to nearest even).

Workload shapes: a tiny needle decode, a Qwen3-8B-shaped decode at 64K, a
variable-budget decode at 128K, a 1M-context decode shaped like Qwen3-30B-A3B's
attention, and a 4096-token chunked prefill at 256K and at 1M.  The pages measure on RULER, LongBench, AIME and
needle-in-a-haystack; these synthetic inputs stand in for them and imitate the
regimes the pages report (a needle query covered by a couple of tokens, a
diffuse query needing thousands; "Full Attention Strikes Back", techwalker
article, section 4).

Readings of the configuration text (each stated where it is used):
  * the indexer projection of a retrieval KV head is one draw W ~ N(0, 1/128)
    shared by W_q of every q-head in that group and by W_k;
  * plant(u, a) = a * sqrt(D) * u + 0.3 * eps, eps ~ N(0, I): "alignment scale a"
    means a times the typical key norm sqrt(D) along the unit vector u;
  * planted positions avoid the sink tokens and the query's own position;
  * cluster sizes ~ U{200..2000}, scaled down together when their sum exceeds
    floor(0.75 * (N - n_sink));
  * the GQA map is kv(h) = h // G and token j sits at RoPE position j.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

D = 128
R = 16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs never overflow 32 bits here (largest: 0xFF7FFFFF + 0x8000)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One seeded layer input.  bf16 tensors are uint16 bit patterns, C-contiguous.

    q_pre  [B][Hq][D]        (decode) or [B][Hq][Tq][D] (prefill chunk)
    k_pre  [B][Hkv][N][D]    pre-RoPE keys of every cached token
    v      [B][Hkv][N][D]
    w_q    [n_ret*G][D][R]   retrieval q-heads in head order
    w_k    [n_ret][D][R]     per retrieval KV head
    """
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    N: int
    ret_kv_heads: List[int]
    n_sink: int
    window: int
    rope_base: float
    top_p: List[float]
    q_pre: np.ndarray
    k_pre: np.ndarray
    v: np.ndarray
    w_q: np.ndarray
    w_k: np.ndarray
    Tq: int = 1
    q_start: int = -1
    idx_scale: float = 1.0
    meta: Dict = dataclasses.field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_ret(self) -> int:
        return len(self.ret_kv_heads)

    @property
    def attn_scale(self) -> float:
        return 1.0 / math.sqrt(D)

    @property
    def is_prefill(self) -> bool:
        return self.q_pre.ndim == 4

    def ret_q_heads(self) -> List[int]:
        return [kv * self.G + g for kv in self.ret_kv_heads for g in range(self.G)]

    def local_q_heads(self) -> List[int]:
        rq = set(self.ret_q_heads())
        return [h for h in range(self.Hq) if h not in rq]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return x / np.linalg.norm(x)


def _plant(rng, u: np.ndarray, a: float) -> np.ndarray:
    return (a * math.sqrt(D) * u + 0.3 * rng.standard_normal(D)).astype(np.float32)


def _projection(rng, n_ret: int, G: int):
    w = (_normal(rng, (n_ret, D, R)) * np.float32(1.0 / math.sqrt(D))).astype(np.float32)
    w_k = f32_to_bf16_bits(w)
    w_q = np.repeat(w_k, G, axis=0)
    return w_q, w_k


def _kv_background(rng, B, Hkv, N, chunk=1 << 16):
    """Gaussian K, V drawn in chunks so fp32 temporaries stay small."""
    k = np.empty((B, Hkv, N, D), dtype=np.uint16)
    v = np.empty((B, Hkv, N, D), dtype=np.uint16)
    for b in range(B):
        for h in range(Hkv):
            for s in range(0, N, chunk):
                e = min(N, s + chunk)
                k[b, h, s:e] = f32_to_bf16_bits(_normal(rng, (e - s, D)))
                v[b, h, s:e] = f32_to_bf16_bits(_normal(rng, (e - s, D)))
    return k, v


def _cluster_sizes(rng, n_clusters: int, N: int, n_sink: int) -> np.ndarray:
    sizes = rng.integers(200, 2001, size=n_clusters)
    cap = int(math.floor(0.75 * (N - n_sink)))
    tot = int(sizes.sum())
    if tot > cap:
        sizes = np.floor(sizes * (cap / tot)).astype(np.int64)
    return np.maximum(sizes, 1)


def _plant_clusters(rng, k_head: np.ndarray, N: int, n_sink: int, n_clusters: int,
                    forbid_last: bool = True):
    """Plant clusters (centroid c ~ N(0,I), members c + 0.3*eps) into one head's keys.

    Returns the centroids (fp32 [n_clusters][D]) and the member positions.
    """
    sizes = _cluster_sizes(rng, n_clusters, N, n_sink)
    hi = N - 1 if forbid_last else N
    perm = rng.permutation(np.arange(n_sink, hi))
    cents = _normal(rng, (n_clusters, D))
    members = []
    off = 0
    for c in range(n_clusters):
        pos = np.sort(perm[off:off + int(sizes[c])])
        off += int(sizes[c])
        keys = cents[c][None, :] + np.float32(0.3) * _normal(rng, (len(pos), D))
        k_head[pos] = f32_to_bf16_bits(keys)
        members.append(pos)
    return cents, members


def tiny_decode(seed: int = 1001, N: int = 4096) -> Workload:
    """Tiny decode: B=1, 4 q / 2 KV heads, KV0 retrieval (p=0.9), KV1 local (W=512).

    Three needles get keys plant(q_hat_{i mod 2}, 4) on KV head 0.
    """
    rng = _rng(seed)
    B, Hq, Hkv = 1, 4, 2
    G = Hq // Hkv
    w_q, w_k = _projection(rng, 1, G)
    q = _normal(rng, (B, Hq, D))
    k, v = _kv_background(rng, B, Hkv, N)
    needle_pos = np.sort(rng.choice(np.arange(4, N - 1), size=3, replace=False))
    owners = []
    for i, pos in enumerate(needle_pos):
        h = i % 2
        k[0, 0, pos] = f32_to_bf16_bits(_plant(rng, _unit(q[0, h]), 4.0))
        owners.append(h)
    return Workload("tiny_decode", seed, B, Hq, Hkv, N, [0], 4, 512, 1e6, [0.9],
                    f32_to_bf16_bits(q), k, v, w_q, w_k,
                    meta={"needles": needle_pos.tolist(), "needle_owner": owners})


def clustered_decode(name: str, seed: int, B: int, Hq: int, Hkv: int, N: int,
                     ret_kv: List[int], n_clusters: int, top_p=(0.9,), window=8192,
                     n_sink=4) -> Workload:
    """Decode with planted topic clusters on the retrieval KV heads.

    Each retrieval q-head is aligned to one random cluster: q = c_t + 0.3*eps.
    """
    rng = _rng(seed)
    G = Hq // Hkv
    w_q, w_k = _projection(rng, len(ret_kv), G)
    q = _normal(rng, (B, Hq, D))
    k, v = _kv_background(rng, B, Hkv, N)
    aligned = {}
    for b in range(B):
        for kv in ret_kv:
            cents, _ = _plant_clusters(rng, k[b, kv], N, n_sink, n_clusters)
            for g in range(G):
                h = kv * G + g
                t = int(rng.integers(0, n_clusters))
                q[b, h] = cents[t] + np.float32(0.3) * _normal(rng, (D,))
                aligned[(b, h)] = t
    return Workload(name, seed, B, Hq, Hkv, N, list(ret_kv), n_sink, window, 1e6,
                    list(top_p), f32_to_bf16_bits(q), k, v, w_q, w_k,
                    meta={"aligned_cluster": aligned})


def qwen3_8b_decode(seed: int = 1002, B: int = 8, N: int = 65536) -> Workload:
    """Qwen3-8B-shaped decode: 32 q / 8 KV heads, KV {0,5} retrieval, 64 clusters."""
    return clustered_decode("qwen3_8b_decode_64k", seed, B, 32, 8, N, [0, 5], 64)


def million_decode(seed: int = 1004, N: int = 1 << 20, n_clusters: int = 512) -> Workload:
    """1M-context decode shaped like Qwen3-30B-A3B attention: 32 q / 4 KV heads, KV0 retrieval."""
    return clustered_decode("million_decode_1m", seed, 1, 32, 4, N, [0], n_clusters)


def variable_budget_decode(seed: int = 1003, B: int = 4, N: int = 131072,
                           n_diffuse: int = 8000) -> Workload:
    """Variable-budget decode at 128K: per retrieval group, 2 diffuse and 2 needle q-heads.

    Diffuse heads share a topic of n_diffuse keys plant(u, 1.5) and query sqrt(D)*u + 0.3*eps;
    needle heads draw q ~ N(0,1) and each plants 2 keys plant(q_hat, 6).
    """
    rng = _rng(seed)
    Hq, Hkv = 32, 8
    G = Hq // Hkv
    ret_kv = [0, 5]
    n_sink = 4
    w_q, w_k = _projection(rng, len(ret_kv), G)
    q = _normal(rng, (B, Hq, D))
    k, v = _kv_background(rng, B, Hkv, N)
    kinds = {}
    for b in range(B):
        for kv in ret_kv:
            u = _unit(_normal(rng, (D,)))
            perm = rng.permutation(np.arange(n_sink, N - 1))
            topic = np.sort(perm[:n_diffuse])
            off = n_diffuse
            keys = (1.5 * math.sqrt(D) * u[None, :]
                    + 0.3 * rng.standard_normal((n_diffuse, D))).astype(np.float32)
            k[b, kv, topic] = f32_to_bf16_bits(keys)
            order = rng.permutation(G)
            for rank, g in enumerate(order):
                h = kv * G + int(g)
                if rank < 2:
                    q[b, h] = (math.sqrt(D) * u + 0.3 * rng.standard_normal(D)).astype(np.float32)
                    kinds[(b, h)] = ("diffuse", [])
                else:
                    qh = _unit(q[b, h])
                    pos = perm[off:off + 2]
                    off += 2
                    for p_ in pos:
                        k[b, kv, p_] = f32_to_bf16_bits(_plant(rng, qh, 6.0))
                    kinds[(b, h)] = ("needle", sorted(int(x) for x in pos))
    return Workload("variable_budget_128k", seed, B, Hq, Hkv, N, ret_kv, n_sink, 8192, 1e6,
                    [0.8, 0.9, 0.95], f32_to_bf16_bits(q), k, v, w_q, w_k,
                    meta={"kinds": kinds})


def chunked_prefill(seed: int = 1005, N: int = 262144, Tq: int = 4096,
                    n_clusters: int = 256, B: int = 1,
                    name: str = "chunked_prefill_256k") -> Workload:
    """Chunked prefill: the last Tq of N cached tokens are the query chunk.

    32 q / 8 KV heads, KV {0,5} retrieval with planted clusters; each (row, retrieval
    q-head) is aligned to an independent random cluster; local q ~ N(0,1).
    """
    rng = _rng(seed)
    Hq, Hkv = 32, 8
    G = Hq // Hkv
    ret_kv = [0, 5]
    n_sink = 4
    w_q, w_k = _projection(rng, len(ret_kv), G)
    q = np.empty((B, Hq, Tq, D), dtype=np.float32)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = _normal(rng, (Tq, D))
    k, v = _kv_background(rng, B, Hkv, N)
    for b in range(B):
        for kv in ret_kv:
            cents, _ = _plant_clusters(rng, k[b, kv], N, n_sink, n_clusters, forbid_last=False)
            for g in range(G):
                h = kv * G + g
                t = rng.integers(0, n_clusters, size=Tq)
                q[b, h] = cents[t] + np.float32(0.3) * _normal(rng, (Tq, D))
    return Workload(name, seed, B, Hq, Hkv, N, ret_kv, n_sink, 8192, 1e6,
                    [0.9], f32_to_bf16_bits(q), k, v, w_q, w_k, Tq=Tq, q_start=N - Tq)


def million_prefill(seed: int = 1006, N: int = 1 << 20, Tq: int = 4096,
                    n_clusters: int = 1024) -> Workload:
    """The chunked prefill at 1M context (the pages quote their largest prefill gain
    there): a 4096-row chunk at the end of 1,048,576 cached keys, the head layout of
    the 256K chunk, and 1024 clusters, the same cluster density as 256 over 256K."""
    return chunked_prefill(seed, N, Tq, n_clusters, name="chunked_prefill_1m")


def random_decode(seed: int, B: int, Hq: int, Hkv: int, N: int, ret_kv: List[int],
                  window: int, n_sink: int = 4, top_p=(0.9,), n_needles: int = 0,
                  needle_scale: float = 4.0, q_scale: float = 1.0) -> Workload:
    """Small random decode shapes for parity sweeps (Gaussian q, K, V, optional needles)."""
    rng = _rng(seed)
    G = Hq // Hkv
    w_q, w_k = _projection(rng, len(ret_kv), G)
    q = _normal(rng, (B, Hq, D)) * np.float32(q_scale)
    k, v = _kv_background(rng, B, Hkv, N)
    lo, hi = min(n_sink, N - 1), N - 1
    if n_needles and hi > lo:
        for b in range(B):
            for kv in ret_kv:
                pos = rng.choice(np.arange(lo, hi), size=min(n_needles, hi - lo), replace=False)
                for i, p_ in enumerate(pos):
                    h = kv * G + (i % G)
                    k[b, kv, p_] = f32_to_bf16_bits(_plant(rng, _unit(q[b, h]), needle_scale))
    return Workload(f"random_decode_s{seed}", seed, B, Hq, Hkv, N, list(ret_kv), n_sink,
                    window, 1e6, list(top_p), f32_to_bf16_bits(q), k, v, w_q, w_k)


def random_prefill(seed: int, B: int, Hq: int, Hkv: int, N: int, Tq: int, ret_kv: List[int],
                   window: int, n_sink: int = 4, top_p=(0.9,), n_clusters: int = 8) -> Workload:
    """Small prefill chunk shapes for parity sweeps: clusters on retrieval heads, rows aligned
    to random clusters."""
    rng = _rng(seed)
    G = Hq // Hkv
    w_q, w_k = _projection(rng, len(ret_kv), G)
    q = _normal(rng, (B, Hq, Tq, D))
    k, v = _kv_background(rng, B, Hkv, N)
    for b in range(B):
        for kv in ret_kv:
            if N - n_sink > 4 * n_clusters:
                cents, _ = _plant_clusters(rng, k[b, kv], N, n_sink, n_clusters,
                                           forbid_last=False)
                for g in range(G):
                    h = kv * G + g
                    t = rng.integers(0, n_clusters, size=Tq)
                    q[b, h] = cents[t] + np.float32(0.3) * _normal(rng, (Tq, D))
    return Workload(f"random_prefill_s{seed}", seed, B, Hq, Hkv, N, list(ret_kv), n_sink,
                    window, 1e6, list(top_p), f32_to_bf16_bits(q), k, v, w_q, w_k,
                    Tq=Tq, q_start=N - Tq)


CONFIGS = {
    1: tiny_decode,
    2: qwen3_8b_decode,
    3: variable_budget_decode,
    4: million_decode,
    5: chunked_prefill,
    6: million_prefill,
}


def make(config: int, seed: Optional[int] = None, **kw) -> Workload:
    """Build configuration 1..6 with seed 1000 + config unless given (6: the chunked
    prefill at 1M context)."""
    fn = CONFIGS[config]
    return fn(seed=1000 + config if seed is None else seed, **kw)
