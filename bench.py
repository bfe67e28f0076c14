"""Benchmark of the head-wise sparse attention decode step on one MI355X.

One step = the whole decode hot path of one layer over one batch:
  append of the newest token (K/V caches + 16-dim index), the retrieval-head
  decode (indexer scan + histogram, threshold, select, resolve, gather attention,
  merge) and the local-head sliding-window attention.
Default workload: 1M-context decode shaped like Qwen3-30B-A3B attention (B=1,
32 q / 4 KV heads, KV head 0 retrieval with a 1M x 16 index, 3 SWA heads with
window 8192 + 4 sinks, 512 planted clusters, p = 0.9), synthetic seeded inputs.

Timing: W warm-up steps, then K timed steps.  Before each timed step a read of
a 512 MiB scratch buffer evicts the step's working set from the 256 MB Infinity
Cache and the L2s, so every step reads it from HBM; HIP events around each step
(flush excluded) give the step time.  The flush reads rather than writes: a
write leaves ~256 MB of dirty lines whose write-back would stall the next
kernel's reads (a 32 MiB cold read takes 15 us after a write flush, 8.6 us
after a read flush on this part), a cost no decode step pays.  A second pass
of K steps records the library's phase events for the
per-kernel durations used by the roofline.  The CPU oracle is timed on a sample
of whole steps on the host cores (rank 0, N=1 only).
The same run also measures the chunked prefill at 256K (a 4096-row chunk
appended to 262,144 cached keys, 32 q / 8 KV heads, 2 retrieval KV heads,
6 local heads with window 8192 + 4 sinks, p = 0.9): append of the chunk,
per-row top-p selection and gather attention of the retrieval heads, and the
causal window attention of the local heads on MFMA tiles; prefill tok/s is
4096 / step time.  Its summary goes in the "prefill" field (skip with
--no-prefill).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode μs/step + achieved HBM GB/s (% peak) at 128K–1M ctx; prefill tok/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "sparse_attention_long_retrieval_amd", "csrc")
# Sources that define the scan kernel; its counter summary is void once they change.
SCAN_SOURCES = ("decode.hip", "rtp_common.h", "rtp_internal.h", "attn_tile.h")
CALIB_BYTES = 256 << 20   # plain device copy run once per bench for counter calibration


def source_digest(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per scan launch from the committed counter summary, or None.

    The summary (profiles/traffic_k_scan_<workload>.txt) holds the FETCH_SIZE and
    WRITE_SIZE readings of the scan kernel already scaled by the plain-copy
    calibration, and the digest of the sources it was taken on.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_k_scan_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(SCAN_SOURCES):
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def flush_caches(buf) -> None:
    """Evict the Infinity Cache and L2s by reading a 512 MiB buffer (clean lines),
    twice: the reads also give the host time to queue the next step behind them."""
    buf.view(-1).sum()
    buf.view(-1).sum()


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Hip:
    """Raw HIP events from the runtime torch already loaded (same SONAME)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")

    def event(self) -> int:
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e: int, stream: int) -> None:
        assert self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a: int, b: int) -> float:
        f = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return f.value


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, choices=[2, 3, 4])
    ap.add_argument("--top-p", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true", help="prefill only (profiling)")
    ap.add_argument("--serial-streams", action="store_true",
                    help="run the decode step's local heads on the main stream too (clean "
                         "per-kernel times under a profiler; the step then does the same work "
                         "serially; the prefill step always runs on one stream)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode "
              "step would shard by (batch, KV head), each GPU running this path on its "
              "share with no exchange)", file=sys.stderr)
        return 2

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    res = {} if args.no_decode else decode_leg(args)
    if not args.no_prefill:
        res["prefill"] = prefill_leg(args)
    print(json.dumps(res), flush=True)
    return 0


def decode_leg(args):
    """The decode step (headline): returns the JSON fields of the bench line."""
    import numpy as np
    import torch

    import sparse_attention_long_retrieval_amd as R
    import workloads as W

    t0 = time.time()
    wl = W.make(args.config)
    top_p = args.top_p if args.top_p is not None else wl.top_p[min(1, len(wl.top_p) - 1)]
    log(f"workload {wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} N={wl.N} ret={wl.ret_kv_heads} "
        f"p={top_p} generated in {time.time() - t0:.1f}s")

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    layer = R.Layer(wl.B, wl.Hq, wl.Hkv, wl.N, wl.ret_kv_heads, wl.n_sink, wl.window,
                    wl.rope_base)
    N, B, G = wl.N, wl.B, wl.G
    k_cache = torch.empty((B, wl.Hkv, N, 128), dtype=torch.int16, device="cuda")
    v_cache = torch.empty_like(k_cache)
    index = torch.empty((B, wl.n_ret, N, 16), dtype=torch.int16, device="cuda")
    w_q, w_k, q = dev(wl.w_q), dev(wl.w_k), dev(wl.q_pre)
    k_pre, v_pre = dev(wl.k_pre), dev(wl.v)
    R.index_append(layer, k_pre, v_pre, w_k, 0, k_cache, v_cache, index)   # bulk prefill of caches
    new_k = k_pre[:, :, N - 1:N].contiguous()
    new_v = v_pre[:, :, N - 1:N].contiguous()
    # local heads as a ring of the sinks + the window (rtp_ring_append)
    ring_len = wl.window
    n_loc = wl.Hkv - wl.n_ret
    k_ring = torch.zeros((B, n_loc, wl.n_sink + ring_len, 128), dtype=torch.int16, device="cuda")
    v_ring = torch.zeros_like(k_ring)
    R.ring_append(layer, k_pre[:, :, :wl.n_sink].contiguous(), v_pre[:, :, :wl.n_sink].contiguous(),
                  0, ring_len, k_ring, v_ring)
    R.ring_append(layer, k_pre[:, :, N - ring_len:].contiguous(),
                  v_pre[:, :, N - ring_len:].contiguous(), N - ring_len, ring_len, k_ring, v_ring)
    del k_pre, v_pre
    out = torch.zeros((B, wl.Hq, 128), dtype=torch.int16, device="cuda")
    ws = torch.zeros(R.workspace_size(layer, R.OP_DECODE, N), dtype=torch.uint8, device="cuda")
    wss = torch.zeros(R.workspace_size(layer, R.OP_SWA, N), dtype=torch.uint8, device="cuda")
    flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device="cuda")
    # plain copy of known size: the reference point for the FETCH_SIZE / WRITE_SIZE counters
    calib_src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    for _ in range(2):
        calib_dst.copy_(calib_src)
    del calib_src, calib_dst
    torch.cuda.synchronize()
    log(f"caches built on the GPU ({time.time() - t0:.1f}s)")

    hip = Hip()
    main_s = torch.cuda.current_stream()
    # local heads run beside the retrieval chain
    side_s = main_s if args.serial_streams else torch.cuda.Stream()
    stream = main_s.cuda_stream
    n_ph = 6
    ph_events = [hip.event() for _ in range(n_ph)]
    extra = [hip.event() for _ in range(3)]
    dbg_ph = R.Debug(0, 0, events=ph_events)
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def step(debug=None, mark=False):
        cur = torch.cuda.current_stream()   # the capture stream while recording a graph
        side = cur if args.serial_streams else side_s
        if mark:
            hip.record(extra[0], cur.cuda_stream)
        R.index_append(layer, new_k, new_v, w_k, N - 1, k_cache, v_cache, index)
        fork.record(cur)
        # the retrieval decode is issued first: its kernels queue behind the append
        # while the host issues the local heads on the side stream
        R.decode_sparse_attn(layer, q, w_q, k_cache, v_cache, index, N, top_p, out, ws,
                             debug=debug)
        side.wait_event(fork)
        if mark:
            hip.record(extra[1], side.cuda_stream)
        R.swa_attn(layer, q, N - 1, 1, k_cache, v_cache, out, wss, stream=side)
        if mark:
            hip.record(extra[2], side.cuda_stream)
        join.record(side)
        cur.wait_event(join)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one untimed step with the inspection outputs: union sizes for the byte count
    dbg_sets = R.Debug(B * wl.n_ret * G, 1, pairs=B * wl.n_ret)
    step(debug=dbg_sets)
    torch.cuda.synchronize()
    union = dbg_sets.union_count.cpu().numpy().astype(np.int64)
    set_sizes = dbg_sets.sel_count.cpu().numpy().tolist()

    # ---- the step captured in a HIP graph (a serving loop may issue it this way)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(main_s)
    with torch.cuda.stream(cap):
        step()
    main_s.wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    # ---- headline: K steps, Infinity Cache flushed before each, events around each
    # step.  The flush is enqueued first, so the step's launches are queued behind it
    # and the GPU does not wait for the host inside the timed region.
    e0, e1 = hip.event(), hip.event()

    def timed(run, cold=True):
        out_ms = []
        for _ in range(args.steps):
            if cold:
                flush_caches(flush)
            hip.record(e0, stream)
            run()
            hip.record(e1, stream)
            torch.cuda.synchronize()
            out_ms.append(hip.elapsed_ms(e0, e1))
        return out_ms

    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_ms = timed(step)
    wall = time.perf_counter() - wall0
    graph_ms = timed(graph.replay)
    ms = float(np.mean(step_ms))
    log(f"cold step: mean {ms * 1e3:.1f} us, median {np.median(step_ms) * 1e3:.1f} us; "
        f"as a graph replay {np.mean(graph_ms) * 1e3:.1f} us")

    # ---- warm: K back-to-back steps without flushing (working set may sit in the
    # Infinity Cache)
    torch.cuda.synchronize()
    hip.record(e0, stream)
    for _ in range(args.steps):
        step()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    warm_ms = hip.elapsed_ms(e0, e1) / args.steps

    # ---- phases: K more cold steps with the library's phase events
    names = ["scan", "threshold", "select", "finish", "merge"]
    ph = {n: [] for n in names + ["append", "swa", "retrieval_total"]}
    for i in range(args.steps):
        flush_caches(flush)
        step(debug=dbg_ph, mark=True)
        torch.cuda.synchronize()
        for k, n in enumerate(names):
            ph[n].append(hip.elapsed_ms(ph_events[k], ph_events[k + 1]))
        ph["append"].append(hip.elapsed_ms(extra[0], ph_events[0]))
        ph["swa"].append(hip.elapsed_ms(extra[1], extra[2]))
        ph["retrieval_total"].append(hip.elapsed_ms(ph_events[0], ph_events[5]))
    phases_us = {k: round(float(np.mean(v)) * 1e3, 2) for k, v in ph.items()}

    # ---- the fixed-budget decode (the pages' ablation baseline) on the same inputs
    topk_us = {}
    for kb in (4096, 16384):
        t_ms = []
        for i in range(max(5, args.steps // 4)):
            flush_caches(flush)
            hip.record(e0, stream)
            R.decode_topk(layer, q, w_q, k_cache, v_cache, index, N, kb, out, ws)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            t_ms.append(hip.elapsed_ms(e0, e1))
        topk_us[f"top{kb}_retrieval_us"] = round(float(np.mean(t_ms)) * 1e3, 2)
    t_ms = []
    for i in range(max(5, args.steps // 4)):
        flush_caches(flush)
        hip.record(e0, stream)
        R.decode_sparse_attn(layer, q, w_q, k_cache, v_cache, index, N, top_p, out, ws)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        t_ms.append(hip.elapsed_ms(e0, e1))
    topk_us["top_p_retrieval_us"] = round(float(np.mean(t_ms)) * 1e3, 2)

    # ---- local heads from the ring versus the full cache (same kernel, same rows)
    ring = {}
    for name, kk, vv, fn in (("full_cache", k_cache, v_cache, None),
                             ("ring", k_ring, v_ring, ring_len)):
        t_ms = []
        for i in range(max(5, args.steps // 4)):
            flush_caches(flush)
            hip.record(e0, stream)
            if fn is None:
                R.swa_attn(layer, q, N - 1, 1, kk, vv, out, wss)
            else:
                R.swa_attn_ring(layer, q, N - 1, 1, fn, kk, vv, out, wss)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            t_ms.append(hip.elapsed_ms(e0, e1))
        ring[f"swa_{name}_us"] = round(float(np.mean(t_ms)) * 1e3, 2)
    ring["local_kv_bytes_full_cache"] = B * n_loc * N * 512
    ring["local_kv_bytes_ring"] = B * n_loc * (wl.n_sink + ring_len) * 512

    # ---- the V2 cluster index (K = 128 clusters, three updates) and decode through it
    K_CL, IT_CL = 128, 3
    seeds = np.stack([np.random.default_rng(wl.seed + i).choice(N, K_CL, replace=False)
                      for i in range(B * wl.n_ret)]).astype(np.int32)
    init = torch.from_numpy(seeds).cuda()
    cen = torch.empty((B * wl.n_ret, K_CL, 16), dtype=torch.float32, device="cuda")
    mem = torch.empty((B * wl.n_ret, N), dtype=torch.int32, device="cuda")
    off = torch.empty((B * wl.n_ret, K_CL + 1), dtype=torch.int32, device="cuda")
    wsb = torch.zeros(R.workspace_size(layer, R.OP_CLUSTER_BUILD, N, Tq=K_CL), dtype=torch.uint8,
                      device="cuda")
    wsc = torch.zeros(R.workspace_size(layer, R.OP_CLUSTER_DECODE, N, Tq=K_CL),
                      dtype=torch.uint8, device="cuda")
    build_ms = []
    for i in range(3):
        flush_caches(flush)
        hip.record(e0, stream)
        R.cluster_build(layer, index, N, K_CL, IT_CL, init, cen, mem, off, wsb)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        build_ms.append(hip.elapsed_ms(e0, e1))
    dbg = R.Debug(B * wl.n_ret * G, N)
    R.decode_cluster_attn(layer, q, w_q, k_cache, v_cache, cen, mem, off, K_CL, N, N, top_p,
                          out, wsc, debug=dbg)
    torch.cuda.synchronize()
    cl_sizes = [int(c) for c in dbg.sel_count.cpu().numpy()]
    del dbg
    t_ms = []
    for i in range(max(5, args.steps // 4)):
        flush_caches(flush)
        hip.record(e0, stream)
        R.decode_cluster_attn(layer, q, w_q, k_cache, v_cache, cen, mem, off, K_CL, N, N, top_p,
                              out, wsc)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        t_ms.append(hip.elapsed_ms(e0, e1))
    cluster = {"clusters": K_CL, "updates": IT_CL, "build_ms": round(float(np.mean(build_ms)), 3),
               "decode_retrieval_us": round(float(np.mean(t_ms)) * 1e3, 2),
               "top_p_retrieval_us": topk_us["top_p_retrieval_us"], "set_sizes": cl_sizes}
    del cen, mem, off, wsb, wsc, init

    # ---- algorithmic bytes of one step
    lo = max(0, N - 1 - wl.window + 1)
    swa_rows = min(wl.n_sink, lo) + (N - 1 - lo + 1)
    bytes_index = B * wl.n_ret * N * 32
    bytes_gather = int(union.sum()) * 512
    bytes_swa = B * n_loc * swa_rows * 512
    bytes_small = B * wl.Hq * 256 * 2 + wl.w_q.size * 2 + B * wl.Hkv * (512 + 512) + \
        B * wl.n_ret * 32
    step_bytes = bytes_index + bytes_gather + bytes_swa + bytes_small
    gbs = step_bytes / (ms * 1e-3) / 1e9
    score_us = phases_us["scan"]
    ach = bytes_index / (score_us * 1e-6) / 1e9

    res = {
        "metric": METRIC,
        "value": round(ms * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32 compute",
        "data": "synthetic (seeded planted-cluster keys, random-init indexer projections)",
        "config": {"workload": wl.name, "batch": B, "context": N, "q_heads": wl.Hq,
                   "kv_heads": wl.Hkv, "retrieval_kv_heads": wl.ret_kv_heads,
                   "window": wl.window, "sinks": wl.n_sink, "top_p": top_p,
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "warm_us_per_step": round(warm_ms * 1e3, 2),
        "median_us_per_step": round(float(np.median(step_ms)) * 1e3, 2),
        "graph_us_per_step": round(float(np.mean(graph_ms)) * 1e3, 2),
        "step_issue": "launched call by call (append, retrieval decode, local-head SWA on "
                      "a second stream); graph_us_per_step: the same step as one HIP "
                      "graph replay",
        "wall_s_timed": round(wall, 3),
        "set_sizes": set_sizes,
        "step_bytes": {"index": bytes_index, "gather_rows": bytes_gather, "swa": bytes_swa,
                       "small": bytes_small, "union_rows": int(union.sum())},
        "phases_us": phases_us,
        "fixed_budget": topk_us,
        "local_ring": ring,
        "cluster_index": cluster,
        "roofline": {"bound": "hbm", "kernel": "k_scan (indexer scan + mass histogram)",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name),
                     "algorithmic_bytes": bytes_index},
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, top_p, args.cpu_seconds)
    del k_cache, v_cache, index, flush, ws, wss, k_ring, v_ring
    torch.cuda.empty_cache()
    return res


def prefill_leg(args):
    """Chunked prefill at 256K: one step = append of the 4096-row chunk, retrieval
    heads (per-row top-p + gather attention), local heads (causal window attention)."""
    import numpy as np
    import torch

    import sparse_attention_long_retrieval_amd as R
    import workloads as W

    t0 = time.time()
    wl = W.make(5)
    top_p = wl.top_p[0]
    B, N, Tq, q0 = wl.B, wl.N, wl.Tq, wl.q_start
    log(f"prefill workload {wl.name}: N={N} Tq={Tq} ret={wl.ret_kv_heads} generated in "
        f"{time.time() - t0:.1f}s")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    layer = R.Layer(B, wl.Hq, wl.Hkv, N, wl.ret_kv_heads, wl.n_sink, wl.window, wl.rope_base)
    k_cache = torch.empty((B, wl.Hkv, N, 128), dtype=torch.int16, device="cuda")
    v_cache = torch.empty_like(k_cache)
    index = torch.empty((B, wl.n_ret, N, 16), dtype=torch.int16, device="cuda")
    w_q, w_k, q = dev(wl.w_q), dev(wl.w_k), dev(wl.q_pre)
    k_pre, v_pre = dev(wl.k_pre), dev(wl.v)
    R.index_append(layer, k_pre[:, :, :q0].contiguous(), v_pre[:, :, :q0].contiguous(), w_k, 0,
                   k_cache, v_cache, index)                      # the cached prefix
    ck = k_pre[:, :, q0:].contiguous()
    cv = v_pre[:, :, q0:].contiguous()
    del k_pre, v_pre
    out = torch.zeros((B, wl.Hq, Tq, 128), dtype=torch.int16, device="cuda")
    ws = torch.empty(R.workspace_size(layer, R.OP_PREFILL, N, Tq=Tq), dtype=torch.uint8,
                     device="cuda")
    flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    hip = Hip()
    main_s = torch.cuda.current_stream()
    stream = main_s.cuda_stream
    ph = [hip.event() for _ in range(5)]
    ex = [hip.event() for _ in range(4)]
    dbg_ph = R.Debug(0, 0, events=ph)

    # One stream: the index kernel keeps two blocks on every CU for its whole run, so
    # local-head blocks beside it only delay some of its blocks (measured: 15.5 ms per
    # chunk with the local heads on a second stream, 14.9 ms one after the other).
    def step(mark=False):
        if mark:
            hip.record(ex[0], stream)
        R.index_append(layer, ck, cv, w_k, q0, k_cache, v_cache, index)
        if mark:
            hip.record(ex[1], stream)
        R.swa_attn(layer, q, q0, Tq, k_cache, v_cache, out)
        if mark:
            hip.record(ex[2], stream)
        R.prefill_chunk(layer, q, q0, w_q, k_cache, v_cache, index, top_p, out, ws,
                        debug=dbg_ph if mark else None)
        if mark:
            hip.record(ex[3], stream)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    step_ms = []
    for i in range(args.prefill_steps):
        flush_caches(flush)
        hip.record(e0, stream)
        step()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        step_ms.append(hip.elapsed_ms(e0, e1))
    names = ["qprep", "index", "resolve", "attend"]
    phs = {n: [] for n in names + ["append", "swa_local", "retrieval_total", "step"]}
    for i in range(max(3, args.prefill_steps // 2)):
        flush_caches(flush)
        step(mark=True)
        torch.cuda.synchronize()
        for k, n in enumerate(names):
            phs[n].append(hip.elapsed_ms(ph[k], ph[k + 1]))
        phs["append"].append(hip.elapsed_ms(ex[0], ex[1]))
        phs["swa_local"].append(hip.elapsed_ms(ex[1], ex[2]))
        phs["retrieval_total"].append(hip.elapsed_ms(ph[0], ph[4]))
        phs["step"].append(hip.elapsed_ms(ex[0], ex[3]))
    phases_ms = {k: round(float(np.median(v)), 4) for k, v in phs.items()}
    ms = float(np.mean(step_ms))
    # the dense alternative for the retrieval heads: p = 1 selects every key, which the
    # library runs as causal flash attention on the matrix cores
    dense_ms = []
    for i in range(max(3, args.prefill_steps // 2)):
        flush_caches(flush)
        hip.record(e0, stream)
        R.prefill_chunk(layer, q, q0, w_q, k_cache, v_cache, index, 1.0, out, ws)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        dense_ms.append(hip.elapsed_ms(e0, e1))
    dense = float(np.median(dense_ms))
    # the local heads alone, without the append before them
    swa_ms = []
    for i in range(max(3, args.prefill_steps // 2)):
        flush_caches(flush)
        hip.record(e0, stream)
        R.swa_attn(layer, q, q0, Tq, k_cache, v_cache, out)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        swa_ms.append(hip.elapsed_ms(e0, e1))
    phases_ms["swa_local_alone"] = round(float(np.median(swa_ms)), 4)
    # selected rows of the chunk (set sizes from one call with the debug counts; not timed)
    n_vec = wl.B * wl.n_ret * wl.G * Tq
    dbg_cnt = R.Debug(n_vec, 1)
    R.prefill_chunk(layer, q, q0, w_q, k_cache, v_cache, index, top_p, out, ws, debug=dbg_cnt)
    torch.cuda.synchronize()
    sel = dbg_cnt.sel_count.to(torch.int64)
    sel_rows, sel_max = int(sel.sum().item()), int(sel.max().item())
    del dbg_cnt, sel
    attend_bytes = sel_rows * 2 * 128 * 2  # K and V rows, bf16
    attend_gbs = attend_bytes / (phases_ms["attend"] * 1e-3) / 1e9
    ret_flops = 4.0 * 128 * sum(q0 + t + 1 for t in range(Tq)) * wl.n_ret * wl.G * B
    # local heads: causal window attention, 4 D flops (QK + PV) per (row, key) pair
    n_loc_q = (wl.Hkv - wl.n_ret) * wl.G * B
    pairs = sum(min(q0 + t + 1, wl.window) + (wl.n_sink if q0 + t + 1 > wl.window else 0)
                for t in range(Tq))
    swa_flops = 4.0 * 128 * pairs * n_loc_q
    swa_tflops = swa_flops / (phases_ms["swa_local_alone"] * 1e-3) / 1e12
    # retrieval indexer: 2 r = 32 flops per causal (row, key) pair and retrieval q-head
    ret_pairs = sum(q0 + t + 1 for t in range(Tq)) * wl.n_ret * wl.G * B
    idx_tflops = 32.0 * ret_pairs / (phases_ms["index"] * 1e-3) / 1e12
    res = {
        "workload": wl.name, "context": N, "chunk": Tq, "top_p": top_p,
        "value": round(Tq * B / (ms * 1e-3), 1), "unit": "tok/s",
        "ms_per_chunk": round(ms, 4), "steps": args.prefill_steps,
        "phases_ms": phases_ms,
        "swa_mfma": {"kernel": "k_swa_prefill (causal window 8192 + 4 sinks, bf16 MFMA)",
                     "algorithmic_tflop": round(swa_flops / 1e12, 2),
                     "achieved": round(swa_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(swa_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        "indexer": {"kernel": "k_pf_index (scores on MFMA, mass histogram, selection)",
                    "pairs": ret_pairs, "algorithmic_tflop": round(32.0 * ret_pairs / 1e12, 3),
                    "achieved": round(idx_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(idx_tflops / MFMA_BF16_PEAK_TFLOPS, 5),
                    "scores_per_s": round(ret_pairs / (phases_ms["index"] * 1e-3), 1)},
        "attend": {"kernel": "k_pf_attend + k_pf_merge (gathered K/V rows of every selected set)",
                   "selected_rows": sel_rows, "mean_rows": round(sel_rows / n_vec, 1),
                   "max_rows": sel_max, "algorithmic_gb": round(attend_bytes / 1e9, 2),
                   "achieved": round(attend_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(attend_gbs / HBM_PEAK_GBS, 4),
                   "note": "achieved counts each selected row once per query vector; rows that "
                           "neighbouring work items share come from L2 and the Infinity Cache, "
                           "so it can exceed the HBM peak"},
        "dense_retrieval": {"kernel": "k_swa_prefill with the window = context (p = 1)",
                            "ms": round(dense, 4),
                            "tflops": round(ret_flops / (dense * 1e-3) / 1e12, 1),
                            "sparse_retrieval_ms": phases_ms["retrieval_total"],
                            "dense_over_sparse": round(dense / phases_ms["retrieval_total"], 3)},
    }
    log(f"prefill: {ms:.3f} ms/chunk -> {res['value']:.0f} tok/s; phases {phases_ms}")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(wl, top_p)
    del k_cache, v_cache, index, flush, ws
    torch.cuda.empty_cache()
    return res


def prefill_cpu_baseline(wl, top_p: float, n_rows: int = 6):
    """The oracle on a sample of chunk rows (every q-head), scaled to the whole chunk."""
    import numpy as np

    from oracle import rtp_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    t0 = time.time()
    rows_loc = np.union1d(np.arange(max(0, wl.q_start - wl.window), wl.N),
                          np.arange(min(wl.n_sink, wl.N)))
    kc, vc, idx = O.caches_for(wl, rows_needed={kv: rows_loc for kv in range(wl.Hkv)
                                                 if kv not in wl.ret_kv_heads})
    log(f"oracle prefill caches built in {time.time() - t0:.1f}s")
    rows = np.linspace(0, wl.Tq - 1, n_rows).astype(int)
    t = time.perf_counter()
    for r in rows:
        for h in range(wl.Hq):
            O.prefill_row(wl, kc, vc, idx, 0, h, int(r), top_p)
    spent = time.perf_counter() - t
    per_row = spent / len(rows)
    tok_s = 1.0 / per_row
    log(f"oracle prefill: {per_row * 1e3:.1f} ms per row (all heads)")
    return {"value": round(tok_s, 3), "unit": "tok/s", "cores": int(threads),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{len(rows)} chunk rows spread over the chunk, all {wl.Hq} q-heads each "
                      f"(append excluded), extrapolated to the {wl.Tq}-row chunk"}


def cpu_baseline(wl, top_p: float, budget_s: float):
    """Time the CPU oracle on whole decode steps of the same workload (host cores)."""
    import numpy as np

    from oracle import rtp_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    t0 = time.time()
    N = wl.N
    lo = max(0, N - wl.window)
    rows = {kv: (None if kv in wl.ret_kv_heads else
                 np.union1d(np.arange(lo, N), np.arange(min(wl.n_sink, N))))
            for kv in range(wl.Hkv)}
    kc, vc, idx = O.caches_for(wl, rows_needed=rows)
    log(f"oracle caches built in {time.time() - t0:.1f}s")
    n, spent = 0, 0.0
    while n == 0 or spent + spent / n <= budget_s:
        t = time.perf_counter()
        O.append(wl.k_pre[:, :, N - 1:N], wl.v[:, :, N - 1:N], wl.w_k, wl.ret_kv_heads, N - 1,
                 wl.rope_base)
        O.decode(wl, kc, vc, idx, top_p)
        spent += time.perf_counter() - t
        n += 1
    us = spent / n * 1e6
    log(f"oracle: {n} steps, {us / 1e3:.1f} ms/step")
    return {"value": round(us, 1), "unit": "us/step", "cores": int(threads),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{n} whole decode steps (append of the newest token + all {wl.Hq} "
                      f"heads) of the same workload; oracle caches built beforehand"}


if __name__ == "__main__":
    sys.exit(main())
