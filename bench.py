"""Benchmark of the head-wise sparse attention step on one MI355X.

One decode step = the whole decode hot path of one layer over one batch: append of
the newest token (K/V caches + 16-dim index), then one rtp_decode_step call: the
retrieval heads (indexer scan + histogram, threshold, select, resolve, gather
attention) and the local heads (sliding window + sinks), whose window segments the
fused index pass attends while it waits for its threshold.

Headline workload: 1M-context decode shaped like Qwen3-30B-A3B attention (B=1, 32 q /
4 KV heads, KV head 0 retrieval with a 1M x 16 index, 3 SWA heads with window 8192 + 4
sinks kept in ring caches, 512 planted clusters, p = 0.9).  The same run measures the
Qwen3-8B-shaped decode at 64K (B=8) and the variable-budget decode at 128K (B=4, p in
{0.8, 0.9, 0.95}) under "configs", and the chunked prefill (a 4096-row chunk, 32 q / 8
KV heads, 2 retrieval KV heads) at 256K and at 1M context under "prefill" and
"prefill_1m".  Inputs are synthetic and seeded.

Timing: W warm-up steps, then exactly K timed steps (the headline value is their
median).  Before every timed step a read of a 512 MiB buffer evicts the working set
from the 256 MB Infinity Cache and the L2s, so each step reads its bytes from HBM;
HIP events on the step's stream bracket each step (flush excluded).  A read flush
leaves clean lines; a write flush would leave dirty lines whose write-back lands in
the next kernel.  A second series of at least 200 steps gives the median, p10 and
p90.  The parts of the step are also timed alone, cold (append; the retrieval decode
and the local heads as separate calls; the step as three calls on two streams), next
to an empty event pair, which is what a timing event pair costs by itself; a last
series records the library's phase events for the fused pass and the finish kernel
(each event adds a few microseconds to the phase it closes).  The CPU oracle is
timed on a bounded sample on the host cores (N=1 only).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode μs/step + achieved HBM GB/s (% peak) at 128K–1M ctx; prefill tok/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3
CSRC = os.path.join(ROOT, "sparse_attention_long_retrieval_amd", "csrc")
# Sources that define the fused pass; its counter summary is void once they change.
PASS_SOURCES = ("decode.hip", "rtp_common.h", "rtp_internal.h", "attn_tile.h", "swa_segment.h")
CALIB_BYTES = 256 << 20   # plain device copy run once per bench for counter calibration


def source_digest(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per fused-pass launch from the committed counter summary, or None.

    The summary (profiles/traffic_k_pass_<workload>.txt) holds the FETCH_SIZE and
    WRITE_SIZE readings of the pass kernel already scaled by the plain-copy
    calibration, and the digest of the sources it was taken on.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_k_pass_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(PASS_SOURCES):
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


def dist(ms, scale=1e3, nd=2):
    """median / p10 / p90 / mean of a list of durations in ms, scaled (default: us)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * scale
    return {"median": round(float(np.median(a)), nd), "p10": round(float(np.percentile(a, 10)), nd),
            "p90": round(float(np.percentile(a, 90)), nd), "mean": round(float(a.mean()), nd),
            "n": int(a.size)}


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


class Timer:
    """Cold timed runs: flush, event, run, event, synchronise."""

    def __init__(self, hip: Hip, flush, stream: int):
        self.hip, self.flush, self.stream = hip, flush, stream
        self.e0, self.e1 = hip.event(), hip.event()

    def runs(self, fn, n: int, cold: bool = True):
        import torch
        out = []
        for _ in range(n):
            if cold:
                flush_caches(self.flush)
            self.hip.record(self.e0, self.stream)
            fn()
            self.hip.record(self.e1, self.stream)
            torch.cuda.synchronize()
            out.append(self.hip.elapsed_ms(self.e0, self.e1))
        return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed steps of the headline")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--dist-steps", type=int, default=200,
                    help="steps of the median/p10/p90 series (at least 200 for the 1M decode)")
    ap.add_argument("--config", type=int, default=4, choices=[2, 3, 4],
                    help="headline decode workload")
    ap.add_argument("--top-p", type=float, default=None)
    ap.add_argument("--no-configs", action="store_true", help="skip the 64K and 128K decodes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-prefill", action="store_true", help="skip both prefill legs")
    ap.add_argument("--no-prefill-1m", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true", help="prefill only (profiling)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the fixed-budget, ring-cache and cluster-index comparisons")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode "
              "step would shard by (batch, KV head), each GPU running this path on its "
              "share with no exchange)", file=sys.stderr)
        return 2

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    res = {}
    if not args.no_decode:
        res = headline(args)
        if not args.no_configs and args.config == 4:
            res["configs"] = {}
            for c in (2, 3):
                name, summ = other_config(args, c)
                res["configs"][name] = summ
    if not args.no_prefill:
        res["prefill"] = prefill_leg(args, 5)
        if not args.no_prefill_1m:
            res["prefill_1m"] = prefill_leg(args, 6)
    print(json.dumps(res), flush=True)
    return 0


# ------------------------------------------------------------------ decode

class DecodeCtx:
    """A decode workload resident on the GPU: caches, index, queries, workspaces, and
    the step (append of the newest token, then one rtp_decode_step call for every
    q-head).  ring=True keeps the local heads' K/V in rings of the window."""

    def __init__(self, wl, args, ring: bool):
        import numpy as np
        import torch

        import sparse_attention_long_retrieval_amd as R
        self.R, self.wl, self.args, self.ring = R, wl, args, ring
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa
        self.layer = R.Layer(wl.B, wl.Hq, wl.Hkv, wl.N, wl.ret_kv_heads, wl.n_sink,
                             wl.window, wl.rope_base)
        N, B = wl.N, wl.B
        self.k_cache = torch.empty((B, wl.Hkv, N, 128), dtype=torch.int16, device="cuda")
        self.v_cache = torch.empty_like(self.k_cache)
        self.index = torch.empty((B, wl.n_ret, N, 16), dtype=torch.int16, device="cuda")
        self.w_q, self.w_k, self.q = dev(wl.w_q), dev(wl.w_k), dev(wl.q_pre)
        k_pre, v_pre = dev(wl.k_pre), dev(wl.v)
        R.index_append(self.layer, k_pre, v_pre, self.w_k, 0, self.k_cache, self.v_cache,
                       self.index)
        self.new_k = k_pre[:, :, N - 1:N].contiguous()
        self.new_v = v_pre[:, :, N - 1:N].contiguous()
        self.n_loc = wl.Hkv - wl.n_ret
        self.ring_len = wl.window
        if ring:
            self.k_ring = torch.zeros((B, self.n_loc, wl.n_sink + self.ring_len, 128),
                                      dtype=torch.int16, device="cuda")
            self.v_ring = torch.zeros_like(self.k_ring)
            R.ring_append(self.layer, k_pre[:, :, :wl.n_sink].contiguous(),
                          v_pre[:, :, :wl.n_sink].contiguous(), 0, self.ring_len,
                          self.k_ring, self.v_ring)
            R.ring_append(self.layer, k_pre[:, :, N - self.ring_len:].contiguous(),
                          v_pre[:, :, N - self.ring_len:].contiguous(), N - self.ring_len,
                          self.ring_len, self.k_ring, self.v_ring)
        del k_pre, v_pre
        self.out = torch.zeros((B, wl.Hq, 128), dtype=torch.int16, device="cuda")
        self.ws_step = torch.zeros(R.workspace_size(self.layer, R.OP_DECODE_STEP, N),
                                   dtype=torch.uint8, device="cuda")
        self.ws = torch.zeros(R.workspace_size(self.layer, R.OP_DECODE, N), dtype=torch.uint8,
                              device="cuda")
        self.wss = torch.zeros(R.workspace_size(self.layer, R.OP_SWA, N), dtype=torch.uint8,
                               device="cuda")
        self.main_s = torch.cuda.current_stream()
        self.side_s = torch.cuda.Stream()
        self.fork, self.join = torch.cuda.Event(), torch.cuda.Event()
        torch.cuda.synchronize()

    def append(self):
        self.R.index_append(self.layer, self.new_k, self.new_v, self.w_k, self.wl.N - 1,
                            self.k_cache, self.v_cache, self.index)

    def decode_step(self, top_p, debug=None):
        R, N = self.R, self.wl.N
        if self.ring:
            R.decode_step(self.layer, self.q, self.w_q, self.k_cache, self.v_cache, self.index,
                          N, top_p, self.out, self.ws_step, ring_len=self.ring_len,
                          k_ring=self.k_ring, v_ring=self.v_ring, debug=debug)
        else:
            R.decode_step(self.layer, self.q, self.w_q, self.k_cache, self.v_cache, self.index,
                          N, top_p, self.out, self.ws_step, debug=debug)

    def step(self, top_p, debug=None):
        """The timed step: append, then the whole layer's decode in one call."""
        self.append()
        self.decode_step(top_p, debug=debug)

    def retrieval(self, top_p):
        self.R.decode_sparse_attn(self.layer, self.q, self.w_q, self.k_cache, self.v_cache,
                                  self.index, self.wl.N, top_p, self.out, self.ws)

    def local(self, stream=None):
        R, N = self.R, self.wl.N
        if self.ring:
            R.swa_attn_ring(self.layer, self.q, N - 1, 1, self.ring_len, self.k_ring,
                            self.v_ring, self.out, self.wss, stream=stream)
        else:
            R.swa_attn(self.layer, self.q, N - 1, 1, self.k_cache, self.v_cache, self.out,
                       self.wss, stream=stream)

    def step_separate(self, top_p):
        """The same step as three calls: append, retrieval decode, and the local heads on
        a second stream beside the retrieval decode."""
        import torch
        cur = torch.cuda.current_stream()
        self.append()
        self.fork.record(cur)
        self.retrieval(top_p)
        self.side_s.wait_event(self.fork)
        self.local(stream=self.side_s)
        self.join.record(self.side_s)
        cur.wait_event(self.join)

    def measure(self, top_p, timer, hip, n_steps, n_dist, n_phase):
        """Step times (K cold steps + a distribution series), the parts alone, the
        library's phases, set sizes, bytes."""
        import numpy as np
        import torch
        R, wl = self.R, self.wl
        B, N = wl.B, wl.N
        for _ in range(self.args.warmup):
            self.step(top_p)
        torch.cuda.synchronize()
        # one untimed step with the inspection outputs: set and union sizes
        dbg_sets = R.Debug(B * wl.n_ret * wl.G, 1, pairs=B * wl.n_ret)
        self.step(top_p, debug=dbg_sets)
        torch.cuda.synchronize()
        union = dbg_sets.union_count.cpu().numpy().astype(np.int64)
        sizes = dbg_sets.sel_count.cpu().numpy().astype(np.int64)
        del dbg_sets
        step_ms = timer.runs(lambda: self.step(top_p), n_steps)
        dist_ms = timer.runs(lambda: self.step(top_p), n_dist) if n_dist > n_steps else step_ms
        med = lambda ms: round(float(np.median(ms)) * 1e3, 2)  # noqa: E731
        # the parts alone (cold), and what an empty event pair costs
        parts_us = {
            "event_pair": med(timer.runs(lambda: None, n_phase)),
            "append": med(timer.runs(self.append, n_phase)),
            "decode_step": med(timer.runs(lambda: self.decode_step(top_p), n_phase)),
            "retrieval_decode": med(timer.runs(lambda: self.retrieval(top_p), n_phase)),
            "local_heads": med(timer.runs(self.local, n_phase)),
            "step_as_three_calls": med(timer.runs(lambda: self.step_separate(top_p), n_phase)),
        }
        # phases inside the decode step: the library's events on its launch stream
        ph_ev = [hip.event() for _ in range(6)]
        dbg_ph = R.Debug(0, 0, events=ph_ev)
        ph = {"pass": [], "finish": []}
        for _ in range(n_phase):
            flush_caches(timer.flush)
            self.append()
            self.decode_step(top_p, debug=dbg_ph)
            torch.cuda.synchronize()
            ph["pass"].append(hip.elapsed_ms(ph_ev[0], ph_ev[1]))
            ph["finish"].append(hip.elapsed_ms(ph_ev[3], ph_ev[4]))
        phases_us = {k: round(float(np.median(v)) * 1e3, 2) for k, v in ph.items()}
        # algorithmic bytes of one step
        lo = max(0, N - wl.window)
        swa_rows = min(wl.n_sink, lo) + (N - lo)
        b_index = B * wl.n_ret * N * 32
        b_gather = int(union.sum()) * 512
        b_local = B * self.n_loc * swa_rows * 512
        b_small = B * wl.Hq * 256 * 2 + wl.w_q.size * 2 + B * wl.Hkv * (512 + 512) + \
            B * wl.n_ret * 32
        step_bytes = b_index + b_gather + b_local + b_small
        med_ms = float(np.median(step_ms))
        gbs = lambda b, us: round(b / (us * 1e-6) / 1e9, 1)  # noqa: E731
        return {
            "top_p": top_p,
            "us_per_step": dist(step_ms),
            "us_per_step_dist": dist(dist_ms),
            "parts_us": parts_us,
            "phases_us": phases_us,
            "set_sizes": {"min": int(sizes.min()), "median": float(np.median(sizes)),
                          "max": int(sizes.max()), "all": sizes.tolist() if sizes.size <= 32
                          else None},
            "union_rows": int(union.sum()),
            "step_bytes": {"index": b_index, "gather_rows": b_gather, "local_window": b_local,
                           "small": b_small, "total": step_bytes},
            "achieved_GBps": gbs(step_bytes, med_ms * 1e3),
            "hbm_frac": round(step_bytes / (med_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "pass_streamed_GBps": gbs(b_index + b_local, phases_us["pass"]),
            "_step_ms": step_ms,
        }

    def free(self):
        import torch
        for a in ("k_cache", "v_cache", "index", "k_ring", "v_ring", "ws", "wss", "ws_step",
                  "out"):
            if hasattr(self, a):
                delattr(self, a)
        torch.cuda.empty_cache()


def attainable_read(timer):
    """Cold streaming reads with a plain read kernel (libreadprobe.so, built beside the
    library): the 32 MiB of the 1M index and 1 GiB, in GB/s, median of 20, best of
    four grid sizes.  This is what one kernel reading that many bytes reaches here,
    launch and ramp included, timed the way the decode kernels are."""
    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_long_retrieval_amd",
                                   "libreadprobe.so"))
    lib.read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_void_p]
    out = torch.zeros(1 << 14, dtype=torch.int32, device="cuda")
    res = {}
    for name, nbytes in (("32MiB", 32 << 20), ("1GiB", 1 << 30)):
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        best = 0.0
        for blocks in (1024, 2048, 4096, 8192):
            fn = lambda: lib.read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks,  # noqa
                                        timer.stream)
            assert fn() == 0
            ms = timer.runs(fn, 20)
            best = max(best, nbytes / (float(np.median(ms)) * 1e-3) / 1e9)
        res[name] = round(best, 1)
        del buf
    res["kernel"] = "k_read_probe (16-byte loads, four in flight per thread), cold, HIP events"
    return res


def headline(args):
    """The 1M decode step (headline), with its extras; returns the bench line fields."""
    import numpy as np
    import torch

    import sparse_attention_long_retrieval_amd as R
    import workloads as W

    t0 = time.time()
    wl = W.make(args.config)
    top_p = args.top_p if args.top_p is not None else wl.top_p[min(1, len(wl.top_p) - 1)]
    log(f"workload {wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} N={wl.N} ret={wl.ret_kv_heads} "
        f"p={top_p} generated in {time.time() - t0:.1f}s")
    ctx = DecodeCtx(wl, args, ring=True)
    N, B, G = wl.N, wl.B, wl.G
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
    stream = ctx.main_s.cuda_stream
    timer = Timer(hip, flush, stream)
    m = ctx.measure(top_p, timer, hip, args.steps, max(args.dist_steps, args.steps), args.steps)
    step_ms = m.pop("_step_ms")
    log(f"cold step: median {m['us_per_step']['median']} us over {args.steps}; "
        f"{m['us_per_step_dist']}")

    # ---- the step captured in a HIP graph (a serving loop may issue it this way)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(ctx.main_s)
    with torch.cuda.stream(cap):
        ctx.step(top_p)
    ctx.main_s.wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        ctx.step(top_p)
    torch.cuda.synchronize()
    graph_ms = timer.runs(graph.replay, args.steps)
    # warm: back-to-back steps without flushing (working set may sit in the Infinity Cache)
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(e0, stream)
    for _ in range(args.steps):
        ctx.step(top_p)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    warm_ms = hip.elapsed_ms(e0, e1) / args.steps

    extras = {}
    if not args.no_extras:
        extras = decode_extras(ctx, top_p, timer, args)
    reads = attainable_read(timer)
    ms = float(np.median(step_ms))
    ph = m["phases_us"]
    b_pass = m["step_bytes"]["index"] + m["step_bytes"]["local_window"]
    ach = b_pass / (ph["pass"] * 1e-6) / 1e9
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
        "value_stat": "median of the K timed cold steps",
        "us_per_step": m["us_per_step"],
        "us_per_step_dist": m["us_per_step_dist"],
        "achieved_GBps": m["achieved_GBps"],
        "hbm_frac": m["hbm_frac"],
        "attainable_read_GBps": reads,
        "hbm_frac_of_attainable": round(m["achieved_GBps"] / reads["1GiB"], 4),
        "warm_us_per_step": round(warm_ms * 1e3, 2),
        "graph_us_per_step": dist(graph_ms),
        "step_issue": "append, then one rtp_decode_step call (retrieval and local heads); "
                      "graph_us_per_step: the same step as one HIP graph replay",
        "set_sizes": m["set_sizes"],
        "union_rows": m["union_rows"],
        "step_bytes": m["step_bytes"],
        "parts_us": m["parts_us"],
        "phases_us": ph,
        "phase_GBps": {"pass_streamed": m["pass_streamed_GBps"]},
        "roofline": {"bound": "hbm",
                     "kernel": "k_pass (fused index scan, threshold, definite rows and the "
                               "local heads' window segments)",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "frac_of_attainable_32MiB": round(ach / reads["32MiB"], 4),
                     "traffic": measured_traffic(wl.name),
                     "algorithmic_bytes": b_pass,
                     "bytes_note": "the index and the local window rows, each read once; "
                                   "the definite-row gathers of the pass are not counted"},
    }
    res.update(extras)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, top_p, args.cpu_seconds)
    ctx.free()
    del flush
    torch.cuda.empty_cache()
    return res


def decode_extras(ctx, top_p, timer, args):
    """Fixed budgets, the ring cache against the full cache, the cluster index."""
    import numpy as np
    import torch
    R, wl = ctx.R, ctx.wl
    N, B, G = wl.N, wl.B, wl.G
    n = max(5, args.steps // 4)
    med = lambda ms: round(float(np.median(ms)) * 1e3, 2)  # noqa: E731
    topk = {}
    for kb in (4096, 16384):
        topk[f"top{kb}_retrieval_us"] = med(timer.runs(
            lambda: R.decode_topk(ctx.layer, ctx.q, ctx.w_q, ctx.k_cache, ctx.v_cache,
                                  ctx.index, N, kb, ctx.out, ctx.ws), n))
    topk["top_p_retrieval_us"] = med(timer.runs(
        lambda: R.decode_sparse_attn(ctx.layer, ctx.q, ctx.w_q, ctx.k_cache, ctx.v_cache,
                                     ctx.index, N, top_p, ctx.out, ctx.ws), n))
    topk["top_p_noalloc_retrieval_us"] = med(timer.runs(
        lambda: R.decode_sparse_attn_noalloc(ctx.layer, ctx.q, ctx.w_q, ctx.k_cache,
                                             ctx.v_cache, ctx.index, N, top_p, ctx.out), n))
    ring = {
        "swa_full_cache_us": med(timer.runs(
            lambda: R.swa_attn(ctx.layer, ctx.q, N - 1, 1, ctx.k_cache, ctx.v_cache, ctx.out,
                               ctx.wss), n)),
        "swa_ring_us": med(timer.runs(
            lambda: R.swa_attn_ring(ctx.layer, ctx.q, N - 1, 1, ctx.ring_len, ctx.k_ring,
                                    ctx.v_ring, ctx.out, ctx.wss), n)),
        "local_kv_bytes_full_cache": B * ctx.n_loc * N * 512,
        "local_kv_bytes_ring": B * ctx.n_loc * (wl.n_sink + ctx.ring_len) * 512,
    }
    K_CL, IT_CL = 128, 3
    seeds = np.stack([np.random.default_rng(wl.seed + i).choice(N, K_CL, replace=False)
                      for i in range(B * wl.n_ret)]).astype(np.int32)
    init = torch.from_numpy(seeds).cuda()
    cen = torch.empty((B * wl.n_ret, K_CL, 16), dtype=torch.float32, device="cuda")
    mem = torch.empty((B * wl.n_ret, N), dtype=torch.int32, device="cuda")
    off = torch.empty((B * wl.n_ret, K_CL + 1), dtype=torch.int32, device="cuda")
    wsb = torch.zeros(R.workspace_size(ctx.layer, R.OP_CLUSTER_BUILD, N, Tq=K_CL),
                      dtype=torch.uint8, device="cuda")
    wsc = torch.zeros(R.workspace_size(ctx.layer, R.OP_CLUSTER_DECODE, N, Tq=K_CL),
                      dtype=torch.uint8, device="cuda")
    build_ms = timer.runs(lambda: R.cluster_build(ctx.layer, ctx.index, N, K_CL, IT_CL, init,
                                                  cen, mem, off, wsb), 3)
    dbg = R.Debug(B * wl.n_ret * G, N)
    R.decode_cluster_attn(ctx.layer, ctx.q, ctx.w_q, ctx.k_cache, ctx.v_cache, cen, mem, off,
                          K_CL, N, N, top_p, ctx.out, wsc, debug=dbg)
    torch.cuda.synchronize()
    cl_sizes = [int(c) for c in dbg.sel_count.cpu().numpy()]
    del dbg
    cl_us = med(timer.runs(
        lambda: R.decode_cluster_attn(ctx.layer, ctx.q, ctx.w_q, ctx.k_cache, ctx.v_cache, cen,
                                      mem, off, K_CL, N, N, top_p, ctx.out, wsc), n))
    cluster = {"clusters": K_CL, "updates": IT_CL,
               "build_ms": round(float(np.median(build_ms)), 3),
               "decode_retrieval_us": cl_us, "top_p_retrieval_us": topk["top_p_retrieval_us"],
               "set_sizes": cl_sizes}
    return {"fixed_budget": topk, "local_ring": ring, "cluster_index": cluster}


def other_config(args, config: int):
    """The 64K (B=8) or 128K (B=4, three p) decode: step distribution, phases, sizes."""
    import torch

    import workloads as W
    t0 = time.time()
    wl = W.make(config)
    log(f"workload {wl.name}: B={wl.B} N={wl.N} p={wl.top_p} generated in "
        f"{time.time() - t0:.1f}s")
    ctx = DecodeCtx(wl, args, ring=False)
    flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device="cuda")
    hip = Hip()
    timer = Timer(hip, flush, ctx.main_s.cuda_stream)
    out = {"batch": wl.B, "context": wl.N, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
           "retrieval_kv_heads": wl.ret_kv_heads, "window": wl.window, "runs": {}}
    n_dist = max(100, args.steps)
    for p in wl.top_p:
        m = ctx.measure(p, timer, hip, args.steps, n_dist, max(10, args.steps // 2))
        m.pop("_step_ms")
        out["runs"][f"p{p}"] = m
        log(f"{wl.name} p={p}: median {m['us_per_step']['median']} us, "
            f"{m['achieved_GBps']} GB/s, sets {m['set_sizes']['min']}..{m['set_sizes']['max']}")
    ctx.free()
    del flush
    torch.cuda.empty_cache()
    return wl.name, out


# ------------------------------------------------------------------ prefill

def prefill_leg(args, config: int):
    """Chunked prefill: one step = append of the 4096-row chunk, the local heads (causal
    window attention on MFMA tiles), the retrieval heads (per-row top-p + gather
    attention), all on one stream.  prefill tok/s = 4096 / step time."""
    import numpy as np
    import torch

    import sparse_attention_long_retrieval_amd as R
    import workloads as W

    t0 = time.time()
    wl = W.make(config)
    top_p = wl.top_p[0]
    B, N, Tq, q0 = wl.B, wl.N, wl.Tq, wl.q_start
    log(f"prefill workload {wl.name}: N={N} Tq={Tq} ret={wl.ret_kv_heads} generated in "
        f"{time.time() - t0:.1f}s")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa
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
    ws_bytes = R.workspace_size(layer, R.OP_PREFILL, N, Tq=Tq)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    timer = Timer(hip, flush, stream)
    ph = [hip.event() for _ in range(5)]
    ex = [hip.event() for _ in range(4)]
    dbg_ph = R.Debug(0, 0, events=ph)

    # One stream: the index kernel keeps two blocks on every CU for its whole run, so
    # local-head blocks beside it only delay some of its blocks.
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
    n_steps = args.prefill_steps if config == 5 else max(10, args.prefill_steps // 2)
    step_ms = timer.runs(step, n_steps)
    names = ["qprep", "index", "resolve", "attend"]
    phs = {n: [] for n in names + ["append", "swa_local", "retrieval_total", "step"]}
    for _ in range(max(5, n_steps // 4)):
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
    ms = float(np.median(step_ms))
    # the dense alternative for the retrieval heads: p = 1 selects every key, which the
    # library runs as causal flash attention on the matrix cores
    dense_ms = timer.runs(lambda: R.prefill_chunk(layer, q, q0, w_q, k_cache, v_cache, index,
                                                  1.0, out, ws), max(5, n_steps // 4))
    dense = float(np.median(dense_ms))
    swa_ms = timer.runs(lambda: R.swa_attn(layer, q, q0, Tq, k_cache, v_cache, out),
                        max(5, n_steps // 4))
    phases_ms["swa_local_alone"] = round(float(np.median(swa_ms)), 4)
    # selected rows of the chunk (set sizes and the union per KV head from one call with
    # the inspection outputs; not timed)
    n_vec = wl.B * wl.n_ret * wl.G * Tq
    dbg_cnt = R.Debug(n_vec, 1, pairs=B * wl.n_ret)
    R.prefill_chunk(layer, q, q0, w_q, k_cache, v_cache, index, top_p, out, ws, debug=dbg_cnt)
    torch.cuda.synchronize()
    sel = dbg_cnt.sel_count.to(torch.int64)
    sel_rows, sel_max = int(sel.sum().item()), int(sel.max().item())
    sel_med = float(sel.float().median().item())
    union_rows = int(dbg_cnt.union_count.to(torch.int64).sum().item())
    del dbg_cnt, sel
    # attend: algorithmic bytes are the distinct selected K/V rows (512 B each) of each
    # retrieval KV head over the chunk; every further read of a row is a re-read
    att_s = phases_ms["attend"] * 1e-3
    attend_bytes = union_rows * 512
    reread_bytes = sel_rows * 512
    attend_flops = 4.0 * 128 * sel_rows          # QK and PV, 2 flops per multiply-add
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
        "ms_per_chunk": dist(step_ms, 1.0, 4), "steps": n_steps,
        "workspace_bytes": ws_bytes,
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
                   "median_rows": sel_med, "max_rows": sel_max,
                   "distinct_rows": union_rows,
                   "algorithmic_bytes": attend_bytes,
                   "achieved": round(attend_bytes / att_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(attend_bytes / att_s / 1e9 / HBM_PEAK_GBS, 4),
                   "row_reads_bytes": reread_bytes,
                   "row_reads_GBps": round(reread_bytes / att_s / 1e9, 1),
                   "flops": attend_flops,
                   "tflops": round(attend_flops / att_s / 1e12, 2),
                   "fp32_valu_frac": round(attend_flops / att_s / 1e12 / FP32_VALU_PEAK_TFLOPS, 4),
                   "note": "algorithmic bytes count each distinct selected row of a KV head "
                           "once; row_reads counts every (row, query vector) read, most of "
                           "which hit L2 and the Infinity Cache"},
        "dense_retrieval": {"kernel": "k_swa_prefill with the window = context (p = 1)",
                            "ms": round(dense, 4),
                            "tflops": round(ret_flops / (dense * 1e-3) / 1e12, 1),
                            "mfma_frac": round(ret_flops / (dense * 1e-3) / 1e12 /
                                               MFMA_BF16_PEAK_TFLOPS, 4),
                            "sparse_retrieval_ms": phases_ms["retrieval_total"],
                            "dense_over_sparse": round(dense / phases_ms["retrieval_total"], 3)},
    }
    log(f"prefill {wl.name}: {ms:.3f} ms/chunk -> {res['value']:.0f} tok/s; phases {phases_ms}")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(wl, top_p, n_rows=6 if config == 5 else 2)
    del k_cache, v_cache, index, flush, ws
    torch.cuda.empty_cache()
    return res


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return 1


def prefill_cpu_baseline(wl, top_p: float, n_rows: int = 6):
    """The oracle on a sample of chunk rows (every q-head), scaled to the whole chunk."""
    import numpy as np

    from oracle import rtp_oracle as O
    t0 = time.time()
    rows = np.linspace(0, wl.Tq - 1, n_rows).astype(int)
    pos = wl.q_start + rows
    win = np.unique(np.concatenate([np.arange(max(0, p - wl.window + 1), p + 1) for p in pos] +
                                   [np.arange(min(wl.n_sink, wl.N))]))
    kc, vc, idx = O.caches_for(wl, rows_needed={kv: win for kv in range(wl.Hkv)
                                                 if kv not in wl.ret_kv_heads})
    log(f"oracle prefill caches built in {time.time() - t0:.1f}s")
    t = time.perf_counter()
    for r in rows:
        for h in range(wl.Hq):
            O.prefill_row(wl, kc, vc, idx, 0, h, int(r), top_p)
    spent = time.perf_counter() - t
    per_row = spent / len(rows)
    log(f"oracle prefill {wl.name}: {per_row * 1e3:.1f} ms per row (all heads)")
    return {"value": round(1.0 / per_row, 3), "unit": "tok/s", "cores": int(_threads()),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{len(rows)} chunk rows spread over the chunk, all {wl.Hq} q-heads each "
                      f"(append excluded), extrapolated to the {wl.Tq}-row chunk"}


def cpu_baseline(wl, top_p: float, budget_s: float):
    """Time the CPU oracle on whole decode steps of the same workload (host cores)."""
    import numpy as np

    from oracle import rtp_oracle as O
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
    return {"value": round(us, 1), "unit": "us/step", "cores": int(_threads()),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{n} whole decode steps (append of the newest token + all {wl.Hq} "
                      f"heads) of the same workload; oracle caches built beforehand"}


if __name__ == "__main__":
    sys.exit(main())
