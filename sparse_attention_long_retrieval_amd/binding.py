"""Thin ctypes binding of librtp (the C ABI in include/rtp.h).

Argument marshalling only: tensors are passed as device pointers and the current
torch stream as the HIP stream.  Every step of the attention path runs in the
HIP kernels of librtp.so; there is no fallback.  If the library is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librtp.so")

OP_DECODE, OP_PREFILL, OP_SWA, OP_APPEND = 0, 1, 2, 3
OP_CLUSTER_BUILD, OP_CLUSTER_DECODE, OP_DECODE_STEP = 4, 5, 6

STATUS = {0: "RTP_OK", 1: "RTP_ERR_NULL", 2: "RTP_ERR_ALIGN", 3: "RTP_ERR_SHAPE",
          4: "RTP_ERR_RANGE", 5: "RTP_ERR_UNSUPPORTED", 6: "RTP_ERR_WORKSPACE", 7: "RTP_ERR_HIP"}

EXPORTED = ["rtp_index_append", "rtp_decode_sparse_attn", "rtp_prefill_chunk", "rtp_swa_attn",
            "rtp_workspace_size", "rtp_status_string", "rtp_last_error", "rtp_abi_version",
            "rtp_decode_topk", "rtp_ring_append", "rtp_swa_attn_ring", "rtp_cluster_build",
            "rtp_decode_cluster_attn", "rtp_decode_sparse_attn_noalloc", "rtp_decode_step"]


class RtpError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("idx_rank", ctypes.c_int32), ("max_seq", ctypes.c_int32),
        ("n_ret", ctypes.c_int32), ("ret_kv_heads", ctypes.POINTER(ctypes.c_int32)),
        ("n_sink", ctypes.c_int32), ("window", ctypes.c_int32), ("rope_base", ctypes.c_double),
    ]


class DebugOut(ctypes.Structure):
    _fields_ = [("sel_idx", ctypes.c_void_p), ("sel_count", ctypes.c_void_p),
                ("tau", ctypes.c_void_p), ("sel_cap", ctypes.c_int32),
                ("union_count", ctypes.c_void_p), ("phase_events", ctypes.c_void_p),
                ("n_phase_events", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librtp.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_long_retrieval_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        dp = ctypes.POINTER(LayerDesc)
        L.rtp_index_append.argtypes = [dp, vp, vp, vp, i32, i32, vp, vp, vp, vp]
        L.rtp_decode_sparse_attn.argtypes = [dp, vp, vp, vp, vp, vp, i32, f32, f32, f32, vp,
                                             ctypes.POINTER(DebugOut), vp, sz, vp]
        L.rtp_decode_topk.argtypes = [dp, vp, vp, vp, vp, vp, i32, i32, f32, f32, vp,
                                      ctypes.POINTER(DebugOut), vp, sz, vp]
        L.rtp_decode_sparse_attn_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, i32, f32, f32, f32,
                                                     vp, ctypes.POINTER(DebugOut), vp]
        L.rtp_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, i32, i32, vp, vp, f32, f32, f32, vp,
                                      ctypes.POINTER(DebugOut), vp, sz, vp]
        L.rtp_prefill_chunk.argtypes = [dp, vp, i32, i32, vp, vp, vp, vp, f32, f32, f32, vp,
                                        ctypes.POINTER(DebugOut), vp, sz, vp]
        L.rtp_swa_attn.argtypes = [dp, vp, i32, i32, vp, vp, f32, vp, vp, sz, vp]
        L.rtp_ring_append.argtypes = [dp, vp, vp, i32, i32, i32, vp, vp, vp]
        L.rtp_swa_attn_ring.argtypes = [dp, vp, i32, i32, i32, vp, vp, f32, vp, vp, sz, vp]
        L.rtp_cluster_build.argtypes = [dp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.rtp_decode_cluster_attn.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                              f32, f32, f32, vp, ctypes.POINTER(DebugOut), vp,
                                              sz, vp]
        L.rtp_workspace_size.argtypes = [dp, i32, i32, i32, ctypes.POINTER(sz)]
        L.rtp_status_string.argtypes = [ctypes.c_int]
        L.rtp_status_string.restype = ctypes.c_char_p
        L.rtp_last_error.argtypes = []
        L.rtp_last_error.restype = ctypes.c_char_p
        L.rtp_abi_version.restype = ctypes.c_int32
        for name in ("rtp_index_append", "rtp_decode_sparse_attn", "rtp_decode_topk",
                     "rtp_prefill_chunk", "rtp_swa_attn", "rtp_workspace_size",
                     "rtp_ring_append", "rtp_swa_attn_ring", "rtp_cluster_build",
                     "rtp_decode_cluster_attn", "rtp_decode_sparse_attn_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise RtpError(status, lib().rtp_last_error().decode())


class Layer:
    """Layer description: sizes, retrieval KV heads, sinks, window, RoPE base."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, max_seq: int,
                 ret_kv_heads: Sequence[int], n_sink: int = 4, window: int = 8192,
                 rope_base: float = 1e6, head_dim: int = 128, idx_rank: int = 16):
        self.batch, self.n_q_heads, self.n_kv_heads = batch, n_q_heads, n_kv_heads
        self.max_seq, self.n_sink, self.window, self.rope_base = max_seq, n_sink, window, rope_base
        self.head_dim, self.idx_rank = head_dim, idx_rank
        self.ret_kv_heads = list(ret_kv_heads)
        self._ret = (ctypes.c_int32 * max(1, len(self.ret_kv_heads)))(*self.ret_kv_heads)
        self._desc = LayerDesc(batch, n_q_heads, n_kv_heads, head_dim, idx_rank, max_seq,
                               len(self.ret_kv_heads),
                               ctypes.cast(self._ret, ctypes.POINTER(ctypes.c_int32)),
                               n_sink, window, rope_base)

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_ret(self) -> int:
        return len(self.ret_kv_heads)

    def desc(self):
        return ctypes.byref(self._desc)


class Debug:
    """Device buffers for the selected sets of one call, and optional phase events
    (see rtp_debug_out).  cap = 0 requests no sets; pairs = B * n_ret enables the
    union counts; events = a sequence of raw hipEvent_t handles (ints)."""

    def __init__(self, entries: int, cap: int, device="cuda", pairs: int = 0,
                 events: Optional[Sequence[int]] = None):
        self.cap = cap
        self.sel_idx = self.sel_count = self.tau = self.union_count = None
        if cap:
            self.sel_idx = torch.full((entries, cap), -1, dtype=torch.int32, device=device)
            self.sel_count = torch.zeros(entries, dtype=torch.int32, device=device)
            self.tau = torch.zeros(entries, dtype=torch.float32, device=device)
        if pairs:
            self.union_count = torch.zeros(pairs, dtype=torch.int32, device=device)
        self._ev = None
        if events:
            self._ev = (ctypes.c_void_p * len(events))(*events)
        ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        self._s = DebugOut(ptr(self.sel_idx), ptr(self.sel_count), ptr(self.tau), cap,
                           ptr(self.union_count),
                           None if self._ev is None else ctypes.cast(self._ev, ctypes.c_void_p),
                           0 if events is None else len(events))

    def ref(self):
        return ctypes.byref(self._s)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to librtp must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(layer: Layer, op: int, seq_len: int, Tq: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rtp_workspace_size(layer.desc(), op, Tq, seq_len, ctypes.byref(n)))
    return n.value


def index_append(layer: Layer, k_pre, v, w_k, start_pos: int, k_cache, v_cache, index,
                 stream=None) -> None:
    T = k_pre.shape[2]
    _check(lib().rtp_index_append(layer.desc(), _p(k_pre), _p(v), _p(w_k), start_pos, T,
                                  _p(k_cache), _p(v_cache), _p(index), _stream(stream)))


def decode_sparse_attn(layer: Layer, q_pre, w_q, k_cache, v_cache, index, seq_len: int,
                       top_p: float, out, workspace, idx_scale: float = 1.0,
                       attn_scale: Optional[float] = None, debug: Optional[Debug] = None,
                       stream=None) -> None:
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_decode_sparse_attn(
        layer.desc(), _p(q_pre), _p(w_q), _p(k_cache), _p(v_cache), _p(index), seq_len,
        top_p, idx_scale, attn_scale, _p(out), None if debug is None else debug.ref(),
        _p(workspace), _nbytes(workspace), _stream(stream)))


def decode_step(layer: Layer, q_pre, w_q, k_cache, v_cache, index, seq_len: int, top_p: float,
                out, workspace, ring_len: int = 0, k_ring=None, v_ring=None,
                idx_scale: float = 1.0, attn_scale: Optional[float] = None,
                debug: Optional[Debug] = None, stream=None) -> None:
    """One decode step of the whole layer (rtp_decode_step): retrieval q-heads by
    dynamic top-p, local q-heads over sinks + window from the full cache (ring_len 0)
    or from the rings."""
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_decode_step(
        layer.desc(), _p(q_pre), _p(w_q), _p(k_cache), _p(v_cache), _p(index), seq_len,
        ring_len, _p(k_ring), _p(v_ring), top_p, idx_scale, attn_scale, _p(out),
        None if debug is None else debug.ref(), _p(workspace), _nbytes(workspace),
        _stream(stream)))


def decode_sparse_attn_noalloc(layer: Layer, q_pre, w_q, k_cache, v_cache, index,
                               seq_len: int, top_p: float, out, idx_scale: float = 1.0,
                               attn_scale: Optional[float] = None,
                               debug: Optional[Debug] = None, stream=None) -> None:
    """The decode step on the library's static scratch (see
    rtp_decode_sparse_attn_noalloc): no workspace argument, nothing allocated."""
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_decode_sparse_attn_noalloc(
        layer.desc(), _p(q_pre), _p(w_q), _p(k_cache), _p(v_cache), _p(index), seq_len,
        top_p, idx_scale, attn_scale, _p(out), None if debug is None else debug.ref(),
        _stream(stream)))


def decode_topk(layer: Layer, q_pre, w_q, k_cache, v_cache, index, seq_len: int, top_k: int,
                out, workspace, idx_scale: float = 1.0, attn_scale: Optional[float] = None,
                debug: Optional[Debug] = None, stream=None) -> None:
    """The decode step with a fixed budget of top_k keys per retrieval q-head."""
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_decode_topk(
        layer.desc(), _p(q_pre), _p(w_q), _p(k_cache), _p(v_cache), _p(index), seq_len,
        top_k, idx_scale, attn_scale, _p(out), None if debug is None else debug.ref(),
        _p(workspace), _nbytes(workspace), _stream(stream)))


def prefill_chunk(layer: Layer, q_pre, q_start: int, w_q, k_cache, v_cache, index,
                  top_p: float, out, workspace, idx_scale: float = 1.0,
                  attn_scale: Optional[float] = None, debug: Optional[Debug] = None,
                  stream=None) -> None:
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    Tq = q_pre.shape[2]
    _check(lib().rtp_prefill_chunk(
        layer.desc(), _p(q_pre), q_start, Tq, _p(w_q), _p(k_cache), _p(v_cache), _p(index),
        top_p, idx_scale, attn_scale, _p(out), None if debug is None else debug.ref(),
        _p(workspace), _nbytes(workspace), _stream(stream)))


def swa_attn(layer: Layer, q_pre, q_start: int, Tq: int, k_cache, v_cache, out,
             workspace=None, attn_scale: Optional[float] = None, stream=None) -> None:
    """Local heads.  Tq = 1: decode (q_pre [B][Hq][D], needs a workspace); Tq > 1: causal
    chunk (q_pre [B][Hq][Tq][D]; no workspace)."""
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_swa_attn(layer.desc(), _p(q_pre), q_start, Tq, _p(k_cache), _p(v_cache),
                              attn_scale, _p(out), _p(workspace), _nbytes(workspace),
                              _stream(stream)))


def ring_append(layer: Layer, k_pre, v, start_pos: int, ring_len: int, k_ring, v_ring,
                stream=None) -> None:
    """Write the new tokens of every local KV head into its ring (see rtp_ring_append)."""
    T = k_pre.shape[2]
    _check(lib().rtp_ring_append(layer.desc(), _p(k_pre), _p(v), start_pos, T, ring_len,
                                 _p(k_ring), _p(v_ring), _stream(stream)))


def swa_attn_ring(layer: Layer, q_pre, q_start: int, Tq: int, ring_len: int, k_ring, v_ring,
                  out, workspace=None, attn_scale: Optional[float] = None, stream=None) -> None:
    """Local heads reading K/V from their rings (see rtp_swa_attn_ring)."""
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_swa_attn_ring(layer.desc(), _p(q_pre), q_start, Tq, ring_len, _p(k_ring),
                                   _p(v_ring), attn_scale, _p(out), _p(workspace),
                                   _nbytes(workspace), _stream(stream)))


def cluster_build(layer: Layer, index, n_tokens: int, n_clusters: int, iters: int, init,
                  centroids, members, offsets, workspace, stream=None) -> None:
    """k-means cluster index over the index rows of tokens 0 .. n_tokens-1 of every
    retrieval KV head (see rtp_cluster_build); init is an int32 device tensor."""
    _check(lib().rtp_cluster_build(layer.desc(), _p(index), n_tokens, n_clusters, iters, _p(init),
                                   _p(centroids), _p(members), _p(offsets), _p(workspace),
                                   _nbytes(workspace), _stream(stream)))


def decode_cluster_attn(layer: Layer, q_pre, w_q, k_cache, v_cache, centroids, members,
                        offsets, n_clusters: int, n_tokens: int, seq_len: int, top_p: float,
                        out, workspace, idx_scale: float = 1.0,
                        attn_scale: Optional[float] = None, debug: Optional[Debug] = None,
                        stream=None) -> None:
    """The decode step through the cluster index (see rtp_decode_cluster_attn)."""
    if attn_scale is None:
        attn_scale = 1.0 / math.sqrt(layer.head_dim)
    _check(lib().rtp_decode_cluster_attn(
        layer.desc(), _p(q_pre), _p(w_q), _p(k_cache), _p(v_cache), _p(centroids), _p(members),
        _p(offsets), n_clusters, n_tokens, seq_len, top_p, idx_scale, attn_scale, _p(out),
        None if debug is None else debug.ref(), _p(workspace), _nbytes(workspace),
        _stream(stream)))
