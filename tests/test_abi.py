"""C ABI contract checks that need no GPU: the library loads, exports every symbol
the header declares, and host-side validation returns its status before any
launch (only invalid arguments are passed here, so nothing is ever enqueued)."""
import ctypes
import os
import re

import pytest

import sparse_attention_long_retrieval_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtp.h")

FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced (validation fails first)
MISALIGNED = ctypes.c_void_p(0x10008)


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rtp_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = R.lib()
    declared = _declared()
    assert set(declared) >= {"rtp_index_append", "rtp_decode_sparse_attn", "rtp_prefill_chunk",
                             "rtp_swa_attn", "rtp_workspace_size"}
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.rtp_abi_version() == 1
    out = os.popen(f"nm -D --defined-only {R.LIB_PATH}").read()
    exported = sorted(set(re.findall(r" T (rtp_\w+)", out)))
    assert exported == declared, (exported, declared)


def _layer(**kw):
    args = dict(batch=1, n_q_heads=8, n_kv_heads=2, max_seq=1000, ret_kv_heads=[0])
    args.update(kw)
    return R.Layer(**args)


def _status(fn):
    try:
        fn()
    except R.RtpError as e:
        return e.status
    return 0


def test_status_strings():
    lib = R.lib()
    for s in range(8):
        assert lib.rtp_status_string(s)
    assert lib.rtp_status_string(99) == b"unknown status"


def test_workspace_query():
    lay = _layer()
    a = R.workspace_size(lay, R.OP_DECODE, 1000)
    b = R.workspace_size(lay, R.OP_DECODE, 10)
    assert a > b > 0 and a % 256 == 0
    assert R.workspace_size(lay, R.OP_APPEND, 5) == 0
    assert R.workspace_size(lay, R.OP_SWA, 1000) > 0
    assert _status(lambda: R.workspace_size(lay, R.OP_DECODE, 0)) == 4
    assert _status(lambda: R.workspace_size(lay, R.OP_DECODE, 1001)) == 4
    assert _status(lambda: R.workspace_size(lay, 17, 10)) == 4


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 5), (dict(idx_rank=8), 5), (dict(batch=0), 3),
    (dict(n_q_heads=7), 3), (dict(ret_kv_heads=[2]), 4), (dict(ret_kv_heads=[1, 0]), 4),
    (dict(ret_kv_heads=[0, 0]), 4), (dict(n_sink=-1), 4), (dict(rope_base=0.0), 4),
    (dict(n_q_heads=6, n_kv_heads=2), 5),  # G = 3 unsupported by the decode kernels
])
def test_desc_validation(kw, status):
    lay = _layer(**kw)
    lib = R.lib()
    st = lib.rtp_decode_sparse_attn(lay.desc(), FAKE, FAKE, FAKE, FAKE, FAKE, 10, 0.9, 1.0,
                                    0.088, FAKE, None, FAKE, 1 << 30, None)
    assert st == status, R.lib().rtp_last_error()


def test_decode_argument_validation():
    lay = _layer()
    lib = R.lib()
    call = lambda **o: lib.rtp_decode_sparse_attn(  # noqa: E731
        lay.desc(), o.get("q", FAKE), FAKE, FAKE, FAKE, FAKE, o.get("n", 10), o.get("p", 0.9),
        1.0, 0.088, FAKE, None, o.get("ws", FAKE), o.get("wsb", 16), None)
    assert call(q=None) == 1
    assert call(q=MISALIGNED) == 2
    assert call(n=0) == 4 and call(n=1001) == 4
    for p in (0.0, -0.5, 1.5, float("nan")):
        assert call(p=p) == 4
    assert call(ws=ctypes.c_void_p(0x10010)) == 2     # workspace must be 256-byte aligned
    assert call(wsb=16) == 6                         # workspace too small
    assert b"workspace" in lib.rtp_last_error()


def test_append_and_swa_validation():
    lay = _layer()
    lib = R.lib()
    assert lib.rtp_index_append(lay.desc(), FAKE, FAKE, FAKE, 995, 6, FAKE, FAKE, FAKE, None) == 4
    assert lib.rtp_index_append(lay.desc(), FAKE, FAKE, FAKE, -1, 1, FAKE, FAKE, FAKE, None) == 4
    assert lib.rtp_index_append(lay.desc(), FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, None) == 3
    assert lib.rtp_index_append(lay.desc(), FAKE, FAKE, None, 0, 1, FAKE, FAKE, FAKE, None) == 1
    assert lib.rtp_swa_attn(lay.desc(), FAKE, 999, 2, FAKE, FAKE, 0.088, FAKE, FAKE, 1 << 20,
                            None) == 4
    assert lib.rtp_swa_attn(_layer(window=0).desc(), FAKE, 5, 1, FAKE, FAKE, 0.088, FAKE, FAKE,
                            1 << 20, None) == 4
    assert lib.rtp_swa_attn(lay.desc(), FAKE, 5, 1, FAKE, FAKE, 0.088, FAKE, FAKE, 16,
                            None) == 6


def test_topk_validation():
    """rtp_decode_topk rejects a budget below 1 before touching any pointer."""
    import ctypes
    import sparse_attention_long_retrieval_amd as R
    layer = R.Layer(1, 4, 2, 1024, [0])
    fake = ctypes.c_void_p(0x10000)
    st = R.lib().rtp_decode_topk(layer.desc(), fake, fake, fake, fake, fake, 100, 0, 1.0,
                                 0.088, fake, None, fake, 1 << 20, None)
    assert st == 4  # RTP_ERR_RANGE


def test_ring_validation():
    """Ring calls reject a ring too short for the window or the chunk before any launch."""
    import ctypes
    import sparse_attention_long_retrieval_amd as R
    layer = R.Layer(1, 4, 2, 1024, [0], n_sink=4, window=256)
    fake = ctypes.c_void_p(0x10000)
    # a 300-row chunk needs ring_len >= 256 + 300 - 1
    st = R.lib().rtp_swa_attn_ring(layer.desc(), fake, 500, 300, 554, fake, fake, 0.088, fake,
                                   None, 0, None)
    assert st == 4
    # a call writing more tokens than ring rows
    st = R.lib().rtp_ring_append(layer.desc(), fake, fake, 0, 600, 555, fake, fake, None)
    assert st == 4


def test_cluster_validation():
    """Cluster calls reject bad sizes before any launch."""
    import ctypes
    import sparse_attention_long_retrieval_amd as R
    layer = R.Layer(1, 8, 2, 4096, [0], n_sink=4, window=256)
    fake = ctypes.c_void_p(0x10000)
    L = R.lib()
    ws = R.workspace_size(layer, R.OP_CLUSTER_BUILD, 3000, Tq=128)
    assert ws > 0
    for K, n_tok, iters, want in ((0, 3000, 2, 3), (257, 3000, 2, 3), (128, 5000, 2, 3),
                                  (128, 0, 2, 3), (128, 3000, -1, 4)):
        st = L.rtp_cluster_build(layer.desc(), fake, n_tok, K, iters, fake, fake, fake, fake,
                                 fake, ws, None)
        assert st == want, (K, n_tok, iters, st)
    st = L.rtp_cluster_build(layer.desc(), fake, 3000, 128, 2, fake, fake, fake, fake, fake,
                             ws - 1, None)
    assert st == 6
    wsd = R.workspace_size(layer, R.OP_CLUSTER_DECODE, 4000, Tq=128)
    assert wsd > 0
    for K, n_tok, seq, p, want in ((128, 4001, 4000, 0.9, 4), (128, 3000, 4097, 0.9, 4),
                                   (128, 3000, 4000, 0.0, 4), (128, 3000, 4000, 1.5, 4),
                                   (300, 3000, 4000, 0.9, 3)):
        st = L.rtp_decode_cluster_attn(layer.desc(), fake, fake, fake, fake, fake, fake, fake, K,
                                       n_tok, seq, p, 1.0, 0.088, fake, None, fake, wsd, None)
        assert st == want, (K, n_tok, seq, p, st)
    st = L.rtp_decode_cluster_attn(layer.desc(), fake, fake, fake, fake, fake, fake, fake, 128,
                                   3000, 4000, 0.9, 1.0, 0.088, fake, None, fake, wsd - 1, None)
    assert st == 6


def test_decode_grid_limit():
    """The decode launches batch * n_ret * G finish blocks in grid y: beyond 65535 the
    call and the workspace query return RTP_ERR_UNSUPPORTED before any launch."""
    lib = R.lib()
    ok = R.Layer(8191, 8, 1, 64, [0])          # 8191 * 8 = 65528 retrieval q-heads
    assert R.workspace_size(ok, R.OP_DECODE, 64) > 0
    big = R.Layer(8192, 8, 1, 64, [0])         # 65536
    assert _status(lambda: R.workspace_size(big, R.OP_DECODE, 64)) == 5
    st = lib.rtp_decode_sparse_attn(big.desc(), FAKE, FAKE, FAKE, FAKE, FAKE, 64, 0.9, 1.0,
                                    0.088, FAKE, None, FAKE, 1 << 40, None)
    assert st == 5 and b"65535" in lib.rtp_last_error()
    st = lib.rtp_decode_topk(big.desc(), FAKE, FAKE, FAKE, FAKE, FAKE, 64, 10, 1.0, 0.088, FAKE,
                             None, FAKE, 1 << 40, None)
    assert st == 5


def test_noalloc_decode_rejects_shapes_beyond_its_scratch():
    """The allocation-free decode refuses, before any HIP call, a shape whose workspace
    exceeds its static scratch; the message names both sizes."""
    lib = R.lib()
    big = R.Layer(2, 16, 2, 1 << 20, [0, 1])      # 2 * 2 * 8 q-heads x 1M keys
    need = R.workspace_size(big, R.OP_DECODE, 1 << 20)
    assert need > 80 << 20
    st = lib.rtp_decode_sparse_attn_noalloc(big.desc(), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                            0.9, 1.0, 0.088, FAKE, None, None)
    assert st == 6 and str(need).encode() in lib.rtp_last_error()
    lay = _layer()
    for n in (0, 1001):
        assert lib.rtp_decode_sparse_attn_noalloc(lay.desc(), FAKE, FAKE, FAKE, FAKE, FAKE, n,
                                                  0.9, 1.0, 0.088, FAKE, None, None) == 4
    fits = R.Layer(1, 32, 4, 1 << 20, [0])         # the 1M-context decode shape fits
    assert R.workspace_size(fits, R.OP_DECODE, 1 << 20) <= 80 << 20


def test_decode_step_validation():
    """rtp_decode_step checks the ring, the window and the workspace before any launch,
    and sizes its workspace to hold the local heads' segment states beside the decode."""
    lib = R.lib()
    lay = R.Layer(1, 8, 2, 1000, [0], n_sink=4, window=256)
    call = lambda **o: lib.rtp_decode_step(  # noqa: E731
        lay.desc(), FAKE, FAKE, FAKE, FAKE, FAKE, o.get("n", 600), o.get("ring", 0),
        o.get("kr", FAKE), o.get("vr", FAKE), o.get("p", 0.9), 1.0, 0.088, FAKE, None,
        o.get("ws", FAKE), o.get("wsb", 16), None)
    assert call(ring=-1) == 4                         # RTP_ERR_RANGE
    assert call(ring=255) == 4                        # shorter than the window
    assert call(ring=300, kr=None) == 1               # a ring needs its buffers
    assert call(n=0) == 4 and call(n=1001) == 4
    assert call(p=1.5) == 4
    assert call(wsb=16) == 6 and b"workspace" in lib.rtp_last_error()
    assert lib.rtp_decode_step(R.Layer(1, 8, 2, 1000, [0], window=0).desc(), FAKE, FAKE, FAKE,
                               FAKE, FAKE, 600, 0, None, None, 0.9, 1.0, 0.088, FAKE, None,
                               FAKE, 1 << 30, None) == 4          # local heads need a window
    # the step's workspace holds the retrieval decode's and the local segment states
    step = R.workspace_size(lay, R.OP_DECODE_STEP, 600)
    assert step > R.workspace_size(lay, R.OP_DECODE, 600)
    # no local heads: the decode's workspace; no retrieval heads: the local heads' one
    only_ret = R.Layer(1, 8, 2, 1000, [0, 1], window=256)
    assert R.workspace_size(only_ret, R.OP_DECODE_STEP, 600) == \
        R.workspace_size(only_ret, R.OP_DECODE, 600)
    only_loc = R.Layer(1, 8, 2, 1000, [], window=256)
    assert R.workspace_size(only_loc, R.OP_DECODE_STEP, 600) == \
        R.workspace_size(only_loc, R.OP_SWA, 600)
