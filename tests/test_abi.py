"""The C-ABI library on the host: it loads, exports every declared entry point,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import chunk_wise_sparse_summary_amd as hils

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hils.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hils_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(hils.EXPORTS)
    L = hils.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    L = hils.lib()
    assert L.hils_abi_version() == 3
    for code in hils.STATUS:
        assert L.hils_status_string(code)
    assert L.hils_status_string(-99) == b"unknown status"


def _shape(**kw):
    base = dict(B=1, Hq=32, Hkv=8, d=128, S=64, W=1024, k=32, T=131072, dtype="bf16")
    base.update(kw)
    return hils.Shape.make(base["B"], base["Hq"], base["Hkv"], base["d"], base["S"], base["W"],
                           base["k"], base["T"], base["dtype"])


def test_workspace_sizes():
    s = _shape()
    assert hils.hils_workspace_bytes(s, hils.OP_SUMMARIZE) == 0
    sel = hils.hils_workspace_bytes(s, hils.OP_SELECT)
    att = hils.hils_workspace_bytes(s, hils.OP_ATTEND_FUSE)
    # partial outputs: B*Hq*T*k*d bf16 dominate the attend workspace
    assert att >= 32 * 131072 * 32 * 128 * 2
    assert 0 < sel < att
    d = _shape(B=4, T=524544, k=32)
    assert hils.hils_workspace_bytes(d, hils.OP_DECODE) > 4 * 32 * (524544 // 64) * 4
    assert hils.hils_workspace_bytes(_shape(S=32), hils.OP_SELECT) == 0     # unsupported
    assert hils.hils_workspace_bytes(_shape(Hq=12, Hkv=8), hils.OP_SELECT) == 0


def _call_select(shape, q=16, ks=16, bs=16, idx=16, sc=16, ws=16, nws=1 << 40):
    L = hils.lib()
    P = ctypes.c_void_p
    return L.hils_select(ctypes.byref(shape), P(q), P(ks), P(bs), P(idx), P(sc), P(ws), nws, None)


def test_validation_before_launch():
    L = hils.lib()
    P = ctypes.c_void_p
    assert _call_select(_shape(), q=0) == -1                       # NULL
    assert _call_select(_shape(), q=8) == -4                       # alignment
    assert _call_select(_shape(Hq=30)) == -2                       # Hq % Hkv
    assert _call_select(_shape(d=96)) == -8                        # unsupported head dim
    assert _call_select(_shape(k=65)) == -8
    assert _call_select(_shape(T=64 * 8193)) == -8                 # > 8192 chunks
    assert _call_select(_shape(), nws=10) == -5                    # workspace
    bad = _shape()
    bad.io_dtype = 7
    assert _call_select(bad) == -3
    neg = _shape()
    neg.scale = -1.0
    assert _call_select(neg) == -2
    assert L.hils_select(None, P(16), P(16), P(16), P(16), P(16), P(16), 1 << 40, None) == -1
    # summarize: chunk range beyond the sequence
    s = _shape()
    assert L.hils_summarize(ctypes.byref(s), P(16), P(16), 2047, 2, P(16), P(16), None) == -2
    assert L.hils_summarize(ctypes.byref(s), P(16), P(16), -1, 1, P(16), P(16), None) == -2
    assert L.hils_summarize(ctypes.byref(s), P(16), P(16), 0, 0, P(16), P(16), None) == 0  # no-op
    # attend: workspace below one KV head's share
    assert L.hils_attend_fuse(ctypes.byref(s), P(16), P(16), P(16), P(16), P(16), P(16), P(16),
                              P(16), 1024, None) == -5


def test_select_qcal_validation():
    """The fused select + Q-Cal call checks everything before launching."""
    L = hils.lib()
    P = ctypes.c_void_p
    s = _shape()
    need = L.hils_select_qcal_workspace_bytes(ctypes.byref(s), 64)
    # z (B T rank fp32, 256-byte padded) ahead of the selection's own workspace
    assert need >= hils.hils_workspace_bytes(s, hils.OP_SELECT) + s.batch * s.seq_len * 64 * 4
    assert L.hils_select_qcal_workspace_bytes(ctypes.byref(s), 48) == 0

    def call(q=16, qh=32, rank=64, dm=4096, nws=need, shape=s):
        return L.hils_select_qcal(ctypes.byref(shape), P(q), P(16), P(16), P(16), dm, rank, P(16), P(16),
                                  P(qh), P(16), P(16), P(16), nws, None)

    assert call(q=0) == -1
    assert call(q=8) == -4
    assert call(rank=48) == -8
    assert call(dm=100) == -8
    assert call(q=16, qh=16) == -2             # q_hat must not alias q
    assert call(nws=1024) == -5                  # below z
    assert call(nws=s.batch * s.seq_len * 64 * 4 + 1024) == -5   # z, but no room for the rank keys
    assert call(shape=_shape(d=96)) == -8


def test_decode_validation():
    L = hils.lib()
    P = ctypes.c_void_p
    s = _shape(B=2, T=4096, k=8, W=128)
    ws = hils.hils_workspace_bytes(s, hils.OP_DECODE)
    assert ws > 0

    def call(pos, qland=16, nws=ws):
        arr = (ctypes.c_int64 * 2)(*pos)
        a = [P(16)] * 4
        return L.hils_decode_step(ctypes.byref(s), arr, *a, P(qland), P(16), P(16), P(16), P(16),
                                  P(16), P(16), P(16), P(16), nws, None)

    assert call([0, 4096]) == -6          # position beyond the cache
    assert call([-1, 3]) == -6
    assert call([62, 63], qland=0) == -7  # sequence 1 completes chunk 0 and no q_land
    assert call([5, 6], nws=ws - 1) == -5
    s2 = _shape(B=2, T=4000, k=8, W=128)  # capacity not a multiple of S
    arr = (ctypes.c_int64 * 2)(1, 2)
    assert L.hils_decode_step(ctypes.byref(s2), arr, *[P(16)] * 13, 1 << 30, None) == -2
    s3 = _shape(B=65, T=4096, k=8)
    arr3 = (ctypes.c_int64 * 65)(*([1] * 65))
    assert L.hils_decode_step(ctypes.byref(s3), arr3, *[P(16)] * 13, 1 << 30, None) == -8


def test_decode_multi_item_limit():
    """A multi-query row fuses k selected chunks and the union of M windows, one
    chunk more than a single window spans: k + W/S + 3 items at most 256."""
    ok = _shape(B=1, T=65536, k=64, W=189 * 64)       # 64 + 189 + 3 = 256
    edge = _shape(B=1, T=65536, k=64, W=190 * 64)     # 257 with M > 1
    assert hils.hils_decode_multi_workspace_bytes(ok, 4) > 0
    assert hils.hils_decode_multi_workspace_bytes(edge, 4) == 0
    assert hils.hils_decode_multi_workspace_bytes(edge, 1) > 0   # M = 1 is the single-query step
    assert hils.hils_workspace_bytes(edge, hils.OP_DECODE) > 0


def test_timing_names_and_errors():
    L = hils.lib()
    assert L.hils_timing_enable(b"no_such_kernel") == -8
    assert L.hils_timing_enable(b"chunk_attend,window") == 0
    ms, n = hils.hils_timing_get("chunk_attend")
    assert (ms, n) == (0.0, 0)
    with pytest.raises(hils.HilsError):
        hils.hils_timing_get("nope")
    assert L.hils_timing_get(b"window", None, None) == -1
    for k in hils.KERNELS:
        hils.hils_timing_enable([k])
    hils.hils_timing_enable("*")
    hils.hils_timing_enable(None)


def test_backward_validation():
    L = hils.lib()
    P = ctypes.c_void_p
    s = _shape(T=8192, k=16, W=512)
    full = hils.hils_workspace_bytes(s, hils.OP_ATTEND_BACKWARD)
    # dq parts of every (query, head, selected chunk), in the bf16 I/O dtype, dominate
    assert full >= 32 * 8192 * 16 * 128 * 2

    def call(ptrs=None, nws=full, shape=s, dlse=16):
        a = [P(16)] * 17 if ptrs is None else ptrs
        a = list(a)
        a[10] = P(dlse)
        return L.hils_attend_fuse_backward(ctypes.byref(shape), *a, P(16), nws, None)

    bad = [P(16)] * 17
    bad[0] = P(0)
    assert call(bad) == -1                       # q NULL
    bad = [P(16)] * 17
    bad[11] = P(8)
    assert call(bad) == -4                       # dq misaligned
    assert call(nws=1024) == -5                  # workspace below one KV head's share
    assert call(shape=_shape(T=8192, k=16, W=512, d=96)) == -8
    assert hils.hils_workspace_bytes(_shape(d=96), hils.OP_ATTEND_BACKWARD) == 0
    # summarize backward: range checks and the no-op
    assert L.hils_summarize_backward(ctypes.byref(s), P(16), P(16), P(16), P(16), 127, 2, P(16), P(16),
                                     None) == -2
    assert L.hils_summarize_backward(ctypes.byref(s), P(16), P(16), P(16), P(16), 0, 0, P(16), P(16),
                                     None) == 0
    assert L.hils_summarize_backward(ctypes.byref(s), P(0), P(16), P(16), P(16), 0, 1, P(16), P(16),
                                     None) == -1


def _nc(i, S, W):
    a = i - W + 1
    return 0 if a <= 0 else a // S


@pytest.mark.parametrize("T", [37, 64, 150, 192, 1000])
def test_short_sequences_tile_and_workspace_math(T):
    """Host model of the selection kernels' summary-row reads for short sequences
    (no complete chunk, or no candidate anywhere): a workgroup whose queries have
    no candidate reads no k' row, and every row read lies in [0, T/S).  Before
    the guard that skips the prefetch when a block has no candidate, the clamp
    min(c0 + row, nc_block - 1) reached row -1, i.e. just before k_sum, or any
    row of an empty k_sum when T < S.  Also: the workspace sizes of every
    prefill call are defined for these shapes."""
    S, W = 64, 128
    NCs = T // S
    for rows_per_block in (256, 64):            # score_lse, rank_keys query blocks
        for qb in range(0, T, rows_per_block):
            nc_block = _nc(min(qb + rows_per_block - 1, T - 1), S, W)
            assert nc_block <= NCs
            if nc_block == 0:
                continue                         # no fetch at all
            cl_last = nc_block - 1
            for c0 in range(0, nc_block, 16):
                for row in range(16):
                    cl = min(c0 + row, cl_last)
                    assert 0 <= cl < NCs, (T, qb, c0, row)
    for i in range(T):                           # per-query reads c < nc(i)
        assert _nc(i, S, W) <= NCs
    s = _shape(B=1, Hq=4, Hkv=2, d=64, T=T, k=2, W=W)
    for op in (hils.OP_SELECT, hils.OP_ATTEND_FUSE, hils.OP_ATTEND_BACKWARD):
        assert hils.hils_workspace_bytes(s, op) > 0
