"""HiLS-Attention forward path on MI355X: Python binding of libhils.so.

The calls keep the names of the C ABI (include/hils.h) and only marshal
arguments: torch tensors supply device memory and the current HIP stream, every
step of the computation runs in the library's kernels.  There is no fallback:
if the library is missing, loading raises.

    hils_summarize(k, q_land, k_sum, b_sum, shape, chunk_begin=0, n_chunks=None)
    hils_select(q_hat, k_sum, b_sum, sel_idx, sel_score, shape, workspace=None)
    hils_attend_fuse(q, k, v, sel_idx, sel_score, out, lse, shape, workspace=None)
    hils_decode_step(pos, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache,
                     k_sum, b_sum, out, lse, sel_idx, shape, workspace=None)
    hils_attend_fuse_backward(q, k, v, q_hat, k_sum, sel_idx, sel_score, out, lse, dout,
                              dlse, dq, dk, dv, dq_hat, dk_sum, db_sum, shape, workspace=None)
    hils_summarize_backward(k, q_land, dk_sum, db_sum, dk, dq_land, shape, chunk_begin=0,
                            n_chunks=None)
    hils_decode_multi(pos, n_queries, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache,
                      k_sum, b_sum, out, lse, sel_idx, shape, workspace=None)
    hils_decode_multi_workspace_bytes(shape, n_queries)
    hils_qcal(q, hs, w_down, w_up, q_hat, shape)
    hils_select_qcal(q, hs, w_down, w_up, k_sum, b_sum, q_hat, sel_idx, sel_score, shape,
                     workspace=None)
    hils_select_qcal_workspace_bytes(shape, rank)
    hils_summarize_shared(k, q_shared, k_sum, b_sum, shape, chunk_begin=0, n_chunks=None)
    hils_bsa_select(q, k, sel_idx, shape, workspace=None)
    hils_selection_overlap(idx_a, idx_b, count, shape)
    hils_workspace_bytes(shape, op)
    hils_timing_enable(kernels), hils_timing_get(kernel)   (diagnostics)

`Shape` mirrors `hils_shape`.  `prefill()` chains the three prefill calls.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhils.so")

HILS_F32, HILS_BF16 = 0, 1
OP_SUMMARIZE, OP_SELECT, OP_ATTEND_FUSE, OP_DECODE, OP_ATTEND_BACKWARD = 0, 1, 2, 3, 4

STATUS = {
    0: "HILS_OK", -1: "HILS_E_NULL", -2: "HILS_E_SHAPE", -3: "HILS_E_DTYPE", -4: "HILS_E_ALIGN",
    -5: "HILS_E_WORKSPACE", -6: "HILS_E_POS", -7: "HILS_E_NEED_QLAND", -8: "HILS_E_UNSUPPORTED",
    -9: "HILS_E_LAUNCH", -10: "HILS_E_SCRATCH",
}

EXPORTS = ("hils_summarize", "hils_select", "hils_attend_fuse", "hils_decode_step",
           "hils_decode_step_noalloc", "hils_attend_fuse_backward", "hils_summarize_backward",
           "hils_bsa_select", "hils_selection_overlap", "hils_qcal", "hils_select_qcal",
           "hils_select_qcal_workspace_bytes", "hils_summarize_shared",
           "hils_decode_multi", "hils_decode_multi_workspace_bytes",
           "hils_workspace_bytes", "hils_status_string", "hils_abi_version",
           "hils_timing_enable", "hils_timing_get")


class HilsError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s returned %s (%d): %s" % (fn, STATUS.get(status, "?"), status, msg))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("window", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("scale", ctypes.c_float),
                ("io_dtype", ctypes.c_int), ("summary_dtype", ctypes.c_int)]

    @classmethod
    def make(cls, B, Hq, Hkv, d, S, W, k, T, dtype, scale=0.0):
        dt = HILS_BF16 if dtype in (torch.bfloat16, "bf16") else HILS_F32
        return cls(B, Hq, Hkv, d, S, W, k, T, float(scale), dt, dt)


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libhils.so is not built (run chunk_wise_sparse_summary_amd/build.py "
                              "or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        SP = ctypes.POINTER(Shape)
        L.hils_summarize.argtypes = [SP, P, P, I64, I64, P, P, P]
        L.hils_select.argtypes = [SP, P, P, P, P, P, P, SZ, P]
        L.hils_attend_fuse.argtypes = [SP, P, P, P, P, P, P, P, P, SZ, P]
        L.hils_decode_step.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.hils_decode_step_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.hils_attend_fuse_backward.argtypes = [SP] + [P] * 18 + [SZ, P]
        L.hils_summarize_backward.argtypes = [SP, P, P, P, P, I64, I64, P, P, P]
        L.hils_bsa_select.argtypes = [SP, P, P, P, P, SZ, P]
        L.hils_selection_overlap.argtypes = [SP, P, P, P, P]
        L.hils_qcal.argtypes = [SP, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P]
        L.hils_select_qcal.argtypes = [SP, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P,
                                       P, SZ, P]
        L.hils_select_qcal_workspace_bytes.argtypes = [SP, ctypes.c_int32]
        L.hils_select_qcal_workspace_bytes.restype = SZ
        L.hils_summarize_shared.argtypes = [SP, P, P, I64, I64, P, P, P]
        L.hils_decode_multi.argtypes = [SP, ctypes.c_int32, P] + [P] * 12 + [P, SZ, P]
        L.hils_decode_multi_workspace_bytes.argtypes = [SP, ctypes.c_int32]
        L.hils_decode_multi_workspace_bytes.restype = SZ
        L.hils_workspace_bytes.argtypes = [SP, ctypes.c_int]
        L.hils_workspace_bytes.restype = SZ
        L.hils_status_string.argtypes = [ctypes.c_int]
        L.hils_status_string.restype = ctypes.c_char_p
        L.hils_abi_version.restype = ctypes.c_int
        L.hils_timing_enable.argtypes = [ctypes.c_char_p]
        L.hils_timing_enable.restype = ctypes.c_int
        L.hils_timing_get.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
        L.hils_timing_get.restype = ctypes.c_int
        for f in ("hils_summarize", "hils_select", "hils_attend_fuse", "hils_decode_step",
                  "hils_decode_step_noalloc", "hils_attend_fuse_backward", "hils_summarize_backward",
                  "hils_bsa_select", "hils_selection_overlap", "hils_qcal", "hils_select_qcal",
                  "hils_summarize_shared", "hils_decode_multi"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise HilsError(fn, st, lib().hils_status_string(st).decode())


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def hils_workspace_bytes(shape: Shape, op: int) -> int:
    return int(lib().hils_workspace_bytes(ctypes.byref(shape), op))


def workspace(shape: Shape, op: int, device="cuda") -> torch.Tensor:
    n = hils_workspace_bytes(shape, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def hils_summarize(k, q_land, k_sum, b_sum, shape: Shape, chunk_begin: int = 0,
                   n_chunks: int | None = None):
    _dev(k, q_land, k_sum, b_sum)
    if n_chunks is None:
        n_chunks = shape.seq_len // shape.chunk - chunk_begin
    _check("hils_summarize", lib().hils_summarize(ctypes.byref(shape), _p(k), _p(q_land),
                                                  chunk_begin, n_chunks, _p(k_sum), _p(b_sum),
                                                  _stream()))


def hils_select(q_hat, k_sum, b_sum, sel_idx, sel_score, shape: Shape, workspace_t=None):
    _dev(q_hat, k_sum, b_sum, sel_idx, sel_score)
    if workspace_t is None:
        workspace_t = workspace(shape, OP_SELECT, q_hat.device)
    _check("hils_select", lib().hils_select(ctypes.byref(shape), _p(q_hat), _p(k_sum), _p(b_sum),
                                            _p(sel_idx), _p(sel_score), _p(workspace_t),
                                            workspace_t.numel(), _stream()))


def hils_attend_fuse(q, k, v, sel_idx, sel_score, out, lse, shape: Shape, workspace_t=None):
    _dev(q, k, v, sel_idx, sel_score, out, lse)
    if workspace_t is None:
        workspace_t = workspace(shape, OP_ATTEND_FUSE, q.device)
    _check("hils_attend_fuse", lib().hils_attend_fuse(ctypes.byref(shape), _p(q), _p(k), _p(v),
                                                      _p(sel_idx), _p(sel_score), _p(out), _p(lse),
                                                      _p(workspace_t), workspace_t.numel(),
                                                      _stream()))


def hils_decode_step(pos, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum, b_sum,
                     out, lse, sel_idx, shape: Shape, workspace_t=None):
    _dev(q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum, b_sum, out, lse, sel_idx)
    pos_arr = (ctypes.c_int64 * shape.batch)(*[int(p) for p in pos])
    if workspace_t is None:
        workspace_t = workspace(shape, OP_DECODE, q.device)
    _check("hils_decode_step", lib().hils_decode_step(
        ctypes.byref(shape), pos_arr, _p(q), _p(q_hat), _p(k_new), _p(v_new), _p(q_land_new),
        _p(k_cache), _p(v_cache), _p(k_sum), _p(b_sum), _p(out), _p(lse), _p(sel_idx),
        _p(workspace_t), workspace_t.numel(), _stream()))


def hils_attend_fuse_backward(q, k, v, q_hat, k_sum, sel_idx, sel_score, out, lse, dout, dlse,
                              dq, dk, dv, dq_hat, dk_sum, db_sum, shape: Shape, workspace_t=None):
    """Gradients of hils_attend_fuse (and of the selection scores), selection held fixed."""
    _dev(q, k, v, q_hat, k_sum, sel_idx, sel_score, out, lse, dout, dlse, dq, dk, dv, dq_hat,
         dk_sum, db_sum)
    if workspace_t is None:
        workspace_t = workspace(shape, OP_ATTEND_BACKWARD, q.device)
    _check("hils_attend_fuse_backward", lib().hils_attend_fuse_backward(
        ctypes.byref(shape), _p(q), _p(k), _p(v), _p(q_hat), _p(k_sum), _p(sel_idx), _p(sel_score),
        _p(out), _p(lse), _p(dout), _p(dlse), _p(dq), _p(dk), _p(dv), _p(dq_hat), _p(dk_sum),
        _p(db_sum), _p(workspace_t), workspace_t.numel(), _stream()))


def hils_summarize_backward(k, q_land, dk_sum, db_sum, dk, dq_land, shape: Shape,
                            chunk_begin: int = 0, n_chunks: int | None = None):
    """Gradients of hils_summarize: adds into dk, writes dq_land."""
    _dev(k, q_land, dk_sum, db_sum, dk, dq_land)
    if n_chunks is None:
        n_chunks = shape.seq_len // shape.chunk - chunk_begin
    _check("hils_summarize_backward", lib().hils_summarize_backward(
        ctypes.byref(shape), _p(k), _p(q_land), _p(dk_sum), _p(db_sum), chunk_begin, n_chunks,
        _p(dk), _p(dq_land), _stream()))


def hils_qcal(q, hs, w_down, w_up, q_hat, shape: Shape):
    """q_hat = q + W_up (W_down hs), rounded once to the io dtype."""
    _dev(q, hs, w_down, w_up, q_hat)
    _check("hils_qcal", lib().hils_qcal(ctypes.byref(shape), _p(q), _p(hs), _p(w_down), _p(w_up),
                                        int(hs.shape[-1]), int(w_down.shape[0]), _p(q_hat), _stream()))


def hils_select_qcal_workspace_bytes(shape: Shape, rank: int) -> int:
    return int(lib().hils_select_qcal_workspace_bytes(ctypes.byref(shape), int(rank)))


def hils_select_qcal(q, hs, w_down, w_up, k_sum, b_sum, q_hat, sel_idx, sel_score, shape: Shape,
                     workspace_t=None):
    """hils_select with q_hat = q + W_up (W_down hs) formed inside its first scoring pass
    (q_hat is written too)."""
    _dev(q, hs, w_down, w_up, k_sum, b_sum, q_hat, sel_idx, sel_score)
    rank = int(w_down.shape[0])
    if workspace_t is None:
        n = hils_select_qcal_workspace_bytes(shape, rank)
        workspace_t = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("hils_select_qcal", lib().hils_select_qcal(
        ctypes.byref(shape), _p(q), _p(hs), _p(w_down), _p(w_up), int(hs.shape[-1]), rank, _p(k_sum),
        _p(b_sum), _p(q_hat), _p(sel_idx), _p(sel_score), _p(workspace_t), workspace_t.numel(), _stream()))


def hils_summarize_shared(k, q_shared, k_sum, b_sum, shape: Shape, chunk_begin: int = 0,
                          n_chunks: int | None = None):
    """Summaries with one shared landmark query per head (q_shared [Hq, d])."""
    _dev(k, q_shared, k_sum, b_sum)
    if n_chunks is None:
        n_chunks = shape.seq_len // shape.chunk - chunk_begin
    _check("hils_summarize_shared", lib().hils_summarize_shared(
        ctypes.byref(shape), _p(k), _p(q_shared), chunk_begin, n_chunks, _p(k_sum), _p(b_sum), _stream()))


def hils_bsa_select(q, k, sel_idx, shape: Shape, workspace_t=None):
    """Naive Block Sparse Attention selection (exact chunk masses), a diagnostic."""
    _dev(q, k, sel_idx)
    if workspace_t is None:
        workspace_t = workspace(shape, OP_SELECT, q.device)
    _check("hils_bsa_select", lib().hils_bsa_select(ctypes.byref(shape), _p(q), _p(k), _p(sel_idx),
                                                    _p(workspace_t), workspace_t.numel(), _stream()))


def hils_selection_overlap(idx_a, idx_b, count, shape: Shape):
    """count[b,g,i] = number of chunk ids rows (b,g,i) of two selections share."""
    _dev(idx_a, idx_b, count)
    _check("hils_selection_overlap", lib().hils_selection_overlap(ctypes.byref(shape), _p(idx_a),
                                                                  _p(idx_b), _p(count), _stream()))


def hils_decode_multi_workspace_bytes(shape: Shape, n_queries: int) -> int:
    return int(lib().hils_decode_multi_workspace_bytes(ctypes.byref(shape), int(n_queries)))


def hils_decode_multi(pos, n_queries, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum,
                      b_sum, out, lse, sel_idx, shape: Shape, workspace_t=None):
    """n_queries adjacent new tokens per sequence at positions pos[b] .. pos[b] + n_queries - 1."""
    _dev(q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum, b_sum, out, lse, sel_idx)
    pos_arr = (ctypes.c_int64 * shape.batch)(*[int(p) for p in pos])
    if workspace_t is None:
        n = hils_decode_multi_workspace_bytes(shape, n_queries)
        workspace_t = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("hils_decode_multi", lib().hils_decode_multi(
        ctypes.byref(shape), int(n_queries), pos_arr, _p(q), _p(q_hat), _p(k_new), _p(v_new),
        _p(q_land_new), _p(k_cache), _p(v_cache), _p(k_sum), _p(b_sum), _p(out), _p(lse), _p(sel_idx),
        _p(workspace_t), workspace_t.numel(), _stream()))


def hils_decode_step_noalloc(pos, q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum,
                             b_sum, out, lse, sel_idx, shape: Shape):
    """hils_decode_step on the library's built-in scratch (no workspace, no allocation)."""
    _dev(q, q_hat, k_new, v_new, q_land_new, k_cache, v_cache, k_sum, b_sum, out, lse, sel_idx)
    pos_arr = (ctypes.c_int64 * shape.batch)(*[int(p) for p in pos])
    _check("hils_decode_step_noalloc", lib().hils_decode_step_noalloc(
        ctypes.byref(shape), pos_arr, _p(q), _p(q_hat), _p(k_new), _p(v_new), _p(q_land_new),
        _p(k_cache), _p(v_cache), _p(k_sum), _p(b_sum), _p(out), _p(lse), _p(sel_idx), _stream()))


KERNELS = ("summarize", "score_lse", "idx_count", "idx_scan_tiles",
           "idx_scan_buckets", "idx_fill", "lsel", "window", "chunk_attend",
           "dec_score", "dec_select", "dec_attend", "dec_fuse", "dec_summarize",
           "v_transpose", "rank_keys", "topk_scores",
           "bwd_rowstat", "bwd_kv", "bwd_dq", "bwd_qhat", "summarize_bwd",
           "bsa_keys", "bsa_topk", "qcal", "dec_append", "dec_gsel", "qcal_zdown")


def hils_timing_enable(kernels):
    """Time launches of the named kernels (iterable of names, "*" for all, None for off)."""
    if kernels is None:
        arg = None
    elif isinstance(kernels, str):
        arg = kernels.encode()
    else:
        arg = ",".join(kernels).encode()
    _check("hils_timing_enable", lib().hils_timing_enable(arg))


def hils_timing_get(kernel: str):
    """(total milliseconds, launches) of a kernel's timed launches since enabling."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check("hils_timing_get", lib().hils_timing_get(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def select_lse(workspace_t: torch.Tensor, shape: Shape) -> torch.Tensor:
    """Each head's L_{h,i} = LSE over the candidates of s_hat, as hils_select leaves
    it at the start of its workspace for groups of more than one head ([B, Hq, T]
    fp32 view of the workspace; hils.h states the layout)."""
    n = shape.batch * shape.heads_q * shape.seq_len
    off = (-workspace_t.data_ptr()) % 256
    return workspace_t[off:off + 4 * n].view(torch.float32).view(shape.batch, shape.heads_q,
                                                                   shape.seq_len)


def prefill(q, k, v, q_land, q_hat, *, S: int, W: int, topk: int, scale: float = 0.0,
            ws_select=None, ws_attend=None):
    """summarize -> select -> attend_fuse for [B,H,T,d] inputs; returns a dict of outputs
    (and the select workspace, whose start holds each head's L_h)."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    shape = Shape.make(B, Hq, Hkv, d, S, W, topk, T, q.dtype, scale)
    NC = T // S
    k_sum = torch.empty((B, Hq, NC, d), dtype=q.dtype, device=q.device)
    b_sum = torch.empty((B, Hq, NC), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hkv, T, topk), dtype=torch.int32, device=q.device)
    ssel = torch.empty((B, Hq, T, topk), dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if ws_select is None:
        ws_select = workspace(shape, OP_SELECT, q.device)
    if NC > 0:
        hils_summarize(k, q_land, k_sum, b_sum, shape)
    hils_select(q_hat, k_sum, b_sum, idx, ssel, shape, ws_select)
    hils_attend_fuse(q, k, v, idx, ssel, out, lse, shape, ws_attend)
    return {"k_sum": k_sum, "b_sum": b_sum, "idx": idx, "ssel": ssel, "out": out, "lse": lse,
            "shape": shape, "ws_select": ws_select}
