"""fp64 CPU oracle of the HiLS-Attention forward path -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  It shares no code with the GPU library
(`chunk_wise_sparse_summary_amd`) and never imports it.

`hils_oracle.c` holds the arithmetic (plain loops in double precision, with
OpenMP across rows); this module builds it with gcc, loads it with ctypes and
marshals arrays.  `brute.py` holds an independent NumPy route (explicit token
weight matrix, dense attention) used to pin this one.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hils_oracle.c")
_LIB = os.path.join(_HERE, "libhils_oracle.so")

ODT_F32, ODT_BF16, ODT_F64 = 0, 1, 2
ORND_NONE, ORND_F32, ORND_BF16 = 0, 1, 2

_lib = None
_lib_path = _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp); returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def use_library(path: str | None) -> None:
    """Load the oracle from another build of the same source (None: the default).

    Only the mutation tests use this, to check that planted mistakes in a copy
    of the oracle are caught by its pins."""
    global _lib, _lib_path
    _lib = None
    _lib_path = _LIB if path is None else path


def lib():
    global _lib
    if _lib is None:
        if _lib_path == _LIB and (not os.path.exists(_LIB)
                                  or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        L = ctypes.CDLL(_lib_path)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_summarize.argtypes = [I, I, I, I, I, D, P, I, I64, P, I, I64, I64, I64, I, P, P, I64]
        L.orc_summarize.restype = I
        L.orc_rows.argtypes = [I, I, I, I, I, I, I, D, I64, P, P, P, P, P, P, I, I64, P, P, I, I64,
                               P, P, I64, P, P, P, P, P, P, P, P, I64]
        L.orc_rows.restype = I
        L.orc_prefill_backward.argtypes = [I, I, I, I, I, I, I, D, I64, P, P, P, I, P, P, I, P, P, I64,
                                           P, P, P, P, P, P, P, P, P, P]
        L.orc_prefill_backward.restype = I
        L.orc_bsa_rows.argtypes = [I, I, I, I, I, I, I, D, I64, P, P, P, P, P, I, I64, P, I, I64,
                                   P, P, P, P, I64, P, I64]
        L.orc_bsa_rows.restype = I
        L.orc_qcal.argtypes = [I, I, I, I64, I, I, P, P, P, P, I, I, P]
        L.orc_qcal.restype = I
        L.orc_window_left.argtypes = [I64, I, I]
        L.orc_window_left.restype = I64
        L.orc_num_candidates.argtypes = [I64, I, I]
        L.orc_num_candidates.restype = I64
        L.orc_max_threads.restype = I
        L.orc_set_threads.argtypes = [I]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def _as_np(x):
    """(contiguous numpy array, oracle dtype code) for a torch tensor or numpy array."""
    if isinstance(x, torch.Tensor):
        x = x.detach()
        if x.device.type != "cpu":
            x = x.cpu()
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy(), ODT_BF16
        if x.dtype == torch.float32:
            return x.numpy(), ODT_F32
        if x.dtype == torch.float64:
            return x.numpy(), ODT_F64
        raise TypeError(x.dtype)
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, ODT_F32
    if x.dtype == np.float64:
        return x, ODT_F64
    if x.dtype in (np.uint16, np.int16):
        return x, ODT_BF16
    raise TypeError(x.dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> int:
    """Use n OpenMP threads from now on; returns the previous count."""
    prev = int(lib().orc_max_threads())
    lib().orc_set_threads(int(n))
    return prev


def window_left(i: int, S: int, W: int) -> int:
    return int(lib().orc_window_left(i, S, W))


def num_candidates(i: int, S: int, W: int) -> int:
    return int(lib().orc_num_candidates(i, S, W))


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def summarize(k, q_land, S: int, Hq: int, scale: float | None = None, ks_round: int = ORND_NONE,
              c0: int = 0, nc: int | None = None, ks_NC: int | None = None,
              ksum: np.ndarray | None = None, bsum: np.ndarray | None = None):
    """Chunk summaries k' [B,Hq,NC,d] and b' [B,Hq,NC] (float64) for chunks [c0, c0+nc)."""
    ka, kdt = _as_np(k)
    qa, qdt = _as_np(q_land)
    B, Hkv, kT, d = ka.shape
    ql_NC = qa.shape[2]
    if nc is None:
        nc = min(kT // S, ql_NC) - c0
    if ks_NC is None:
        ks_NC = c0 + nc
    if scale is None:
        scale = default_scale(d)
    if ksum is None:
        ksum = np.zeros((B, Hq, ks_NC, d), np.float64)
        bsum = np.zeros((B, Hq, ks_NC), np.float64)
    rc = lib().orc_summarize(B, Hq, Hkv, d, S, float(scale), _ptr(ka), kdt, kT, _ptr(qa), qdt,
                             ql_NC, c0, nc, ks_round, _ptr(ksum), _ptr(bsum), ks_NC)
    if rc != 0:
        raise RuntimeError("orc_summarize failed: %d" % rc)
    return ksum, bsum


def rows(rb, rg, ri, rq, q, q_hat, k, v, ksum, bsum, *, S: int, W: int, topk: int,
         scale: float | None = None, forced_idx=None, want_r: bool = False):
    """Evaluate the path on a list of query rows (b, g, position i, query row iq).

    Returns a dict of numpy arrays: idx [n,k], ssel [n,G,k], gap [n], ncand [n],
    out [n,G,d], lse [n,G] and (if want_r) r [n, NC] (rank key per candidate).
    """
    qa, qdt = _as_np(q)
    qha, qhdt = _as_np(q_hat)
    assert qdt == qhdt
    ka, kdt = _as_np(k)
    va, vdt = _as_np(v)
    assert kdt == vdt
    B, Hq, qT, d = qa.shape
    Hkv, kvT = ka.shape[1], ka.shape[2]
    G = Hq // Hkv
    ksum = np.ascontiguousarray(ksum, np.float64)
    bsum = np.ascontiguousarray(bsum, np.float64)
    ksNC = ksum.shape[2]
    if scale is None:
        scale = default_scale(d)
    rb = np.ascontiguousarray(rb, np.int32)
    rg = np.ascontiguousarray(rg, np.int32)
    ri = np.ascontiguousarray(ri, np.int64)
    rq = np.ascontiguousarray(rq, np.int64)
    n = rb.shape[0]
    kk = max(topk, 1)
    idx = np.zeros((n, kk), np.int32)
    ssel = np.zeros((n, G, kk), np.float64)
    gap = np.zeros(n, np.float64)
    ncand = np.zeros(n, np.int64)
    out = np.zeros((n, G, d), np.float64)
    lse = np.zeros((n, G), np.float64)
    r = np.full((n, max(ksNC, 1)), np.nan, np.float64) if want_r else None
    fi = None
    if forced_idx is not None:
        fi = np.ascontiguousarray(forced_idx, np.int32)
        assert fi.shape == (n, topk)
    rc = lib().orc_rows(B, Hq, Hkv, d, S, W, topk, float(scale), n, _ptr(rb), _ptr(rg), _ptr(ri),
                        _ptr(rq), _ptr(qa), _ptr(qha), qdt, qT, _ptr(ka), _ptr(va), kdt, kvT,
                        _ptr(ksum), _ptr(bsum), ksNC, _ptr(fi) if fi is not None else None,
                        _ptr(idx), _ptr(ssel), _ptr(gap), _ptr(ncand), _ptr(out), _ptr(lse),
                        _ptr(r) if r is not None else None, r.shape[1] if r is not None else 0)
    if rc != 0:
        raise RuntimeError("orc_rows failed: %d" % rc)
    res = {"idx": idx[:, :topk], "ssel": ssel[:, :, :topk], "gap": gap, "ncand": ncand,
           "out": out, "lse": lse}
    if want_r:
        res["r"] = r
    return res


def bsa_rows(rb, rg, ri, rq, q, k, *, S: int, W: int, topk: int, scale: float | None = None,
             want_r: bool = False, want_lz: bool = False):
    """Naive BSA selection (exact chunk mass) on a list of query rows (b, g, i, iq).

    Returns idx [n,k], gap [n], ncand [n], and if asked r [n, NC] (rank key per
    candidate) and lz [n, G, NC] (log chunk mass per head and candidate)."""
    qa, qdt = _as_np(q)
    ka, kdt = _as_np(k)
    B, Hq, qT, d = qa.shape
    Hkv, kvT = ka.shape[1], ka.shape[2]
    G = Hq // Hkv
    NC = max(kvT // S, 1)
    if scale is None:
        scale = default_scale(d)
    rb = np.ascontiguousarray(rb, np.int32)
    rg = np.ascontiguousarray(rg, np.int32)
    ri = np.ascontiguousarray(ri, np.int64)
    rq = np.ascontiguousarray(rq, np.int64)
    n = rb.shape[0]
    kk = max(topk, 1)
    idx = np.zeros((n, kk), np.int32)
    gap = np.zeros(n, np.float64)
    ncand = np.zeros(n, np.int64)
    r = np.full((n, NC), np.nan, np.float64) if want_r else None
    lz = np.full((n, G, NC), np.nan, np.float64) if want_lz else None
    rc = lib().orc_bsa_rows(B, Hq, Hkv, d, S, W, topk, float(scale), n, _ptr(rb), _ptr(rg), _ptr(ri),
                            _ptr(rq), _ptr(qa), qdt, qT, _ptr(ka), kdt, kvT, _ptr(idx), _ptr(gap),
                            _ptr(ncand), _ptr(r) if r is not None else None, NC if r is not None else 0,
                            _ptr(lz) if lz is not None else None, NC if lz is not None else 0)
    if rc != 0:
        raise RuntimeError("orc_bsa_rows failed: %d" % rc)
    res = {"idx": idx[:, :topk], "gap": gap, "ncand": ncand}
    if want_r:
        res["r"] = r
    if want_lz:
        res["lz"] = lz
    return res


def selection_recall(idx_a, idx_b, ncand, topk: int) -> dict:
    """Recall of selection A against selection B over the rows where a choice is
    made (|C_i| > k): the fraction of B's chunks that A also holds."""
    a = np.asarray(idx_a).reshape(-1, topk)
    b = np.asarray(idx_b).reshape(-1, topk)
    nc = np.asarray(ncand).reshape(-1)
    ev = nc > topk
    hits = 0
    for x, y in zip(a[ev], b[ev]):
        hits += len(set(x[x >= 0].tolist()) & set(y[y >= 0].tolist()))
    n = int(ev.sum())
    return {"events": n, "hits": hits, "recall": hits / (n * topk) if n else float("nan")}


def qcal(q, h, w_down, w_up, round_mode: int = ORND_NONE) -> np.ndarray:
    """Calibrated retrieval query q_hat = q + W_up W_down h [B,Hq,T,d] (float64,
    rounded once to round_mode).  h [B,T,dm], w_down [r,dm], w_up [Hq,d,r]."""
    qa, dt = _as_np(q)
    ha, hdt = _as_np(h)
    wd, wddt = _as_np(w_down)
    wu, wudt = _as_np(w_up)
    assert dt == hdt == wddt == wudt
    B, Hq, T, d = qa.shape
    dm = ha.shape[2]
    r = wd.shape[0]
    assert ha.shape == (B, T, dm) and wd.shape == (r, dm) and wu.shape == (Hq, d, r)
    out = np.zeros((B, Hq, T, d), np.float64)
    rc = lib().orc_qcal(B, Hq, d, T, dm, r, _ptr(ha), _ptr(wd), _ptr(wu), _ptr(qa), dt, round_mode,
                        _ptr(out))
    if rc != 0:
        raise RuntimeError("orc_qcal failed: %d" % rc)
    return out


def ks_round_for(summary_dtype) -> int:
    if summary_dtype in (torch.bfloat16, "bf16"):
        return ORND_BF16
    if summary_dtype in (torch.float32, "f32"):
        return ORND_F32
    return ORND_NONE


def prefill(inp: dict, *, S: int, W: int, topk: int, scale: float | None = None,
            ks_round: int | None = None, positions=None, want_r: bool = False) -> dict:
    """The whole prefill forward for inputs q, k, v, q_land, q_hat.

    `positions` restricts the evaluated query rows (default: every position).
    Returns k_sum, b_sum, and per-row results with rows ordered (b, g, i).
    """
    q, k, v, ql, qh = inp["q"], inp["k"], inp["v"], inp["q_land"], inp["q_hat"]
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if ks_round is None:
        ks_round = ks_round_for(q.dtype)
    ksum, bsum = summarize(k, ql, S, Hq, scale=scale, ks_round=ks_round, nc=T // S)
    pos = np.arange(T) if positions is None else np.asarray(positions, np.int64)
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), pos, indexing="ij")
    rb, rg, ri = rb.ravel(), rg.ravel(), ri.ravel()
    res = rows(rb, rg, ri, ri, q, qh, k, v, ksum, bsum, S=S, W=W, topk=topk, scale=scale,
               want_r=want_r)
    res.update(k_sum=ksum, b_sum=bsum, rb=rb, rg=rg, ri=ri)
    return res


def to_dense(res: dict, B: int, Hq: int, Hkv: int, T: int, topk: int):
    """Reshape full-prefill row results to the GPU output layouts."""
    G = Hq // Hkv
    d = res["out"].shape[-1]
    idx = res["idx"].reshape(B, Hkv, T, topk)
    gap = res["gap"].reshape(B, Hkv, T)
    ncand = res["ncand"].reshape(B, Hkv, T)
    ssel = res["ssel"].reshape(B, Hkv, T, G, topk).transpose(0, 1, 3, 2, 4).reshape(B, Hq, T, topk)
    out = res["out"].reshape(B, Hkv, T, G, d).transpose(0, 1, 3, 2, 4).reshape(B, Hq, T, d)
    lse = res["lse"].reshape(B, Hkv, T, G).transpose(0, 1, 3, 2).reshape(B, Hq, T)
    res = {"idx": idx, "gap": gap, "ncand": ncand, "ssel": ssel, "out": out, "lse": lse}
    return {k: np.ascontiguousarray(v) for k, v in res.items()}


def prefill_backward(inp: dict, sel_idx, dout, dlse=None, *, S: int, W: int, topk: int,
                     scale: float | None = None, ksum=None, bsum=None) -> dict:
    """Gradients of sum(dout * out) + sum(dlse * lse) of the prefill forward with the
    selection held at sel_idx [B,Hkv,T,k]: dq, dq_hat [B,Hq,T,d], dk, dv [B,Hkv,T,d]
    (dk includes the summaries' part), dk_sum [B,Hq,NC,d], db_sum [B,Hq,NC] and
    dq_land [B,Hq,NC,d], as float64.  ksum / bsum: the summaries the forward used
    (default: the oracle's own, unrounded k')."""
    q, k, v, ql, qh = inp["q"], inp["k"], inp["v"], inp["q_land"], inp["q_hat"]
    qa, qdt = _as_np(q)
    qha, _ = _as_np(qh)
    qla, qldt = _as_np(ql)
    assert qldt == qdt
    ka, kdt = _as_np(k)
    va, _ = _as_np(v)
    B, Hq, T, d = qa.shape
    Hkv = ka.shape[1]
    NC = T // S
    if scale is None:
        scale = default_scale(d)
    if ksum is None:
        ksum, bsum = summarize(k, ql, S, Hq, scale=scale, ks_round=ORND_NONE, nc=NC)
    ksum = np.ascontiguousarray(ksum, np.float64)
    bsum = np.ascontiguousarray(bsum, np.float64)
    si = np.ascontiguousarray(sel_idx, np.int32)
    assert si.shape == (B, Hkv, T, topk)
    g = np.ascontiguousarray(dout, np.float64)
    gl = None if dlse is None else np.ascontiguousarray(dlse, np.float64)
    out = {"dq": np.zeros((B, Hq, T, d)), "dq_hat": np.zeros((B, Hq, T, d)),
           "dk": np.zeros((B, Hkv, T, d)), "dv": np.zeros((B, Hkv, T, d)),
           "dk_sum": np.zeros((B, Hq, NC, d)), "db_sum": np.zeros((B, Hq, NC)),
           "dq_land": np.zeros((B, Hq, NC, d))}
    rc = lib().orc_prefill_backward(B, Hq, Hkv, d, S, W, topk, float(scale), T, _ptr(qa), _ptr(qha),
                                    _ptr(qla), qdt, _ptr(ka), _ptr(va), kdt, _ptr(ksum), _ptr(bsum), NC,
                                    _ptr(si), _ptr(g), _ptr(gl) if gl is not None else None,
                                    *[_ptr(out[n]) for n in ("dq", "dq_hat", "dk", "dv", "dk_sum",
                                                             "db_sum", "dq_land")])
    if rc != 0:
        raise RuntimeError("orc_prefill_backward failed: %d" % rc)
    return out
