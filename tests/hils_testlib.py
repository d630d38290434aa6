"""Shared helpers of the parity tests: GPU runs through the C ABI, the oracle on
the same bytes, and the comparison rules.

Comparison rules
  * Selected chunk ids are integers decided by floating point.  An event (one
    (b, g, i) with |C_i| > k) is "decided" when the oracle's gap between the k-th
    and (k+1)-th rank key is at least TAU; there the GPU ids must equal the
    oracle's bit for bit.  Below TAU several selections are correct: the GPU's
    set must hold every candidate whose key exceeds r_(k) + TAU and only
    candidates whose key reaches r_(k) - TAU, and its outputs are checked
    against the oracle evaluated on that (validated) set.
  * TAU = 1e-5 when both sides score identical stored summaries; 3e-5 end to
    end in bf16, where the GPU's own k' may differ from the oracle's by one bf16
    rounding (|q_hat| |dk'| / sqrt(d) below about 7e-6).
  * Floating-point outputs: bf16 max-abs 2e-2 and rel-L2 5e-3; fp32 max-abs 1e-5.
  * The band itself is checked: the GPU's rank keys on its chosen chunks, rebuilt
    from its own outputs (each head's s_hat on the choice and each head's L_h),
    must agree with the oracle's keys on the same stored summaries within TAU/4
    (check_rank_keys).  End to end in bf16 the two sides' k' may also differ by
    one bf16 rounding; that part is bounded separately (kprime_rank_bound).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TAU_STAGE = 1e-5
TAU_E2E_BF16 = 3e-5
TAU_E2E_F32 = 1e-5


def tol_out(dtype) -> dict:
    if dtype == torch.bfloat16:
        return {"max_abs": 2e-2, "rel_l2": 5e-3}
    return {"max_abs": 1e-5, "rel_l2": 1e-5}


def tol_lse(dtype) -> float:
    return 2e-3 if dtype == torch.bfloat16 else 1e-5


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, np.float64)


def assert_close(got, want, max_abs, rel_l2=None, what=""):
    got, want = f64(got), f64(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    err = np.abs(got - want)
    ma = float(err.max()) if err.size else 0.0
    assert ma <= max_abs, "%s: max-abs %.3g > %.3g (at %s)" % (what, ma, max_abs,
                                                               np.unravel_index(err.argmax(), err.shape))
    if rel_l2 is not None and want.size:
        rl = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
        assert rl <= rel_l2, "%s: rel-L2 %.3g > %.3g" % (what, rl, rel_l2)


def check_selection(gpu_idx: np.ndarray, orc: dict, topk: int, tau: float) -> dict:
    """Compare GPU ids [n, k] with oracle rows (oracle.rows(..., want_r=True)).

    Returns counts and the boolean mask of rows whose GPU selection differs from
    the oracle's (all of them undecided and validated)."""
    n = gpu_idx.shape[0]
    oidx = orc["idx"]
    gap, ncand = orc["gap"], orc["ncand"]
    differ = np.zeros(n, bool)
    n_dec = n_und = 0
    for t in range(n):
        g = gpu_idx[t].tolist()
        o = oidx[t].tolist()
        nc = int(ncand[t])
        nsel = min(nc, topk)
        valid = [c for c in g if c >= 0]
        assert g[nsel:] == [-1] * (topk - nsel), ("pads", t, g)
        assert len(valid) == nsel and valid == sorted(set(valid)), ("ids", t, g)
        assert all(0 <= c < nc for c in valid), ("range", t, g, nc)
        if nc <= topk or gap[t] >= tau:
            n_dec += nc > topk
            assert g == o, ("decided selection differs", t, g, o, gap[t])
            continue
        n_und += 1
        if g == o:
            continue
        r = orc["r"][t, :nc]
        rk = np.sort(r)[::-1][topk - 1]
        assert r[valid].min() >= rk - tau, ("undecided set below band", t)
        must = set(np.nonzero(r > rk + tau)[0].tolist())
        assert must <= set(valid), ("undecided set misses a sure chunk", t)
        differ[t] = True
    return {"decided": n_dec, "undecided": n_und, "differ": differ}


def gpu_rank_keys(ssel_rows: np.ndarray, L_rows, G: int) -> np.ndarray:
    """The GPU's rank key of each chosen slot, from its own outputs: s_hat for a
    group of one head, else max over heads of (s_hat_h - L_h).  ssel_rows [n, G, k],
    L_rows [n, G] (ignored for G == 1).  Pads come out -inf."""
    if G == 1:
        return ssel_rows[:, 0, :].copy()
    with np.errstate(invalid="ignore"):      # rows without candidates: -inf - -inf
        return np.max(ssel_rows - np.asarray(L_rows)[:, :, None], axis=1)


def check_rank_keys(gpu_idx: np.ndarray, r_gpu: np.ndarray, orc: dict, topk: int,
                    limit: float, what: str = "") -> dict:
    """max |r_gpu - r_oracle| over every chosen slot of every row with candidates.

    orc must come from oracle.rows(..., want_r=True) on the same stored summaries.
    Asserts the maximum is at most `limit`; returns it with the number of keys."""
    err = 0.0
    n = 0
    for t in range(gpu_idx.shape[0]):
        nc = int(orc["ncand"][t])
        if nc == 0 or topk == 0:
            continue
        c = gpu_idx[t][gpu_idx[t] >= 0]
        ro = orc["r"][t, c]
        rg_ = r_gpu[t, :len(c)]
        assert np.all(np.isfinite(rg_)), ("non-finite GPU rank key", t)
        e = np.abs(rg_ - ro)
        err = max(err, float(e.max()))
        n += len(c)
    assert err <= limit, "%s: max |r_gpu - r_oracle| = %.3g > %.3g" % (what, err, limit)
    return {"max_err": err, "keys": n}


def kprime_rank_bound(ks_gpu: np.ndarray, ks_orc: np.ndarray, qh_rows: np.ndarray, rb, rg, G: int,
                      scale: float) -> float:
    """Largest change of any rank key that the difference between two stores of k'
    can cause on the given rows: scale * sum_e |q_hat_e| |dk'_e| per (row, head,
    chunk), doubled for the shift of L_h.  qh_rows [n, G, d] (the rows' q_hat)."""
    dk = np.abs(f64(ks_gpu) - f64(ks_orc))                 # [B, Hq, NC, d]
    bound = 0.0
    for t in range(len(rb)):
        heads = slice(rg[t] * G, (rg[t] + 1) * G)
        m = scale * np.einsum("hd,hcd->hc", np.abs(qh_rows[t]), dk[rb[t], heads])
        bound = max(bound, 2.0 * float(m.max()) if m.size else 0.0)
    return bound


def rows_layout(B: int, Hkv: int, positions) -> tuple:
    pos = np.asarray(positions, np.int64)
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), pos, indexing="ij")
    return rb.ravel(), rg.ravel(), ri.ravel()


def gather_rows(t: torch.Tensor, rb, rg, ri, G: int) -> np.ndarray:
    """Per-row view of a [B, H, T, ...] GPU output: rows (b, g, i) -> [n, G, ...]."""
    x = t.detach().cpu()
    out = []
    for b, g, i in zip(rb, rg, ri):
        out.append(x[b, g * G:(g + 1) * G, i])
    return torch.stack(out).to(torch.float64).numpy() if x.dtype != torch.int32 else torch.stack(out).numpy()
