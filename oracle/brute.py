"""Independent NumPy routes used to pin the C oracle -- TEST INFRASTRUCTURE ONLY.

`hils_brute` evaluates the fused output through the explicit token-weight
matrix of the hierarchical softmax (summary page, Methodology 2, Eq. 10):

    w_ij = exp(s_ij) / Z_{i,c(j)} * Zhat_{i,c(j)} / Zhat_i,
    Zhat_{i,c} = exp(s_hat_{i,c}) for selected chunks, Zhat_{i,win} = Z_{i,win},
    Zhat_i = sum of Zhat over the selected chunks and the window,

and out_i = sum_j w_ij v_j.  It forms every weight of every row, checks that
each row of the weight matrix sums to one, and multiplies by V -- a different
code route from the oracle's per-group outputs and log-sum-exp fusion.  The
summaries are computed vectorised (softmax along the chunk axis), and the
selection by Python's sort on (-key, chunk) tuples.

`dense_causal` is plain softmax(Q K^T * scale + causal mask) V.
Only small inputs: everything is materialised.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, np.float64)


def _logsumexp(x: np.ndarray, axis=-1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def summaries(k, q_land, S: int, Hq: int, scale: float):
    """k' [B,Hq,NC,d], b' [B,Hq,NC] via a batched softmax over each chunk (Eq. 8)."""
    k = _f64(k)
    ql = _f64(q_land)
    B, Hkv, T, d = k.shape
    G = Hq // Hkv
    NC = T // S
    kc = k[:, :, : NC * S].reshape(B, Hkv, NC, S, d)
    kc = np.repeat(kc, G, axis=1)                                  # [B,Hq,NC,S,d]
    logits = scale * np.einsum("bhcd,bhcsd->bhcs", ql[:, :, :NC], kc)
    p = np.exp(logits - _logsumexp(logits)[..., None])
    ksum = np.einsum("bhcs,bhcsd->bhcd", p, kc)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    bsum = -plogp.sum(-1)
    return ksum, bsum


def hils_brute(q, k, v, q_hat, ksum, bsum, *, S: int, W: int, topk: int, scale: float):
    """Full prefill by the explicit weight matrix.  Returns (out [B,Hq,T,d], sel list)."""
    q, k, v, qh = _f64(q), _f64(k), _f64(v), _f64(q_hat)
    ksum, bsum = _f64(ksum), _f64(bsum)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, T, d))
    sels = {}
    for b in range(B):
        for g in range(Hkv):
            heads = list(range(g * G, (g + 1) * G))
            for i in range(T):
                lw = max(0, S * math.floor((i - W + 1) / S))
                cand = list(range(lw // S))
                shat = {h: [scale * float(qh[b, h, i] @ ksum[b, h, c]) + float(bsum[b, h, c])
                            for c in cand] for h in heads}
                if len(cand) <= topk:
                    sel = cand
                else:
                    if G == 1:
                        key = shat[heads[0]]
                    else:
                        L = {h: float(_logsumexp(np.array(shat[h]))) for h in heads}
                        key = [max(shat[h][c] - L[h] for h in heads) for c in cand]
                    order = sorted(cand, key=lambda c: (-key[c], c))
                    sel = sorted(order[:topk])
                sels[(b, g, i)] = sel
                for h in heads:
                    wrow = np.zeros(T)
                    logits = scale * (k[b, g, : i + 1] @ q[b, h, i])
                    # masses: true window mass, surrogate mass for selected chunks
                    Zw = np.exp(logits[lw: i + 1]).sum()
                    Zhat_i = Zw + sum(math.exp(shat[h][c]) for c in sel)
                    for j in range(lw, i + 1):
                        wrow[j] = math.exp(logits[j]) / Zw * Zw / Zhat_i
                    for c in sel:
                        Zc = np.exp(logits[c * S:(c + 1) * S]).sum()
                        for j in range(c * S, (c + 1) * S):
                            wrow[j] = math.exp(logits[j]) / Zc * math.exp(shat[h][c]) / Zhat_i
                    assert abs(wrow.sum() - 1.0) < 1e-12, wrow.sum()
                    out[b, h, i] = wrow @ v[b, g]
    return out, sels


def dense_causal(q, k, v, scale: float):
    """Plain causal softmax attention in fp64: out [B,Hq,T,d], lse [B,Hq,T]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=1)
    vv = np.repeat(v, G, axis=1)
    s = scale * np.einsum("bhid,bhjd->bhij", q, kk)
    mask = np.tril(np.ones((T, T), bool))
    s = np.where(mask, s, -np.inf)
    lse = _logsumexp(s)
    p = np.exp(s - lse[..., None])
    return np.einsum("bhij,bhjd->bhid", p, vv), lse


def sliding_window(q, k, v, *, S: int, W: int, scale: float):
    """Softmax attention over the aligned window [l_i, i] only (the k = 0 case)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                lw = max(0, S * math.floor((i - W + 1) / S))
                s = scale * (k[b, g, lw: i + 1] @ q[b, h, i])
                p = np.exp(s - s.max())
                out[b, h, i] = (p / p.sum()) @ v[b, g, lw: i + 1]
    return out
