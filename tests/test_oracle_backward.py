"""Pins of the oracle's backward (gradients of the prefill forward).

The forward is differentiable once the selection is held fixed (top-k is
piecewise constant), so the gradient of sum(dout * out) + sum(dlse * lse) is
pinned three independent ways:
  * central finite differences of that loss, evaluated with the oracle's forward
    (selection forced) on summaries from the independent NumPy route
    (oracle/brute.py), for every element of q, q_hat, K, V and the landmark
    queries of a tiny problem;
  * chunk size 1 with every candidate selected and q_hat = q: the path is dense
    causal softmax attention (summary page, Eq. 8 with S = 1), whose gradients
    torch's autograd gives in float64;
  * V = 1: the output is 1 whatever the queries and keys (the fused weights sum
    to one), so every gradient but dV vanishes and dV sums to sum(dout).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def _gen(B, Hq, Hkv, T, d, NC, seed, scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    f = lambda *s: rng.standard_normal(s) * scale
    return {"q": f(B, Hq, T, d), "k": f(B, Hkv, T, d), "v": f(B, Hkv, T, d),
            "q_land": f(B, Hq, NC, d), "q_hat": f(B, Hq, T, d)}


def _loss(x, sel, dout, dlse, S, W, topk, sc):
    """sum(dout * out) + sum(dlse * lse) with the selection forced to `sel`."""
    B, Hq, T, d = x["q"].shape
    Hkv = x["k"].shape[1]
    ks, bs = brute.summaries(x["k"], x["q_land"], S, Hq, sc)
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(T), indexing="ij")
    rb, rg, ri = rb.ravel(), rg.ravel(), ri.ravel()
    r = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], ks, bs, S=S, W=W, topk=topk,
                    scale=sc, forced_idx=sel.reshape(-1, topk))
    dn = oracle.to_dense(r, B, Hq, Hkv, T, topk)
    return float(np.sum(dout * dn["out"]) + np.sum(dlse * dn["lse"]))


@pytest.mark.parametrize("G", [1, 2])
def test_backward_matches_finite_differences(G):
    B, Hkv, d, S, W, topk, T = 1, 1, 3, 4, 4, 2, 28
    Hq = G * Hkv
    sc = 0.7
    x = _gen(B, Hq, Hkv, T, d, T // S, seed=40 + G, scale=0.9)
    ks, bs = brute.summaries(x["k"], x["q_land"], S, Hq, sc)
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(T), indexing="ij")
    r = oracle.rows(rb.ravel(), rg.ravel(), ri.ravel(), ri.ravel(), x["q"], x["q_hat"], x["k"], x["v"],
                    ks, bs, S=S, W=W, topk=topk, scale=sc)
    sel = r["idx"].reshape(B, Hkv, T, topk)
    assert np.sum(r["ncand"] > topk) > 5               # real choices were made
    rng = np.random.Generator(np.random.PCG64(7))
    dout = rng.standard_normal((B, Hq, T, d))
    dlse = rng.standard_normal((B, Hq, T))
    gr = oracle.prefill_backward(x, sel, dout, dlse, S=S, W=W, topk=topk, scale=sc, ksum=ks, bsum=bs)
    h = 1e-6
    for name, gname in (("q", "dq"), ("q_hat", "dq_hat"), ("k", "dk"), ("v", "dv"),
                        ("q_land", "dq_land")):
        a = x[name]
        num = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + h
            lp = _loss(x, sel, dout, dlse, S, W, topk, sc)
            a[idx] = old - h
            lm = _loss(x, sel, dout, dlse, S, W, topk, sc)
            a[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - gr[gname]).max()
        assert err < 2e-6 * max(1.0, np.abs(num).max()), (name, err)


def test_backward_chunk_size_one_is_dense_attention_backward():
    B, Hq, Hkv, T, d = 1, 2, 1, 20, 4
    sc = 0.5
    x = _gen(B, Hq, Hkv, T, d, T, seed=51)
    x["q_hat"] = x["q"].copy()
    W, topk = 3, T                       # every candidate chosen
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=1, Hq=Hq, scale=sc, nc=T)
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(T), indexing="ij")
    r = oracle.rows(rb.ravel(), rg.ravel(), ri.ravel(), ri.ravel(), x["q"], x["q_hat"], x["k"],
                    x["v"], ks, bs, S=1, W=W, topk=topk, scale=sc)
    sel = r["idx"].reshape(B, Hkv, T, topk)
    rng = np.random.Generator(np.random.PCG64(9))
    dout = rng.standard_normal((B, Hq, T, d))
    dlse = rng.standard_normal((B, Hq, T))
    gr = oracle.prefill_backward(x, sel, dout, dlse, S=1, W=W, topk=topk, scale=sc)
    # dense causal attention by torch autograd (float64)
    q = torch.tensor(x["q"], requires_grad=True)
    k = torch.tensor(x["k"], requires_grad=True)
    v = torch.tensor(x["v"], requires_grad=True)
    kk = k.repeat_interleave(Hq // Hkv, dim=1)
    vv = v.repeat_interleave(Hq // Hkv, dim=1)
    s = sc * q @ kk.transpose(-1, -2)
    mask = torch.tril(torch.ones(T, T, dtype=torch.bool))
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, -1)
    out = torch.softmax(s, -1) @ vv
    (torch.sum(torch.tensor(dout) * out) + torch.sum(torch.tensor(dlse) * lse)).backward()
    # q reaches the loss through the token logits (dq) and, as q_hat, through s_hat
    np.testing.assert_allclose(gr["dq"] + gr["dq_hat"], q.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(gr["dk"], k.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(gr["dv"], v.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(gr["dq_land"], 0.0, atol=1e-12)   # a one-token softmax is constant


def test_backward_values_of_ones():
    B, Hq, Hkv, T, d, S, W, topk = 2, 4, 2, 40, 5, 4, 6, 3
    x = _gen(B, Hq, Hkv, T, d, T // S, seed=61)
    x["v"] = np.ones_like(x["v"])
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=S, Hq=Hq, scale=0.6, nc=T // S)
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(T), indexing="ij")
    r = oracle.rows(rb.ravel(), rg.ravel(), ri.ravel(), ri.ravel(), x["q"], x["q_hat"], x["k"],
                    x["v"], ks, bs, S=S, W=W, topk=topk, scale=0.6)
    sel = r["idx"].reshape(B, Hkv, T, topk)
    dout = np.random.Generator(np.random.PCG64(3)).standard_normal((B, Hq, T, d))
    gr = oracle.prefill_backward(x, sel, dout, None, S=S, W=W, topk=topk, scale=0.6, ksum=ks, bsum=bs)
    for n in ("dq", "dq_hat", "dk", "dk_sum", "db_sum", "dq_land"):
        np.testing.assert_allclose(gr[n], 0.0, atol=1e-12, err_msg=n)
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            np.testing.assert_allclose(gr["dv"][b, g].sum(0), dout[b, g * G:(g + 1) * G].sum((0, 1)),
                                       atol=1e-10)
