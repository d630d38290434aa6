"""Pins of the oracle's naive Block Sparse Attention selection (exact chunk mass).

The paper-body page's Block Sparse Attention preliminaries define the chunk
mass of a candidate chunk as the sum of the query's exponentiated token logits
over the chunk, and naive BSA keeps the k candidates of largest mass; with GQA
the group rule of the retrieval scores applies to the log-masses.  Pinned by:
  * an independent NumPy route (dense logits, per-chunk log-sum-exp, lexsort);
  * chunk size 1: the chunk mass is one token's logit, so the selection is the
    k largest logits left of the window;
  * identical keys inside each chunk: log Z_c = scale q . kappa_c + log S;
  * the Taylor identity of the summaries (summary page, Eq. 7 and Eq. 8): with
    every landmark query and the retrieval query equal to the query itself, the
    surrogate equals the exact log-mass, so HiLS's selection and rank keys equal
    naive BSA's at that position.
"""
import numpy as np
import pytest

import oracle


def _rows_all(B, Hkv, T):
    rb, rg, ri = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(T), indexing="ij")
    return rb.ravel(), rg.ravel(), ri.ravel()


def _numpy_bsa(q, k, S, W, topk, scale):
    """Dense NumPy route: logits, chunk log-masses, group rule, lexsort."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = []
    for b in range(B):
        for g in range(Hkv):
            kk = k[b, g]
            for i in range(T):
                a = i - W + 1
                lw = 0 if a <= 0 else (a // S) * S
                nc = lw // S
                lz = np.zeros((G, nc))
                for hh in range(G):
                    s = scale * kk[:nc * S] @ q[b, g * G + hh, i]
                    s = s.reshape(nc, S)
                    m = s.max(axis=1, keepdims=True) if nc else s
                    lz[hh] = (m[:, 0] + np.log(np.exp(s - m).sum(axis=1))) if nc else lz[hh]
                if G == 1:
                    r = lz[0]
                else:
                    L = np.array([np.logaddexp.reduce(lz[hh]) for hh in range(G)]) if nc else np.zeros(G)
                    r = (lz - L[:, None]).max(axis=0) if nc else np.zeros(0)
                order = np.lexsort((np.arange(nc), -r))
                sel = np.sort(order[:min(nc, topk)])
                idx = np.full(topk, -1)
                idx[:len(sel)] = sel
                gap = r[order[topk - 1]] - r[order[topk]] if nc > topk else np.inf
                out.append((idx, gap, r, lz))
    return out


@pytest.mark.parametrize("G", [1, 2])
def test_bsa_matches_numpy_route(G):
    rng = np.random.Generator(np.random.PCG64(70 + G))
    B, Hkv, T, d, S, W, topk = 2, 2, 52, 5, 4, 6, 3
    Hq = G * Hkv
    sc = 0.8
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    rb, rg, ri = _rows_all(B, Hkv, T)
    got = oracle.bsa_rows(rb, rg, ri, ri, q, k, S=S, W=W, topk=topk, scale=sc, want_r=True, want_lz=True)
    want = _numpy_bsa(q, k, S, W, topk, sc)
    assert int(np.sum(got["ncand"] > topk)) > 20        # real choices were made
    for t, (idx, gap, r, lz) in enumerate(want):
        nc = len(r)
        np.testing.assert_array_equal(got["idx"][t], idx)
        np.testing.assert_allclose(got["r"][t, :nc], r, atol=1e-12)
        np.testing.assert_allclose(got["lz"][t, :, :nc], lz, atol=1e-12)
        if np.isfinite(gap):
            assert abs(got["gap"][t] - gap) < 1e-12
        else:
            assert np.isinf(got["gap"][t])


def test_bsa_chunk_size_one_is_top_logits():
    rng = np.random.Generator(np.random.PCG64(81))
    B, Hq, Hkv, T, d, W, topk = 1, 1, 1, 40, 6, 5, 4
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    rb, rg, ri = _rows_all(B, Hkv, T)
    got = oracle.bsa_rows(rb, rg, ri, ri, q, k, S=1, W=W, topk=topk, scale=0.5, want_lz=True)
    for i in range(T):
        nc = max(0, i - W + 1)
        logits = 0.5 * k[0, 0, :nc] @ q[0, 0, i]
        np.testing.assert_allclose(got["lz"][i, 0, :nc], logits, atol=1e-13)
        top = np.sort(np.argsort(-logits, kind="stable")[:min(nc, topk)])
        want = np.full(topk, -1)
        want[:len(top)] = top
        np.testing.assert_array_equal(got["idx"][i], want)


def test_bsa_identical_keys_per_chunk():
    rng = np.random.Generator(np.random.PCG64(82))
    B, Hq, Hkv, T, d, S, W, topk = 1, 2, 1, 64, 4, 8, 8, 2
    kappa = rng.standard_normal((T // S, d))
    k = np.repeat(kappa, S, axis=0)[None, None]
    q = rng.standard_normal((B, Hq, T, d))
    rb, rg, ri = _rows_all(B, Hkv, T)
    got = oracle.bsa_rows(rb, rg, ri, ri, q, k, S=S, W=W, topk=topk, scale=0.7, want_lz=True)
    for i in range(T):
        nc = int(got["ncand"][i])
        for hh in range(Hq):
            want = 0.7 * kappa[:nc] @ q[0, hh, i] + np.log(S)
            np.testing.assert_allclose(got["lz"][i, hh, :nc], want, atol=1e-12)


@pytest.mark.parametrize("G", [1, 4])
def test_hils_equals_bsa_at_the_landmark_query(G):
    """q'_c := q_i* for every chunk and q_hat_i* := q_i*: s_hat = log Z exactly."""
    rng = np.random.Generator(np.random.PCG64(83 + G))
    B, Hkv, T, d, S, W, topk = 1, 1, 96, 6, 8, 8, 3
    Hq = G * Hkv
    sc = 0.9
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    istar = T - 1
    NC = T // S
    ql = np.repeat(q[:, :, istar:istar + 1, :], NC, axis=2)
    qh = rng.standard_normal((B, Hq, T, d))
    qh[:, :, istar] = q[:, :, istar]
    ks, bs = oracle.summarize(k, ql, S, Hq, scale=sc)
    one = (np.zeros(1, np.int32), np.zeros(1, np.int32), np.array([istar]), np.array([istar]))
    h = oracle.rows(*one, q, qh, k, v, ks, bs, S=S, W=W, topk=topk, scale=sc, want_r=True)
    z = oracle.bsa_rows(*one, q, k, S=S, W=W, topk=topk, scale=sc, want_r=True)
    nc = int(z["ncand"][0])
    assert nc > topk
    np.testing.assert_allclose(h["r"][0, :nc], z["r"][0, :nc], atol=1e-12)
    np.testing.assert_array_equal(h["idx"], z["idx"])


def test_selection_recall_counts():
    a = np.array([[0, 2, 5], [1, 3, -1], [0, 1, 2]])
    b = np.array([[0, 2, 4], [1, 3, -1], [3, 4, 5]])
    nc = np.array([9, 2, 7])
    r = oracle.selection_recall(a, b, nc, 3)
    assert r["events"] == 2 and r["hits"] == 2 and abs(r["recall"] - 2 / 6) < 1e-15
    assert oracle.selection_recall(b, b, nc, 3)["recall"] == 1.0
