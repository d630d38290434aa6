"""Pins of the oracle's low-rank query calibration, q_hat = q + W_up W_down h
(paper-body page, implementation: Q-Cal; summary page, practical enhancements),
and of the shared-query summaries (paper-body page, implementation: one shared
learnable query per layer in place of the landmark tokens).

  * a zero up-projection, or a zero hidden state, leaves q_hat = q exactly;
  * a rank-1 calibration that reads one hidden component m (one-hot row of
    W_down) adds u_{h,e} h_m: a closed form, element by element, with shapes
    chosen so that a transposed or mis-indexed weight reads other values;
  * without rounding the correction is linear in h;
  * the stored q_hat is the exact value rounded to nearest-even by torch's own
    fp64 -> bf16 / fp32 conversion;
  * shared-query summaries are Eq. 8 with q'_c = q' for every chunk: a zero
    shared query gives the mean key and b' = log S.
"""
import numpy as np
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_zero_up_projection_or_hidden_state_is_identity():
    rng = np.random.Generator(np.random.PCG64(90))
    B, Hq, T, d, dm, r = 2, 3, 5, 4, 7, 2
    q = _rand(rng, B, Hq, T, d)
    h = _rand(rng, B, T, dm)
    wd = _rand(rng, r, dm)
    wu = np.zeros((Hq, d, r))
    np.testing.assert_array_equal(oracle.qcal(q, h, wd, wu), q)
    wu = _rand(rng, Hq, d, r)
    np.testing.assert_array_equal(oracle.qcal(q, np.zeros_like(h), wd, wu), q)


def test_rank_one_one_hot_closed_form():
    rng = np.random.Generator(np.random.PCG64(91))
    B, Hq, T, d, dm, r = 1, 3, 4, 5, 9, 2
    q = _rand(rng, B, Hq, T, d)
    h = _rand(rng, B, T, dm)
    m = 6
    wd = np.zeros((r, dm))
    wd[1, m] = 1.0                      # z_1 = h_m, z_0 = 0
    wu = _rand(rng, Hq, d, r)
    got = oracle.qcal(q, h, wd, wu)
    for b in range(B):
        for hd in range(Hq):
            for t in range(T):
                for e in range(d):
                    want = q[b, hd, t, e] + wu[hd, e, 1] * h[b, t, m]
                    assert abs(got[b, hd, t, e] - want) < 1e-15


def test_correction_is_linear_in_h():
    rng = np.random.Generator(np.random.PCG64(92))
    B, Hq, T, d, dm, r = 1, 2, 6, 8, 16, 4
    q = _rand(rng, B, Hq, T, d)
    h1, h2 = _rand(rng, B, T, dm), _rand(rng, B, T, dm)
    wd, wu = _rand(rng, r, dm), _rand(rng, Hq, d, r)
    f = lambda h: oracle.qcal(q, h, wd, wu) - q
    np.testing.assert_allclose(f(h1 + h2), f(h1) + f(h2), atol=1e-12)
    np.testing.assert_allclose(f(2.5 * h1), 2.5 * f(h1), atol=1e-12)


def test_stored_query_rounds_to_nearest_even():
    rng = np.random.Generator(np.random.PCG64(93))
    B, Hq, T, d, dm, r = 1, 2, 16, 8, 32, 4
    mk = lambda *s: torch.tensor(_rand(rng, *s) * 0.5, dtype=torch.float32)
    for dt, mode in ((torch.bfloat16, oracle.ORND_BF16), (torch.float32, oracle.ORND_F32)):
        q, h, wd, wu = mk(B, Hq, T, d).to(dt), mk(B, T, dm).to(dt), mk(r, dm).to(dt), mk(Hq, d, r).to(dt)
        exact = oracle.qcal(q, h, wd, wu, oracle.ORND_NONE)
        got = oracle.qcal(q, h, wd, wu, mode)
        want = torch.tensor(exact, dtype=torch.float64).to(dt).to(torch.float64).numpy()
        np.testing.assert_array_equal(got, want)


def test_shared_zero_query_summaries_are_mean_keys():
    rng = np.random.Generator(np.random.PCG64(94))
    B, Hq, Hkv, T, d, S = 1, 4, 2, 32, 6, 8
    k = _rand(rng, B, Hkv, T, d)
    ql = np.zeros((B, Hq, T // S, d))       # one shared query (zero), every chunk
    ks, bs = oracle.summarize(k, ql, S, Hq)
    for hd in range(Hq):
        g = hd // (Hq // Hkv)
        np.testing.assert_allclose(ks[0, hd], k[0, g].reshape(T // S, S, d).mean(axis=1), atol=1e-14)
        np.testing.assert_allclose(bs[0, hd], np.log(S), atol=1e-14)
