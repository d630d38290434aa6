"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test states the property and the passage it comes from.  None of these
re-types the oracle's formulas: they compare against closed forms, a
hand-derived example, dense attention, an exact-rational selection, or the
independent NumPy route of `oracle/brute.py` (explicit Eq. 10 weight matrix).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import brute
import workloads as wk


def _gen(B=1, Hq=1, Hkv=1, T=64, d=8, NC=None, seed=0, scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    NC = NC if NC is not None else T
    f = lambda *s: (rng.standard_normal(s) * scale)
    return {"q": f(B, Hq, T, d), "k": f(B, Hkv, T, d), "v": f(B, Hkv, T, d),
            "q_land": f(B, Hq, NC, d), "q_hat": f(B, Hq, T, d)}


def _all_rows(inp, S, W, topk, scale, ks_round=oracle.ORND_NONE):
    return oracle.prefill(inp, S=S, W=W, topk=topk, scale=scale, ks_round=ks_round)


# ---------------------------------------------------------------- golden, by hand
def test_golden_hand_example(golden):
    """Worked example derived by hand from Eq. 8 and Eq. 10 (tests/golden/hand_example.txt)."""
    g = golden("hand_example.txt")
    k = np.array([0, math.log(3), 0, 0, math.log(2), 0], np.float64).reshape(1, 1, 6, 1)
    v = np.arange(1, 7, dtype=np.float64).reshape(1, 1, 6, 1)
    q = np.ones((1, 1, 6, 1))
    ql = np.ones((1, 1, 3, 1))
    ks, bs = oracle.summarize(k, ql, S=2, Hq=1, scale=1.0)
    assert ks[0, 0, 0, 0] == pytest.approx(g["ksum0"], abs=1e-15)
    assert bs[0, 0, 0] == pytest.approx(g["bsum0"], abs=1e-7)   # b' is stored in fp32
    assert ks[0, 0, 1, 0] == pytest.approx(g["ksum1"], abs=1e-15)
    assert bs[0, 0, 1] == pytest.approx(g["bsum1"], abs=1e-7)
    # exact fp64 b' for the row evaluation (the fp32 storage point is pinned above)
    bs64 = np.array([[[g["bsum0"], g["bsum1"], math.log(2)]]])
    r = oracle.rows([0], [0], [5], [5], q, q, k, v, ks, bs64, S=2, W=2, topk=1, scale=1.0)
    assert r["idx"][0].tolist() == [int(g["idx"])]
    assert r["ssel"][0, 0, 0] == pytest.approx(g["shat0"], abs=1e-14)
    assert r["gap"][0] == pytest.approx(g["gap"], abs=1e-14)
    assert r["out"][0, 0, 0] == pytest.approx(g["out"], abs=1e-14)
    assert r["lse"][0, 0] == pytest.approx(g["lse"], abs=1e-14)


def test_golden_forced_selection(golden):
    """The forced-selection branch (used when a GPU's near-tie selection differs):
    forcing chunk 1 in the hand example gives its hand-derived out = 23/5, lse = ln 5."""
    g = golden("hand_example.txt")
    k = np.array([0, math.log(3), 0, 0, math.log(2), 0], np.float64).reshape(1, 1, 6, 1)
    v = np.arange(1, 7, dtype=np.float64).reshape(1, 1, 6, 1)
    q = np.ones((1, 1, 6, 1))
    ks = np.array([[[[g["ksum0"]], [g["ksum1"]], [0.0]]]])
    bs = np.array([[[g["bsum0"], g["bsum1"], math.log(2)]]])
    r = oracle.rows([0], [0], [5], [5], q, q, k, v, ks, bs, S=2, W=2, topk=1, scale=1.0,
                    forced_idx=np.array([[1]]))
    assert r["idx"][0].tolist() == [1]
    assert r["ssel"][0, 0, 0] == pytest.approx(g["forced1_shat"], abs=1e-14)
    assert r["out"][0, 0, 0] == pytest.approx(g["forced1_out"], abs=1e-14)
    assert r["lse"][0, 0] == pytest.approx(g["forced1_lse"], abs=1e-14)


@pytest.mark.parametrize("G,topk", [(1, 3), (4, 2)])
def test_forced_own_selection_is_identical(G, topk):
    """Forcing the oracle's own selection reproduces its out, lse and scores bit for bit,
    on every row (rows with fewer candidates than k included)."""
    x = _gen(B=2, Hq=2 * G, Hkv=2, T=160, d=8, NC=20, seed=31, scale=0.8)
    S, W = 8, 16
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=S, Hq=2 * G, scale=0.4)
    rb, rg, ri = np.meshgrid(np.arange(2), np.arange(2), np.arange(160), indexing="ij")
    rb, rg, ri = rb.ravel(), rg.ravel(), ri.ravel()
    a = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], ks, bs, S=S, W=W,
                    topk=topk, scale=0.4)
    assert np.sum(a["ncand"] > topk) > 100
    b = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], ks, bs, S=S, W=W,
                    topk=topk, scale=0.4, forced_idx=a["idx"])
    for key in ("idx", "ssel", "out", "lse", "ncand"):
        assert np.array_equal(a[key], b[key]), key


def test_golden_gqa_rule(golden):
    """GQA rule: max over heads of per-head normalised weights (tests/golden/gqa_rule.txt)."""
    g = golden("gqa_rule.txt")
    T = 8
    k = np.zeros((1, 1, T, 1))
    v = np.zeros((1, 1, T, 1))
    q = np.zeros((1, 2, T, 1))
    ks = np.zeros((1, 2, 4, 1))
    bs = np.zeros((1, 2, 4))
    bs[0, 0, :3] = g["bsumA"]
    bs[0, 1, :3] = g["bsumB"]
    r = oracle.rows([0], [0], [7], [7], q, q, k, v, ks, bs, S=2, W=2, topk=1, scale=1.0)
    assert r["ncand"][0] == 3
    assert r["idx"][0].tolist() == [int(g["idx_group"])]
    assert r["gap"][0] == pytest.approx(g["gap_group"], abs=1e-12)
    r1 = oracle.rows([0], [0], [7], [7], q[:, :1], q[:, :1], k, v, ks[:, :1], bs[:, :1],
                     S=2, W=2, topk=1, scale=1.0)
    assert r1["idx"][0].tolist() == [int(g["idx_headA"])]


# ---------------------------------------------------------------- window / candidates
def test_window_and_candidates():
    """Aligned window and candidate set (paper-body page, BSA preliminaries)."""
    S, W = 64, 1024
    for i in range(0, 4000, 7):
        lw = oracle.window_left(i, S, W)
        assert lw % S == 0 and 0 <= lw <= i
        # left edge rounded down from i-W+1, so the window holds >= W tokens once i >= W-1
        if i >= W - 1:
            assert i - lw + 1 == W + ((i - W + 1) % S)
        else:
            assert lw == 0
        assert oracle.num_candidates(i, S, W) == lw // S
    # first position with a candidate: W + S - 1
    assert oracle.num_candidates(W + S - 2, S, W) == 0
    assert oracle.num_candidates(W + S - 1, S, W) == 1
    # floor toward -inf with a negative operand, and a window shorter than a chunk
    assert oracle.window_left(0, 64, 64) == 0
    assert oracle.window_left(130, 64, 1) == 128


# ---------------------------------------------------------------- P1, P7, P8: summaries
def test_p1_taylor_exact_at_landmark():
    """Eq. 7 is exact at q = q'_c: scale*q'.k' + b' = LSE_j(scale*q'.k_j) (summary page Eq. 7/8)."""
    x = _gen(B=2, Hq=4, Hkv=2, T=96, d=16, NC=6, seed=1)
    S, sc = 16, 0.37
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=S, Hq=4, scale=sc)
    # exact fp64 b' for the identity (b' is stored in fp32)
    _, bs64 = brute.summaries(x["k"], x["q_land"], S, 4, sc)
    for b in range(2):
        for h in range(4):
            for c in range(6):
                kc = x["k"][b, h // 2, c * S:(c + 1) * S]
                ql = x["q_land"][b, h, c]
                true = logsumexp(sc * kc @ ql)
                assert sc * ql @ ks[b, h, c] + bs64[b, h, c] == pytest.approx(true, abs=1e-12)
                assert bs[b, h, c] == pytest.approx(bs64[b, h, c], abs=1e-6)


def test_p1_through_rows():
    """Taylor exactness seen through the retrieval score of the row path."""
    T, S, W, d = 64, 8, 8, 8
    x = _gen(T=T, d=d, NC=T // S, seed=2)
    i = T - 1
    c_star = 2
    x["q_hat"][0, 0, i] = x["q_land"][0, 0, c_star]
    ks, bs = brute.summaries(x["k"], x["q_land"], S, 1, 0.5)
    r = oracle.rows([0], [0], [i], [i], x["q"], x["q_hat"], x["k"], x["v"], ks, bs,
                    S=S, W=W, topk=64, scale=0.5)
    sel = r["idx"][0].tolist()
    true = logsumexp(0.5 * x["k"][0, 0, c_star * S:(c_star + 1) * S] @ x["q_land"][0, 0, c_star])
    assert r["ssel"][0, 0, sel.index(c_star)] == pytest.approx(true, abs=1e-12)


def test_p7_mean_pool_special_case():
    """q'_c = 0 gives the mean-pooled key and b' = log S (paper-body page, BSA analysis)."""
    x = _gen(B=1, Hq=2, Hkv=1, T=64, d=8, NC=4, seed=3)
    ql = np.zeros_like(x["q_land"])
    ks, bs = oracle.summarize(x["k"], ql, S=16, Hq=2, scale=0.3)
    for c in range(4):
        mean = x["k"][0, 0, c * 16:(c + 1) * 16].mean(0)
        for h in range(2):
            np.testing.assert_allclose(ks[0, h, c], mean, rtol=0, atol=1e-14)
            assert bs[0, h, c] == pytest.approx(math.log(16), abs=1e-6)


def test_p8_entropy_regimes():
    """0 <= b' <= log S; identical keys -> (key, log S); one dominant key -> (that key, ~0)."""
    x = _gen(B=1, Hq=1, Hkv=1, T=256, d=8, NC=16, seed=4)
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=16, Hq=1, scale=1.0)
    assert np.all(bs >= 0) and np.all(bs <= math.log(16) + 1e-6)
    k = x["k"].copy()
    k[0, 0, 16:32] = k[0, 0, 16]            # chunk 1: identical keys
    u = np.zeros(8)
    u[0] = 1.0
    k[0, 0, 32:48] *= 0.01
    k[0, 0, 40] = 60.0 * u                  # chunk 2: one dominant key
    ql = x["q_land"].copy()
    ql[0, 0, 2] = u
    ks, bs = oracle.summarize(k, ql, S=16, Hq=1, scale=1.0)
    np.testing.assert_allclose(ks[0, 0, 1], k[0, 0, 16], atol=1e-14)
    assert bs[0, 0, 1] == pytest.approx(math.log(16), abs=1e-6)
    np.testing.assert_allclose(ks[0, 0, 2], k[0, 0, 40], atol=1e-20)
    assert abs(bs[0, 0, 2]) < 1e-20


def test_summary_rounding_points():
    """k' is rounded once (nearest-even) onto the bf16 grid; b' onto fp32."""
    x = _gen(B=1, Hq=2, Hkv=1, T=128, d=16, NC=8, seed=5)
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=16, Hq=2, scale=0.25)
    kr, br = oracle.summarize(x["k"], x["q_land"], S=16, Hq=2, scale=0.25,
                              ks_round=oracle.ORND_BF16)
    ref = torch.from_numpy(ks).to(torch.bfloat16).to(torch.float64).numpy()
    # double -> bf16 in one rounding equals torch's (double -> fp32 -> bf16) except
    # at double-rounding ties, which random data does not hit
    np.testing.assert_array_equal(kr, ref)
    np.testing.assert_array_equal(br, bs.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- P3: weights sum to 1
def test_p3_fused_weights_sum_to_one():
    """Zhat_i normalises over selected chunks and the window (summary page, Eq. 10)."""
    x = _gen(B=1, Hq=4, Hkv=2, T=160, d=8, NC=10, seed=6)
    x["v"] = np.ones_like(x["v"])
    res = _all_rows(x, S=16, W=32, topk=3, scale=0.4)
    np.testing.assert_allclose(res["out"], 1.0, atol=1e-13)
    u = np.arange(8) * 0.25 - 1.0
    x["v"] = x["v"] * 0.0 + np.random.default_rng(0).standard_normal(x["v"].shape)
    a = _all_rows(x, S=16, W=32, topk=3, scale=0.4)
    x2 = dict(x)
    x2["v"] = x["v"] + u
    b2 = _all_rows(x2, S=16, W=32, topk=3, scale=0.4)
    np.testing.assert_allclose(b2["out"], a["out"] + u, atol=1e-12)
    np.testing.assert_array_equal(a["idx"], b2["idx"])


# ---------------------------------------------------------------- P4, P5, P6: dense collapse
@pytest.mark.parametrize("W", [1, 3, 8])
def test_p4_chunk_size_one_is_dense(W):
    """S = 1: k' = k, b' = 0; with q_hat = q and top-k = all, out is dense causal attention."""
    T, d = 40, 8
    x = _gen(B=1, Hq=2, Hkv=1, T=T, d=d, NC=T, seed=7)
    x["q_hat"] = x["q"].copy()
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=1, Hq=2, scale=0.35)
    for h in range(2):
        np.testing.assert_array_equal(ks[0, h], x["k"][0, 0])
    np.testing.assert_array_equal(bs, 0.0)
    res = _all_rows(x, S=1, W=W, topk=T, scale=0.35)
    d_out, d_lse = brute.dense_causal(x["q"], x["k"], x["v"], 0.35)
    dense = oracle.to_dense(res, 1, 2, 1, T, T)
    np.testing.assert_allclose(dense["out"], d_out, atol=1e-12)
    np.testing.assert_allclose(dense["lse"], d_lse, atol=1e-12)


def test_p5_single_query_exact_any_chunk_size():
    """q'_c := q_hat_i* := q_i* for every chunk: row i* equals the dense causal row."""
    T, S, d = 96, 8, 8
    x = _gen(B=1, Hq=1, Hkv=1, T=T, d=d, NC=T // S, seed=8)
    i = T - 1
    x["q_land"][0, 0, :] = x["q"][0, 0, i]
    x["q_hat"][0, 0, i] = x["q"][0, 0, i]
    ks, bs = brute.summaries(x["k"], x["q_land"], S, 1, 0.6)
    r = oracle.rows([0], [0], [i], [i], x["q"], x["q_hat"], x["k"], x["v"], ks, bs,
                    S=S, W=S, topk=T, scale=0.6)
    d_out, d_lse = brute.dense_causal(x["q"], x["k"], x["v"], 0.6)
    np.testing.assert_allclose(r["out"][0, 0], d_out[0, 0, i], atol=1e-12)
    assert r["lse"][0, 0] == pytest.approx(d_lse[0, 0, i], abs=1e-12)


def test_p6_short_prefix_and_window_only():
    """No candidates before W+S-1 (dense rows); top-k = 0 is aligned sliding-window attention."""
    T, S, W, d = 128, 8, 16, 8
    x = _gen(B=1, Hq=2, Hkv=2, T=T, d=d, NC=T // S, seed=9)
    res = oracle.to_dense(_all_rows(x, S=S, W=W, topk=2, scale=0.5), 1, 2, 2, T, 2)
    d_out, _ = brute.dense_causal(x["q"], x["k"], x["v"], 0.5)
    n0 = W + S - 1
    np.testing.assert_allclose(res["out"][:, :, :n0], d_out[:, :, :n0], atol=1e-12)
    res0 = oracle.to_dense(_all_rows(x, S=S, W=W, topk=0, scale=0.5), 1, 2, 2, T, 0)
    sw = brute.sliding_window(x["q"], x["k"], x["v"], S=S, W=W, scale=0.5)
    np.testing.assert_allclose(res0["out"], sw, atol=1e-12)


# ---------------------------------------------------------------- P2: tangent bound
def test_p2_tangent_lower_bound():
    """With q_hat = q, s_hat_{i,c} <= log Z_{i,c} (LSE is convex; Eq. 7 is its tangent)."""
    T, S, W, d = 128, 8, 8, 8
    x = _gen(B=1, Hq=2, Hkv=1, T=T, d=d, NC=T // S, seed=10)
    x["q_hat"] = x["q"].copy()
    res = _all_rows(x, S=S, W=W, topk=T, scale=0.5)
    for t in range(len(res["ri"])):
        i = res["ri"][t]
        for hh in range(2):
            for s_, c in enumerate(res["idx"][t]):
                if c < 0:
                    continue
                logz = logsumexp(0.5 * x["k"][0, 0, c * S:(c + 1) * S] @ x["q"][0, hh, i])
                assert res["ssel"][t, hh, s_] <= logz + 1e-12


# ---------------------------------------------------------------- P9: brute force
@pytest.mark.parametrize("cfg", [
    dict(B=1, Hq=1, Hkv=1, T=32, d=4, S=2, W=4, k=3),
    dict(B=2, Hq=2, Hkv=1, T=32, d=8, S=4, W=4, k=2),
    dict(B=1, Hq=4, Hkv=2, T=28, d=6, S=4, W=6, k=1),
    dict(B=1, Hq=2, Hkv=2, T=30, d=5, S=2, W=3, k=4),
    dict(B=1, Hq=2, Hkv=1, T=24, d=8, S=4, W=1, k=0),
])
def test_p9_brute_force_matrix_form(cfg):
    """Oracle == explicit token-weight matrix of Eq. 10 with a sort-based selection."""
    T, S = cfg["T"], cfg["S"]
    x = _gen(B=cfg["B"], Hq=cfg["Hq"], Hkv=cfg["Hkv"], T=T, d=cfg["d"], NC=T // S, seed=11)
    sc = 0.45
    res = _all_rows(x, S=S, W=cfg["W"], topk=cfg["k"], scale=sc)
    ks_b, bs_b = brute.summaries(x["k"], x["q_land"], S, cfg["Hq"], sc)
    np.testing.assert_allclose(res["k_sum"], ks_b, atol=1e-13)
    np.testing.assert_allclose(res["b_sum"], bs_b, atol=1e-6)   # fp32 storage point
    out_b, sels = brute.hils_brute(x["q"], x["k"], x["v"], x["q_hat"], res["k_sum"], res["b_sum"],
                                   S=S, W=cfg["W"], topk=cfg["k"], scale=sc)
    dense = oracle.to_dense(res, cfg["B"], cfg["Hq"], cfg["Hkv"], T, cfg["k"])
    np.testing.assert_allclose(dense["out"], out_b, atol=1e-12)
    for t in range(len(res["ri"])):
        key = (res["rb"][t], res["rg"][t], res["ri"][t])
        got = [c for c in res["idx"][t].tolist() if c >= 0]
        assert got == sels[key]


# ---------------------------------------------------------------- P-sel: exact ties
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 1), (4, 2)])
def test_psel_exact_ties_lower_index_wins(Hq, Hkv):
    """Dyadic scores are exact: selection equals an exact-rational sort, ties -> lower index."""
    x = wk.make_dyadic_select(B=1, Hq=Hq, Hkv=Hkv, T=256, d=16, S=8, k=5, W=16, seed=12)
    wl = x["wl"]
    qh = x["q_hat"].numpy()
    ks = x["k_sum"].numpy().astype(np.float64)
    bs = x["b_sum"].numpy().astype(np.float64)
    T = 256
    dummy = np.zeros((1, Hkv, T, 16))
    rb = np.zeros(Hkv * T, np.int32)
    rg = np.repeat(np.arange(Hkv), T)
    ri = np.tile(np.arange(T), Hkv)
    res = oracle.rows(rb, rg, ri, ri, qh, qh, dummy, dummy, ks, bs, S=8, W=16, topk=5,
                      scale=x["scale"])
    G = Hq // Hkv
    n_ties = 0
    for t in range(len(ri)):
        i, g = int(ri[t]), int(rg[t])
        nc = oracle.num_candidates(i, 8, 16)
        h = g * G            # identical heads in a group: the GQA key orders like s_hat
        shat = [Fraction(float(x["scale"])) * sum(Fraction(float(a)) * Fraction(float(b_))
                                                  for a, b_ in zip(qh[0, h, i], ks[0, h, c]))
                + Fraction(float(bs[0, h, c])) for c in range(nc)]
        order = sorted(range(nc), key=lambda c: (-shat[c], c))
        want = sorted(order[:5]) if nc > 5 else list(range(nc))
        got = [c for c in res["idx"][t].tolist() if c >= 0]
        assert got == want
        if nc > 5 and shat[order[4]] == shat[order[5]]:
            n_ties += 1
    assert n_ties > 0          # the planted ties do reach the k / k+1 boundary


# ---------------------------------------------------------------- P10: needle
def test_p10_needle_selected():
    """The planted needle chunk wins by more than 1 in s_hat and in the GQA key (8K layout)."""
    wl = wk.custom(name="needle", dtype="bf16", B=1, Hq=8, Hkv=2, d=128, T=2048, S=64, k=8,
                   W=256, needles=1)
    x = wk.make_prefill(wl, seed=0)
    m = x["meta"]
    res = oracle.prefill(x, S=64, W=256, topk=8, positions=[m["needle_query"]], want_r=True)
    t = 0      # row (b=0, g=0, i*)
    assert m["needle_chunk"] in res["idx"][t].tolist()
    r = res["r"][t, : res["ncand"][t]]
    c = m["needle_chunk"]
    assert r[c] - np.max(np.delete(r, c)) > 1.0
    ks, bs = res["k_sum"], res["b_sum"]
    qh = x["q_hat"].to(torch.float64).numpy()
    for h in range(4):
        sh = qh[0, h, m["needle_query"]] @ ks[0, h, : res["ncand"][t]].T / math.sqrt(128) \
            + bs[0, h, : res["ncand"][t]]
        assert sh[c] - np.max(np.delete(sh, c)) > 1.0


# ---------------------------------------------------------------- P11, P12, P13
def test_p11_gqa_identical_heads_equals_mha():
    """Identical heads in a group: the GQA selection equals one head's own selection."""
    x = _gen(B=1, Hq=4, Hkv=1, T=256, d=8, NC=32, seed=13)
    for key in ("q", "q_hat", "q_land"):
        x[key][:, 1:] = x[key][:, :1]
    g = _all_rows(x, S=8, W=16, topk=4, scale=0.5)
    one = {k_: (v_[:, :1] if k_ in ("q", "q_hat", "q_land") else v_) for k_, v_ in x.items()}
    m = _all_rows(one, S=8, W=16, topk=4, scale=0.5)
    np.testing.assert_array_equal(g["idx"], m["idx"])


def test_p12_batch_independence():
    """Changing sequence 1 leaves sequence 0's outputs bitwise unchanged."""
    x = _gen(B=2, Hq=2, Hkv=1, T=128, d=8, NC=16, seed=14)
    a = oracle.to_dense(_all_rows(x, S=8, W=16, topk=3, scale=0.5), 2, 2, 1, 128, 3)
    y = {k_: v_.copy() for k_, v_ in x.items()}
    for key in y:
        y[key][1] = np.random.default_rng(1).standard_normal(y[key][1].shape)
    b = oracle.to_dense(_all_rows(y, S=8, W=16, topk=3, scale=0.5), 2, 2, 1, 128, 3)
    for key in ("out", "lse", "idx", "ssel"):
        np.testing.assert_array_equal(a[key][0], b[key][0])
    assert not np.array_equal(a["out"][1], b["out"][1])


def test_p13_decode_row_equals_prefill_row():
    """A decode step at position t (cache with unused rows beyond t) is prefill's row t."""
    T, S, W, d = 200, 8, 16, 8
    x = _gen(B=1, Hq=2, Hkv=1, T=T, d=d, NC=T // S, seed=15)
    ks, bs = oracle.summarize(x["k"], x["q_land"], S=S, Hq=2, scale=0.5)
    cap = 256
    kc = np.full((1, 1, cap, d), 1e30)
    vc = np.full((1, 1, cap, d), np.nan)
    kc[:, :, :T] = x["k"]
    vc[:, :, :T] = x["v"]
    for t in (31, 120, 199):
        p = oracle.rows([0], [0], [t], [t], x["q"], x["q_hat"], x["k"], x["v"], ks, bs,
                        S=S, W=W, topk=3, scale=0.5)
        dq = x["q"][:, :, t:t + 1].copy()
        dqh = x["q_hat"][:, :, t:t + 1].copy()
        dc = oracle.rows([0], [0], [t], [0], dq, dqh, kc, vc, ks, bs, S=S, W=W, topk=3, scale=0.5)
        for key in ("idx", "ssel", "out", "lse", "gap"):
            np.testing.assert_array_equal(p[key], dc[key])
