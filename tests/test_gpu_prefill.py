"""GPU parity of the prefill path through the C ABI against the fp64 oracle.

Each case draws seeded inputs on the host, copies the same bytes to the GPU and
evaluates both sides.  Stage tests feed both sides identical stored
intermediate values (summaries, selections) taken from the oracle, so each
kernel is checked alone; end-to-end tests run the whole GPU path.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from hils_testlib import (TAU_E2E_BF16, TAU_E2E_F32, TAU_STAGE, assert_close, check_rank_keys,
                          check_selection, f64, gather_rows, gpu_rank_keys, kprime_rank_bound,
                          rows_layout, tol_lse, tol_out)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def hils():
    import chunk_wise_sparse_summary_amd as h
    h.lib()
    return h


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # name: workload, positions evaluated by the oracle (None = all)
    "tiny": (wk.CONFIGS["tiny"], None),
    "bf16_g4_d128": (wk.custom(name="g4", dtype="bf16", B=1, Hq=8, Hkv=2, d=128, T=1600, S=64,
                               k=6, W=128), None),
    "bf16_g1_d64_ragged": (wk.custom(name="g1", dtype="bf16", B=2, Hq=2, Hkv=2, d=64, T=1317,
                                     S=64, k=5, W=100), None),
    "f32_g2_d128": (wk.custom(name="g2", dtype="f32", B=1, Hq=4, Hkv=2, d=128, T=900, S=64, k=3,
                              W=64), None),
    "bf16_g8_d64": (wk.custom(name="g8", dtype="bf16", B=1, Hq=8, Hkv=1, d=64, T=1100, S=64, k=4,
                              W=200), None),
}


def _inputs(wl, seed=0):
    x = wk.make_prefill(wl, seed=seed)                       # host bytes
    xd = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    return x, xd


def _shape(hils, wl, k=None):
    return hils.Shape.make(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k if k is None else k, wl.T,
                           wl.torch_dtype)


@pytest.mark.parametrize("name", list(CASES))
def test_summarize_parity(hils, name):
    wl, _ = CASES[name]
    say("summarize", name)
    x, xd = _inputs(wl, seed=1)
    sh = _shape(hils, wl)
    NC = wl.T // wl.S
    ks = torch.empty((wl.B, wl.Hq, NC, wl.d), dtype=wl.torch_dtype, device=DEV)
    bs = torch.empty((wl.B, wl.Hq, NC), dtype=torch.float32, device=DEV)
    hils.hils_summarize(xd["k"], xd["q_land"], ks, bs, sh)
    torch.cuda.synchronize()
    oks, obs = oracle.summarize(x["k"], x["q_land"], wl.S, wl.Hq,
                                ks_round=oracle.ks_round_for(wl.dtype))
    assert_close(bs, obs, 1e-5, what="b'")
    if wl.dtype == "bf16":
        # both sides round once to bf16: equal, or one bf16 step apart near a tie
        got = f64(ks)
        diff = np.abs(got - oks)
        step = np.abs(oks) * 2.0 ** -7 + 1e-30
        assert np.all(diff <= step * 1.0001), "k' differs by more than one bf16 step"
        assert np.mean(diff > 0) < 0.02
        assert_close(ks, oks, 1e-2, 5e-3, what="k'")
    else:
        assert_close(ks, oks, 1e-5, what="k'")


def _oracle_summaries_as_stored(x, wl):
    """The oracle's summaries, rounded to the storage dtypes, as host tensors."""
    oks, obs = oracle.summarize(x["k"], x["q_land"], wl.S, wl.Hq,
                                ks_round=oracle.ks_round_for(wl.dtype))
    return torch.from_numpy(oks).to(wl.torch_dtype), torch.from_numpy(obs).to(torch.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_select_stage_parity(hils, name):
    """hils_select on the oracle's stored summaries: ids and s_hat vs the oracle."""
    wl, _ = CASES[name]
    say("select", name)
    x, xd = _inputs(wl, seed=2)
    ks, bs = _oracle_summaries_as_stored(x, wl)
    sh = _shape(hils, wl)
    idx = torch.empty((wl.B, wl.Hkv, wl.T, wl.k), dtype=torch.int32, device=DEV)
    ssel = torch.empty((wl.B, wl.Hq, wl.T, wl.k), dtype=torch.float32, device=DEV)
    ws = hils.workspace(sh, hils.OP_SELECT, DEV)
    hils.hils_select(xd["q_hat"], ks.to(DEV), bs.to(DEV), idx, ssel, sh, ws)
    torch.cuda.synchronize()
    rb, rg, ri = rows_layout(wl.B, wl.Hkv, range(wl.T))
    orc = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], ks.double().numpy(),
                      bs.double().numpy(), S=wl.S, W=wl.W, topk=wl.k, want_r=True)
    gi = idx.cpu().numpy().reshape(-1, wl.k)
    res = check_selection(gi, orc, wl.k, TAU_STAGE)
    G = wl.G
    gs = gather_rows(ssel, rb, rg, ri, G)
    gL = gather_rows(hils.select_lse(ws, sh), rb, rg, ri, G) if G > 1 else None
    rk = check_rank_keys(gi, gpu_rank_keys(gs, gL, G), orc, wl.k, TAU_STAGE / 4, "rank keys")
    say("  decided", res["decided"], "undecided", res["undecided"], "differ", res["differ"].sum(),
        "rank-key max err %.3g on %d keys" % (rk["max_err"], rk["keys"]))
    same = ~res["differ"]
    o = orc["ssel"][same]
    g = gs[same]
    fin = np.isfinite(o)
    assert np.array_equal(fin, np.isfinite(g))
    assert_close(g[fin], o[fin], 2e-5, what="s_hat on selection")


@pytest.mark.parametrize("name", list(CASES))
def test_attend_stage_parity(hils, name):
    """hils_attend_fuse on the oracle's selection and scores: out and lse vs the oracle."""
    wl, _ = CASES[name]
    say("attend", name)
    x, xd = _inputs(wl, seed=3)
    ks, bs = _oracle_summaries_as_stored(x, wl)
    rb, rg, ri = rows_layout(wl.B, wl.Hkv, range(wl.T))
    orc = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], ks.double().numpy(),
                      bs.double().numpy(), S=wl.S, W=wl.W, topk=wl.k)
    dense = oracle.to_dense(orc, wl.B, wl.Hq, wl.Hkv, wl.T, wl.k)
    idx = torch.from_numpy(dense["idx"].astype(np.int32)).to(DEV)
    ssel = torch.from_numpy(dense["ssel"].astype(np.float32)).to(DEV)
    out = torch.empty_like(xd["q"])
    lse = torch.empty((wl.B, wl.Hq, wl.T), dtype=torch.float32, device=DEV)
    hils.hils_attend_fuse(xd["q"], xd["k"], xd["v"], idx, ssel, out, lse, _shape(hils, wl))
    torch.cuda.synchronize()
    t = tol_out(wl.torch_dtype)
    # the oracle's fusion used fp64 scores; the GPU reads them rounded to fp32
    assert_close(out, dense["out"], t["max_abs"], t["rel_l2"], what="out")
    assert_close(lse, dense["lse"], tol_lse(wl.torch_dtype), what="lse")


def _gpu_prefill(hils, xd, wl, k=None):
    r = hils.prefill(xd["q"], xd["k"], xd["v"], xd["q_land"], xd["q_hat"], S=wl.S, W=wl.W,
                     topk=wl.k if k is None else k)
    torch.cuda.synchronize()
    return r


def _e2e_check(hils, x, xd, wl, positions=None, seed_note=""):
    r = _gpu_prefill(hils, xd, wl)
    pos = range(wl.T) if positions is None else positions
    rb, rg, ri = rows_layout(wl.B, wl.Hkv, pos)
    ksr = oracle.ks_round_for(wl.dtype)
    oks, obs = oracle.summarize(x["k"], x["q_land"], wl.S, wl.Hq, ks_round=ksr)
    orc = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], oks, obs, S=wl.S,
                      W=wl.W, topk=wl.k, want_r=True)
    tau = TAU_E2E_BF16 if wl.dtype == "bf16" else TAU_E2E_F32
    G = wl.G
    gi = gather_rows(r["idx"], rb, rg, ri, 1)[:, 0].astype(np.int64) if wl.k > 0 else \
        np.zeros((len(rb), 0), np.int64)
    res = check_selection(gi, orc, wl.k, tau) if wl.k > 0 else {"differ": np.zeros(len(rb), bool),
                                                                 "decided": 0, "undecided": 0}
    if wl.k > 0:
        # the band's premise: the GPU's own rank keys on its choice, rebuilt from its
        # outputs, agree with the oracle's on the same stored summaries within TAU/4
        gs = gather_rows(r["ssel"], rb, rg, ri, G)
        gL = gather_rows(hils.select_lse(r["ws_select"], r["shape"]), rb, rg, ri, G) if G > 1 else None
        rgpu = gpu_rank_keys(gs, gL, G)
        orc_g = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], f64(r["k_sum"]),
                            f64(r["b_sum"]), S=wl.S, W=wl.W, topk=wl.k, want_r=True)
        rk = check_rank_keys(gi, rgpu, orc_g, wl.k, TAU_STAGE / 4, "rank keys (same summaries)")
        # against the oracle's own summaries the keys may move further by the two
        # sides' k' rounding, which is bounded from the measured k' difference
        qh_rows = gather_rows(xd["q_hat"], rb, rg, ri, G)
        kb = kprime_rank_bound(r["k_sum"], oks, qh_rows, rb, rg, G, oracle.default_scale(wl.d))
        rk2 = check_rank_keys(gi, rgpu, orc, wl.k, TAU_STAGE / 4 + kb, "rank keys (oracle k')")
        say("  rank keys: same summaries max err %.3g on %d keys; vs oracle k' %.3g (k' bound %.3g,"
            " tau/4 %.3g)" % (rk["max_err"], rk["keys"], rk2["max_err"], kb, tau / 4))
    say("  %s decided %d undecided %d differ %d" % (seed_note, res["decided"], res["undecided"],
                                                    res["differ"].sum()))
    out_g = gather_rows(r["out"], rb, rg, ri, G)
    lse_g = gather_rows(r["lse"], rb, rg, ri, G)
    want_out = orc["out"].copy()
    want_lse = orc["lse"].copy()
    d = res["differ"]
    if d.any():
        alt = oracle.rows(rb[d], rg[d], ri[d], ri[d], x["q"], x["q_hat"], x["k"], x["v"], oks, obs,
                          S=wl.S, W=wl.W, topk=wl.k, forced_idx=gi[d])
        want_out[d] = alt["out"]
        want_lse[d] = alt["lse"]
    t = tol_out(wl.torch_dtype)
    assert_close(out_g, want_out, t["max_abs"], t["rel_l2"], what="out")
    assert_close(lse_g, want_lse, tol_lse(wl.torch_dtype), what="lse")
    return r, orc, res


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_end_to_end(hils, name):
    wl, pos = CASES[name]
    say("e2e", name)
    x, xd = _inputs(wl, seed=4)
    _e2e_check(hils, x, xd, wl, pos, name)


def test_prefill_8k_needle(hils):
    """The 8K workload (32/8 heads, d=128, k=16, W=512, planted needle) on sampled rows."""
    wl = wk.CONFIGS["8k"]
    say("e2e 8k")
    x, xd = _inputs(wl, seed=0)
    m = x["meta"]
    pos = sorted(set([0, 1, 511, 512, 575, 576, 577, 1000, 2047, 4096, 6000, 8190, m["needle_query"]]
                     + list(range(7000, 7064))))
    r, orc, _ = _e2e_check(hils, x, xd, wl, pos, "8k")
    # the needle row of group 0 selects the needle chunk
    gi = r["idx"][0, 0, m["needle_query"]].cpu().tolist()
    assert m["needle_chunk"] in gi


@pytest.mark.parametrize("topk", [0, 1, 64])
def test_prefill_topk_edges(hils, topk):
    """k = 0 (window only), k = 1, and k = 64 >= |C_i| for every row (all candidates)."""
    wl = wk.custom(name="edge", dtype="bf16", B=1, Hq=4, Hkv=1, d=128, T=1000, S=64, k=topk, W=64)
    say("edge k", topk)
    x, xd = _inputs(wl, seed=5)
    _e2e_check(hils, x, xd, wl, None, "k=%d" % topk)


def test_prefill_short_sequences(hils):
    """T below one chunk, T below W + S (no candidate anywhere), T = W + S."""
    for T in (37, 64, 150, 192):
        wl = wk.custom(name="short", dtype="bf16", B=1, Hq=4, Hkv=2, d=64, T=T, S=64, k=2, W=128)
        say("short T", T)
        x, xd = _inputs(wl, seed=6)
        _e2e_check(hils, x, xd, wl, None, "T=%d" % T)


def test_select_exact_ties(hils):
    """Dyadic summaries: every score is exact in fp32, so ids match bit for bit, ties included."""
    for Hq, Hkv, dt in ((4, 1, torch.bfloat16), (4, 2, torch.float32), (1, 1, torch.bfloat16)):
        x = wk.make_dyadic_select(B=1, Hq=Hq, Hkv=Hkv, T=640, d=64, S=64, k=3, W=64, seed=7)
        say("dyadic", Hq, Hkv, dt)
        sh = hils.Shape.make(1, Hq, Hkv, 64, 64, 64, 3, 640, dt, x["scale"])
        qh = x["q_hat"].to(dt)
        ks = x["k_sum"].to(dt)
        assert torch.equal(qh.float(), x["q_hat"]) and torch.equal(ks.float(), x["k_sum"])
        idx = torch.empty((1, Hkv, 640, 3), dtype=torch.int32, device=DEV)
        ssel = torch.empty((1, Hq, 640, 3), dtype=torch.float32, device=DEV)
        hils.hils_select(qh.to(DEV), ks.to(DEV), x["b_sum"].to(DEV), idx, ssel, sh)
        torch.cuda.synchronize()
        rb, rg, ri = rows_layout(1, Hkv, range(640))
        dummy = np.zeros((1, Hkv, 640, 64))
        orc = oracle.rows(rb, rg, ri, ri, qh, qh, dummy, dummy, x["k_sum"].double().numpy(),
                          x["b_sum"].double().numpy(), S=64, W=64, topk=3, scale=x["scale"])
        gi = idx.cpu().numpy().reshape(-1, 3)
        np.testing.assert_array_equal(gi, orc["idx"])
        assert np.sum(orc["gap"] == 0) > 0      # real ties were decided by the index rule


def test_deterministic(hils):
    """Two runs give bitwise identical outputs."""
    wl = CASES["bf16_g4_d128"][0]
    x, xd = _inputs(wl, seed=8)
    a = _gpu_prefill(hils, xd, wl)
    b = _gpu_prefill(hils, xd, wl)
    for key in ("k_sum", "b_sum", "idx", "ssel", "out", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_values_of_ones_give_ones(hils):
    """Fused weights sum to one: V = 1 gives out = 1; V + u gives out + u."""
    wl = CASES["bf16_g4_d128"][0]
    x, xd = _inputs(wl, seed=9)
    xd["v"] = torch.ones_like(xd["v"])
    r = _gpu_prefill(hils, xd, wl)
    assert_close(r["out"], np.ones(r["out"].shape), 4e-3, what="ones")


def test_batch_independence(hils):
    wl = wk.custom(name="bi", dtype="bf16", B=2, Hq=4, Hkv=1, d=64, T=700, S=64, k=3, W=64)
    x, xd = _inputs(wl, seed=10)
    a = _gpu_prefill(hils, xd, wl)
    y = {k_: (v_.clone() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in xd.items()}
    for key in ("q", "k", "v", "q_land", "q_hat"):
        y[key][1] = torch.randn_like(y[key][1].float()).to(y[key].dtype)
    b = _gpu_prefill(hils, y, wl)
    for key in ("k_sum", "b_sum", "idx", "ssel", "out", "lse"):
        assert torch.equal(a[key][0], b[key][0]), key


def test_select_in_group_passes(hils):
    """A workspace too small for every (b, group)'s rank keys makes hils_select
    rank a few pairs per launch (here 1 and 3 of 8); idx and s_hat must equal the
    one-pass run bit for bit, and one byte less than a single pair is refused."""
    wl = wk.custom(name="selpasses", dtype="bf16", B=2, Hq=8, Hkv=4, d=128, T=3000, S=64, k=8, W=128)
    say("select passes")
    x, xd = _inputs(wl, seed=7)
    shape = _shape(hils, wl)
    full = _gpu_prefill(hils, xd, wl)
    NC = wl.T // wl.S
    ks = torch.empty((wl.B, wl.Hq, NC, wl.d), dtype=wl.torch_dtype, device=DEV)
    bs = torch.empty((wl.B, wl.Hq, NC), dtype=torch.float32, device=DEV)
    hils.hils_summarize(xd["k"], xd["q_land"], ks, bs, shape)
    al = lambda n: -(-n // 256) * 256
    J = next(j for j in (1, 4, 16, 32, 64) if 64 * j >= NC)
    fixed = al(wl.B * wl.Hq * wl.T * 4) + 256          # per-head LSE (G > 1)
    per = al(wl.T * 64 * J * 4)                        # one (b, group)'s rank keys
    assert hils.hils_workspace_bytes(shape, hils.OP_SELECT) == fixed + wl.B * wl.Hkv * per
    for pairs in (1, 3):
        ws = torch.empty(fixed + pairs * per, dtype=torch.uint8, device=DEV)
        idx = torch.empty((wl.B, wl.Hkv, wl.T, wl.k), dtype=torch.int32, device=DEV)
        ssel = torch.empty((wl.B, wl.Hq, wl.T, wl.k), dtype=torch.float32, device=DEV)
        hils.hils_select(xd["q_hat"], ks, bs, idx, ssel, shape, ws)
        torch.cuda.synchronize()
        assert torch.equal(idx, full["idx"]), pairs
        assert torch.equal(ssel, full["ssel"]), pairs
    small = torch.empty(fixed + per - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(hils.HilsError):
        hils.hils_select(xd["q_hat"], ks, bs, torch.empty_like(full["idx"]),
                         torch.empty_like(full["ssel"]), shape, small)


def test_attend_in_group_passes(hils):
    """A workspace too small for every KV head's partial outputs makes hils_attend_fuse
    run the selected part a few groups at a time (here 1 and 3 of 4 groups per
    pass); the outputs must equal the single-pass run bit for bit."""
    wl = wk.custom(name="passes", dtype="bf16", B=2, Hq=8, Hkv=4, d=128, T=700, S=64, k=4, W=128)
    say("attend passes")
    x, xd = _inputs(wl, seed=6)
    shape = _shape(hils, wl)
    full = _gpu_prefill(hils, xd, wl)
    full_bytes = hils.hils_workspace_bytes(shape, hils.OP_ATTEND_FUSE)
    per = -(-(wl.B * wl.G * wl.T * wl.k * wl.d * 2) // 256) * 256   # one KV head's partials
    fixed = full_bytes - wl.Hkv * per
    for heads in (1, 3):
        ws = torch.empty(fixed + heads * per, dtype=torch.uint8, device=DEV)
        out = torch.empty_like(xd["q"])
        lse = torch.empty((wl.B, wl.Hq, wl.T), dtype=torch.float32, device=DEV)
        hils.hils_attend_fuse(xd["q"], xd["k"], xd["v"], full["idx"], full["ssel"], out, lse, shape, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, full["out"]), heads
        assert torch.equal(lse, full["lse"]), heads
    small = torch.empty(fixed + per - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(hils.HilsError):
        hils.hils_attend_fuse(xd["q"], xd["k"], xd["v"], full["idx"], full["ssel"],
                              torch.empty_like(xd["q"]), None, shape, small)
