"""GPU parity of the low-rank query calibration and of the shared-query summaries.

hils_qcal computes q + W_up (W_down h) in fp32 and rounds once; the oracle
computes it exactly and rounds once.  In fp32 the two agree to a few ulp.  In
bf16 they store the same value except where the exact value lies so close to a
rounding midpoint that the fp32 sum's own error decides the side (about 1e-6 of
the summed magnitudes, which can be many bf16 steps of a result that cancels
to near zero): there the GPU's value still rounds a number within that error
of the exact one.
End to end, the calibrated query feeds the selection and the attention; the
selection is compared with the end-to-end tie band, the outputs with the usual
bounds.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from hils_testlib import TAU_E2E_BF16, assert_close, check_selection, f64, gather_rows, tol_lse, tol_out

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hils():
    import chunk_wise_sparse_summary_amd as h
    h.lib()
    return h


QCASES = {
    "f32_h1_d64": (wk.custom(name="qa", dtype="f32", B=1, Hq=1, Hkv=1, d=64, T=1024, S=64, k=4, W=64), 64, 16),
    "bf16_h8_d128_ragged": (wk.custom(name="qb", dtype="bf16", B=2, Hq=8, Hkv=2, d=128, T=700, S=64, k=6,
                                      W=128), 1024, 64),
    "bf16_h4_d64_r128": (wk.custom(name="qc", dtype="bf16", B=1, Hq=4, Hkv=1, d=64, T=333, S=64, k=3,
                                   W=64), 256, 128),
    "f32_h4_d128_r32": (wk.custom(name="qd", dtype="f32", B=1, Hq=4, Hkv=2, d=128, T=200, S=64, k=3,
                                  W=64), 96, 32),
    "bf16_h2_d128_r16": (wk.custom(name="qe", dtype="bf16", B=1, Hq=2, Hkv=1, d=128, T=150, S=64, k=3,
                                   W=64), 64, 16),
}


def _gpu_qcal(hils, wl, xd, cd):
    sh = hils.Shape.make(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T, wl.torch_dtype)
    qh = torch.full_like(xd["q"], float("nan"))
    hils.hils_qcal(xd["q"], cd["h"], cd["w_down"], cd["w_up"], qh, sh)
    torch.cuda.synchronize()
    return qh


def _check_qcal(got, x, c, wl):
    mode = oracle.ORND_BF16 if wl.dtype == "bf16" else oracle.ORND_F32
    want = oracle.qcal(x["q"], c["h"], c["w_down"], c["w_up"], mode)
    g = f64(got)
    assert np.all(np.isfinite(g))
    if wl.dtype == "f32":
        exact = oracle.qcal(x["q"], c["h"], c["w_down"], c["w_up"], oracle.ORND_NONE)
        err = np.abs(g - exact)
        bound = 2e-6 * (np.abs(exact) + np.abs(f64(x["q"])) + 1.0)
        say("    fp32 q_hat: max error / bound %.3g" % float((err / bound).max()))
        assert np.all(err <= bound), float((err / bound).max())
        return 0
    diff = g != want
    n = int(diff.sum())
    if n:
        exact = oracle.qcal(x["q"], c["h"], c["w_down"], c["w_up"], oracle.ORND_NONE)[diff]
        qd = f64(x["q"])[diff]
        # the GPU's fp32 value is the exact one within eps: the fp32 sums of the
        # two products and the add err by a few units of 2^-24 of the summed
        # magnitudes (about 1e-7 of |q| + |correction| here; eps allows 4e-6);
        # its bf16 rounding then lies within half a bf16 step of that value
        eps = 4e-6 * (np.abs(qd) + np.abs(exact - qd)) + 4e-7
        mag = np.maximum(np.abs(g[diff]), np.abs(exact))
        half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-38))) - 8)
        assert np.all(np.abs(g[diff] - exact) <= half_ulp + eps), \
            float((np.abs(g[diff] - exact) / (half_ulp + eps)).max())
    say("    q_hat elements rounded to the other side: %d of %d" % (n, diff.size))
    assert n <= max(4, diff.size // 1000)
    return n


@pytest.mark.parametrize("name", list(QCASES))
def test_qcal_matches_oracle(hils, name):
    wl, dm, r = QCASES[name]
    say("qcal", name)
    x = wk.make_prefill(wl, seed=31)
    c = wk.make_qcal(wl, dm, r, seed=31)
    xd = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    cd = {k_: v_.to(DEV) for k_, v_ in c.items()}
    _check_qcal(_gpu_qcal(hils, wl, xd, cd), x, c, wl)


def test_qcal_end_to_end(hils):
    """Calibrated query -> selection -> attention, against the oracle's own q_hat."""
    wl, dm, r = QCASES["bf16_h8_d128_ragged"]
    say("qcal end to end")
    x = wk.make_prefill(wl, seed=32)
    c = wk.make_qcal(wl, dm, r, seed=32)
    xd = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    cd = {k_: v_.to(DEV) for k_, v_ in c.items()}
    qh = _gpu_qcal(hils, wl, xd, cd)
    _check_qcal(qh, x, c, wl)
    res = hils.prefill(xd["q"], xd["k"], xd["v"], xd["q_land"], qh, S=wl.S, W=wl.W, topk=wl.k)
    torch.cuda.synchronize()
    # the oracle's stored q_hat (bf16 values, so the conversion is exact)
    oqh = torch.from_numpy(oracle.qcal(x["q"], c["h"], c["w_down"], c["w_up"], oracle.ORND_BF16)).to(torch.bfloat16)
    rb, rg, ri = np.meshgrid(np.arange(wl.B), np.arange(wl.Hkv), np.arange(wl.T), indexing="ij")
    rb, rg, ri = rb.ravel(), rg.ravel(), ri.ravel()
    oks, obs = oracle.summarize(x["k"], x["q_land"], wl.S, wl.Hq, ks_round=oracle.ks_round_for(wl.dtype))
    orc = oracle.rows(rb, rg, ri, ri, x["q"], oqh, x["k"], x["v"], oks, obs, S=wl.S, W=wl.W, topk=wl.k,
                      want_r=True)
    gi = res["idx"].cpu().numpy()[rb, rg, ri]
    sel = check_selection(gi, orc, wl.k, TAU_E2E_BF16)
    say("    decided %d undecided %d differ %d" % (sel["decided"], sel["undecided"], sel["differ"].sum()))
    G = wl.Hq // wl.Hkv
    out = gather_rows(res["out"], rb, rg, ri, G)
    lse = gather_rows(res["lse"], rb, rg, ri, G)
    want_out, want_lse = orc["out"].copy(), orc["lse"].copy()
    d = sel["differ"]
    if d.any():
        alt = oracle.rows(rb[d], rg[d], ri[d], ri[d], x["q"], oqh, x["k"], x["v"], oks, obs, S=wl.S, W=wl.W,
                          topk=wl.k, forced_idx=gi[d])
        want_out[d], want_lse[d] = alt["out"], alt["lse"]
    t = tol_out(wl.torch_dtype)
    assert_close(out, want_out, t["max_abs"], t["rel_l2"], what="out")
    assert_close(lse, want_lse, tol_lse(wl.torch_dtype), what="lse")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_summarize_shared_query(hils, dtype):
    """One query per head for every chunk: identical to hils_summarize on the
    replicated query (bit for bit), and to the oracle."""
    wl = wk.custom(name="sq", dtype=dtype, B=2, Hq=8, Hkv=2, d=128, T=1000, S=64, k=4, W=64)
    say("shared query", dtype)
    x = wk.make_prefill(wl, seed=33)
    qs = x["q_land"][0, :, 0].contiguous()                  # [Hq, d]
    NC = wl.T // wl.S
    rep = qs[None, :, None, :].expand(wl.B, wl.Hq, NC, wl.d).contiguous()
    sh = hils.Shape.make(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T, wl.torch_dtype)
    kd = x["k"].to(DEV)
    ks1 = torch.empty((wl.B, wl.Hq, NC, wl.d), dtype=wl.torch_dtype, device=DEV)
    bs1 = torch.empty((wl.B, wl.Hq, NC), dtype=torch.float32, device=DEV)
    ks2, bs2 = torch.empty_like(ks1), torch.empty_like(bs1)
    hils.hils_summarize_shared(kd, qs.to(DEV), ks1, bs1, sh)
    hils.hils_summarize(kd, rep.to(DEV), ks2, bs2, sh)
    torch.cuda.synchronize()
    assert torch.equal(ks1, ks2) and torch.equal(bs1, bs2)
    oks, obs = oracle.summarize(x["k"], rep, wl.S, wl.Hq, ks_round=oracle.ks_round_for(wl.dtype))
    assert_close(bs1, obs, 1e-5, what="b'")
    tol = 2e-2 if dtype == "bf16" else 1e-5
    assert_close(ks1, oks, tol, 5e-3 if dtype == "bf16" else 1e-5, what="k'")


@pytest.mark.parametrize("name", ["bf16_h8_d128_ragged", "f32_h4_d128_r32", "bf16_h2_d128_r16",
                                  "bf16_h4_d64_r128", "f32_h1_d64"])
def test_select_qcal_fused_is_qcal_then_select(hils, name):
    """Q-Cal fused into the selection's scoring pass stores the same q_hat and
    makes the same selection and scores as hils_qcal followed by hils_select,
    bit for bit (G = 1 included, where the pass only forms q_hat); q_hat itself
    is pinned to the oracle above."""
    wl, dm, r = QCASES[name]
    say("select with fused qcal", name)
    x = wk.make_prefill(wl, seed=34)
    c = wk.make_qcal(wl, dm, r, seed=34)
    xd = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    cd = {k_: v_.to(DEV) for k_, v_ in c.items()}
    sh = hils.Shape.make(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T, wl.torch_dtype)
    NC = wl.T // wl.S
    ks = torch.empty((wl.B, wl.Hq, NC, wl.d), dtype=wl.torch_dtype, device=DEV)
    bs = torch.empty((wl.B, wl.Hq, NC), dtype=torch.float32, device=DEV)
    hils.hils_summarize(xd["k"], xd["q_land"], ks, bs, sh)
    # separate: Q-Cal, then the selection on its output
    qh1 = _gpu_qcal(hils, wl, xd, cd)
    idx1 = torch.full((wl.B, wl.Hkv, wl.T, wl.k), -7, dtype=torch.int32, device=DEV)
    sc1 = torch.full((wl.B, wl.Hq, wl.T, wl.k), 7.0, dtype=torch.float32, device=DEV)
    hils.hils_select(qh1, ks, bs, idx1, sc1, sh)
    # fused
    qh2 = torch.full_like(qh1, float("nan"))
    idx2 = torch.full_like(idx1, -7)
    sc2 = torch.full_like(sc1, 7.0)
    hils.hils_select_qcal(xd["q"], cd["h"], cd["w_down"], cd["w_up"], ks, bs, qh2, idx2, sc2, sh)
    torch.cuda.synchronize()
    assert torch.equal(qh1.view(torch.int16) if qh1.dtype == torch.bfloat16 else qh1.view(torch.int32),
                       qh2.view(torch.int16) if qh2.dtype == torch.bfloat16 else qh2.view(torch.int32))
    assert torch.equal(idx1, idx2)
    assert torch.equal(sc1.view(torch.int32), sc2.view(torch.int32))
    _check_qcal(qh2, x, c, wl)
