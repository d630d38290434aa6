"""GPU parity of hils_decode_multi (M adjacent new tokens per sequence per call)
against the fp64 oracle, call by call.

Token m of sequence b is the prefill row i = pos[b] + m on the cache that holds
every earlier token, the new ones included; the oracle evaluates exactly those
rows on its own host copy of the caches and its own summaries (updated when a
chunk completes), and the selection is compared with the end-to-end tie band.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from hils_testlib import TAU_E2E_BF16, TAU_E2E_F32, assert_close, check_selection, tol_lse, tol_out

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


def _step_inputs(wl, M, step, seed):
    """M tokens' q, q_hat, k_new, v_new ([B, M, H, d]) and q_land_new, drawn as M
    single decode steps of the generator."""
    xs = [wk.make_decode_step(wl, step * M + m, seed=seed) for m in range(M)]
    cat = lambda n: torch.stack([x[n] for x in xs], dim=1).contiguous()
    return {"q": cat("q"), "q_hat": cat("q_hat"), "k_new": cat("k_new"), "v_new": cat("v_new"),
            "q_land_new": xs[-1]["q_land_new"]}


def run_multi(hils, wl, M, starts, ncalls, seed=0):
    B, Hq, Hkv, d, S = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S
    G = Hq // Hkv
    cap = -(-(max(starts) + ncalls * M) // S) * S + S
    dt = wl.torch_dtype
    base = wk.make_decode_cache(wl, seed=seed, length=max(starts), capacity=cap)
    kc_h, vc_h, ql_h = base["k_cache"].clone(), base["v_cache"].clone(), base["q_land"].clone()
    for b in range(B):
        kc_h[b, :, starts[b]:] = 0
        vc_h[b, :, starts[b]:] = 0
    kc, vc = kc_h.to(DEV), vc_h.to(DEV)
    for b in range(B):   # rows past each sequence's length hold NaN until written
        kc[b, :, starts[b]:] = float("nan")
        vc[b, :, starts[b]:] = float("nan")
    NCcap = cap // S
    ks = torch.zeros((B, Hq, NCcap, d), dtype=dt, device=DEV)
    bs = torch.zeros((B, Hq, NCcap), dtype=torch.float32, device=DEV)
    shape = hils.Shape.make(B, Hq, Hkv, d, S, wl.W, wl.k, cap, dt)
    ql_d = ql_h.to(DEV)
    for b in range(B):
        nb_ = starts[b] // S
        if nb_:
            sb = hils.Shape.make(1, Hq, Hkv, d, S, wl.W, wl.k, cap, dt)
            hils.hils_summarize(kc[b:b + 1], ql_d[b:b + 1], ks[b:b + 1], bs[b:b + 1], sb, 0, nb_)
    nws = hils.hils_decode_multi_workspace_bytes(shape, M)
    assert nws > 0
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    out = torch.empty((B, M, Hq, d), dtype=dt, device=DEV)
    lse = torch.empty((B, M, Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, M, Hkv, max(wl.k, 1)), dtype=torch.int32, device=DEV)
    ksr = oracle.ks_round_for(wl.dtype)
    oks = np.zeros((B, Hq, NCcap, d))
    obs = np.zeros((B, Hq, NCcap))
    for b in range(B):
        nb_ = starts[b] // S
        if nb_:
            a_, b_ = oracle.summarize(kc_h[b:b + 1], ql_h[b:b + 1], S, Hq, ks_round=ksr, nc=nb_)
            oks[b, :, :nb_], obs[b, :, :nb_] = a_[0], b_[0]
    tau = TAU_E2E_BF16 if wl.dtype == "bf16" else TAU_E2E_F32
    n_dec = n_und = 0
    for st in range(ncalls):
        pos = [s_ + st * M for s_ in starts]
        x = _step_inputs(wl, M, st, seed)
        xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
        hils.hils_decode_multi(pos, M, xd["q"], xd["q_hat"], xd["k_new"], xd["v_new"], xd["q_land_new"],
                               kc, vc, ks, bs, out, lse, idx if wl.k > 0 else None, shape, ws)
        torch.cuda.synchronize()
        for b in range(B):
            for m in range(M):
                kc_h[b, :, pos[b] + m] = x["k_new"][b, m]
                vc_h[b, :, pos[b] + m] = x["v_new"][b, m]
        # oracle rows (b, g, i = pos[b] + m) with query row m of [B, Hq, M, d]
        rb, rg, rm = np.meshgrid(np.arange(B), np.arange(Hkv), np.arange(M), indexing="ij")
        rb, rg, rm = rb.ravel(), rg.ravel(), rm.ravel()
        ri = np.array([pos[b] + m for b, m in zip(rb, rm)], np.int64)
        qT = x["q"].transpose(1, 2).contiguous()       # [B, Hq, M, d]
        qhT = x["q_hat"].transpose(1, 2).contiguous()
        orc = oracle.rows(rb, rg, ri, rm, qT, qhT, kc_h, vc_h, oks, obs, S=S, W=wl.W, topk=wl.k,
                          want_r=True)
        if wl.k > 0:
            gi = idx.cpu().numpy()[rb, rm, rg][:, :wl.k]
            res = check_selection(gi, orc, wl.k, tau)
            n_dec += res["decided"]
            n_und += res["undecided"]
        else:
            res = {"differ": np.zeros(len(rb), bool)}
        want_out, want_lse = orc["out"].copy(), orc["lse"].copy()
        dm = res["differ"]
        if dm.any():
            alt = oracle.rows(rb[dm], rg[dm], ri[dm], rm[dm], qT, qhT, kc_h, vc_h, oks, obs, S=S, W=wl.W,
                              topk=wl.k, forced_idx=gi[dm])
            want_out[dm], want_lse[dm] = alt["out"], alt["lse"]
        o = out.cpu().to(torch.float64).numpy()          # [B, M, Hq, d]
        got = np.stack([o[b, m, g * G:(g + 1) * G] for b, g, m in zip(rb, rg, rm)])
        l_ = lse.cpu().to(torch.float64).numpy()
        gl = np.stack([l_[b, m, g * G:(g + 1) * G] for b, g, m in zip(rb, rg, rm)])
        t = tol_out(dt)
        assert_close(got, want_out, t["max_abs"], t["rel_l2"], what="out call %d" % st)
        assert_close(gl, want_lse, tol_lse(dt), what="lse call %d" % st)
        for b in range(B):   # chunk completed by these tokens
            for m in range(M):
                if (pos[b] + m + 1) % S == 0:
                    c = (pos[b] + m) // S
                    ql_h[b, :, c] = x["q_land_new"][b]
                    a_, b_ = oracle.summarize(kc_h[b:b + 1], ql_h[b:b + 1], S, Hq, ks_round=ksr, c0=c, nc=1,
                                              ks_NC=NCcap)
                    oks[b, :, c], obs[b, :, c] = a_[0, :, c], b_[0, :, c]
    say("  decided %d undecided %d" % (n_dec, n_und))
    return {"k_sum": ks, "b_sum": bs, "oks": oks, "obs": obs}


@pytest.mark.parametrize("name,wl,M,starts,ncalls", [
    ("gqa4_bf16_M4", wk.custom(name="m1", kind="decode", dtype="bf16", B=2, Hq=8, Hkv=2, d=128, T=2000,
                               S=64, k=6, W=256), 4, [2000, 1990], 40),
    ("mha_f32_M16", wk.custom(name="m2", kind="decode", dtype="f32", B=1, Hq=2, Hkv=2, d=64, T=700,
                              S=64, k=3, W=64), 16, [700], 10),
    ("g2_bf16_M8_short", wk.custom(name="m3", kind="decode", dtype="bf16", B=3, Hq=4, Hkv=2, d=64,
                                   T=60, S=64, k=4, W=100), 8, [60, 5, 0], 20),
    ("g8_bf16_M2", wk.custom(name="m4", kind="decode", dtype="bf16", B=2, Hq=8, Hkv=1, d=128, T=1500,
                             S=64, k=5, W=192), 2, [1500, 1473], 40),
    ("g4_bf16_M3_k0", wk.custom(name="m5", kind="decode", dtype="bf16", B=1, Hq=4, Hkv=1, d=128, T=900,
                                S=64, k=0, W=128), 3, [900], 10),
])
def test_decode_multi_matches_oracle(hils, name, wl, M, starts, ncalls):
    say("decode multi", name)
    r = run_multi(hils, wl, M, starts, ncalls, seed=13)
    ks = r["k_sum"].cpu().to(torch.float64).numpy()
    bs = r["b_sum"].cpu().to(torch.float64).numpy()
    for b, s0 in enumerate(starts):
        c_hi = (s0 + ncalls * M) // wl.S
        if c_hi:
            assert_close(bs[b, :, :c_hi], r["obs"][b, :, :c_hi], 1e-5, what="b' seq %d" % b)
            assert_close(ks[b, :, :c_hi], r["oks"][b, :, :c_hi], 2e-2 if wl.dtype == "bf16" else 1e-5,
                         5e-3, what="k' seq %d" % b)


def test_decode_multi_limits(hils):
    sh = hils.Shape.make(2, 8, 2, 128, 64, 256, 6, 4096, torch.bfloat16)   # G = 4
    assert hils.hils_decode_multi_workspace_bytes(sh, 4) > 0
    assert hils.hils_decode_multi_workspace_bytes(sh, 5) == 0        # M G > 16
    assert hils.hils_decode_multi_workspace_bytes(sh, 0) == 0
