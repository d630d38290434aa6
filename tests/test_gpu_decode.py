"""GPU parity of hils_decode_step against the fp64 oracle, step by step.

The oracle keeps its own host copy of the caches, built from the generator's
bytes (initial cache plus each step's k_new / v_new), and its own summaries
(initial landmark queries plus each step's q_land_new at chunk completions).
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


def run_decode(hils, wl, starts, nsteps, seed=0, check_every=1, poison=False):
    B, Hq, Hkv, d, S = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S
    G = Hq // Hkv
    cap = -(-(max(starts) + nsteps) // S) * S + S
    dt = wl.torch_dtype
    base = wk.make_decode_cache(wl, seed=seed, length=max(starts), capacity=cap)
    kc_h, vc_h, ql_h = base["k_cache"].clone(), base["v_cache"].clone(), base["q_land"].clone()
    for b in range(B):                      # each sequence holds exactly starts[b] tokens
        kc_h[b, :, starts[b]:] = 0
        vc_h[b, :, starts[b]:] = 0
    kc, vc = kc_h.to(DEV), vc_h.to(DEV)
    if poison:   # rows past each sequence's length hold NaN until a step writes them
        for b in range(B):
            kc[b, :, starts[b]:] = float("nan")
            vc[b, :, starts[b]:] = float("nan")
    NCcap = cap // S
    ks = torch.zeros((B, Hq, NCcap, d), dtype=dt, device=DEV)
    bs = torch.zeros((B, Hq, NCcap), dtype=torch.float32, device=DEV)
    shape = hils.Shape.make(B, Hq, Hkv, d, S, wl.W, wl.k, cap, dt)
    ql_d = ql_h.to(DEV)
    for b in range(B):                      # summaries of every complete chunk
        nb_ = starts[b] // S
        if nb_:
            sb = hils.Shape.make(1, Hq, Hkv, d, S, wl.W, wl.k, cap, dt)
            hils.hils_summarize(kc[b:b + 1], ql_d[b:b + 1], ks[b:b + 1], bs[b:b + 1], sb, 0, nb_)
    ws = hils.workspace(shape, hils.OP_DECODE, DEV)
    out = torch.empty((B, Hq, d), dtype=dt, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, max(wl.k, 1)), dtype=torch.int32, device=DEV)
    # oracle state
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
    hist = []
    for st in range(nsteps):
        pos = [s_ + st for s_ in starts]
        x = wk.make_decode_step(wl, st, seed=seed)
        xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
        hils.hils_decode_step(pos, xd["q"], xd["q_hat"], xd["k_new"], xd["v_new"], xd["q_land_new"],
                              kc, vc, ks, bs, out, lse, idx if wl.k > 0 else None, shape, ws)
        torch.cuda.synchronize()
        for b in range(B):
            kc_h[b, :, pos[b]] = x["k_new"][b]
            vc_h[b, :, pos[b]] = x["v_new"][b]
        if st % check_every == 0:
            rb = np.repeat(np.arange(B), Hkv).astype(np.int32)
            rg = np.tile(np.arange(Hkv), B).astype(np.int32)
            ri = np.array([pos[b] for b in rb], np.int64)
            rq = np.zeros_like(ri)
            qh = x["q_hat"][:, :, None, :]
            q = x["q"][:, :, None, :]
            # rows of sequence b use query row 0 of their own batch entry
            orc = oracle.rows(rb, rg, ri, rq, q, qh, kc_h, vc_h, oks, obs, S=S, W=wl.W, topk=wl.k,
                              want_r=True)
            gi = idx.cpu().numpy().reshape(B * Hkv, -1)[:, :wl.k]
            res = check_selection(gi, orc, wl.k, tau) if wl.k > 0 else {"differ": np.zeros(len(rb), bool),
                                                                        "decided": 0, "undecided": 0}
            n_dec += res["decided"]
            n_und += res["undecided"]
            want_out, want_lse = orc["out"].copy(), orc["lse"].copy()
            dmask = res["differ"]
            if dmask.any():
                alt = oracle.rows(rb[dmask], rg[dmask], ri[dmask], rq[dmask], q, qh, kc_h, vc_h, oks,
                                  obs, S=S, W=wl.W, topk=wl.k, forced_idx=gi[dmask])
                want_out[dmask], want_lse[dmask] = alt["out"], alt["lse"]
            got = out.cpu().to(torch.float64).numpy().reshape(B, Hkv, G, d).reshape(B * Hkv, G, d)
            gl = lse.cpu().to(torch.float64).numpy().reshape(B * Hkv, G)
            t = tol_out(dt)
            assert_close(got, want_out, t["max_abs"], t["rel_l2"], what="out step %d" % st)
            assert_close(gl, want_lse, tol_lse(dt), what="lse step %d" % st)
            hist.append(gi.copy())
        for b in range(B):                   # chunk completed by this step's token
            if (pos[b] + 1) % S == 0:
                c = pos[b] // S
                ql_h[b, :, c] = x["q_land_new"][b]
                a_, b_ = oracle.summarize(kc_h[b:b + 1], ql_h[b:b + 1], S, Hq, ks_round=ksr, c0=c,
                                          nc=1, ks_NC=NCcap)
                oks[b, :, c], obs[b, :, c] = a_[0, :, c], b_[0, :, c]
    say("  decode decided %d undecided %d" % (n_dec, n_und))
    return {"k_sum": ks, "b_sum": bs, "oks": oks, "obs": obs, "kc": kc, "kc_h": kc_h}


@pytest.mark.parametrize("name,wl,starts,nsteps", [
    ("gqa_bf16", wk.custom(name="d1", kind="decode", dtype="bf16", B=2, Hq=8, Hkv=2, d=128, T=2000,
                          S=64, k=6, W=256), [2000, 1990], 140),
    ("mha_f32", wk.custom(name="d2", kind="decode", dtype="f32", B=1, Hq=2, Hkv=2, d=64, T=700,
                          S=64, k=3, W=64), [700], 70),
    ("g8_bf16_short", wk.custom(name="d3", kind="decode", dtype="bf16", B=3, Hq=8, Hkv=1, d=64,
                               T=60, S=64, k=4, W=100), [60, 5, 0], 130),
])
def test_decode_matches_oracle(hils, name, wl, starts, nsteps):
    say("decode", name)
    r = run_decode(hils, wl, starts, nsteps, seed=11)
    # incremental summaries of completed chunks match the oracle's
    ks = r["k_sum"].cpu().to(torch.float64).numpy()
    bs = r["b_sum"].cpu().to(torch.float64).numpy()
    for b, s0 in enumerate(starts):
        c_hi = (s0 + nsteps) // wl.S
        if c_hi:
            assert_close(bs[b, :, :c_hi], r["obs"][b, :, :c_hi], 1e-5, what="b' seq %d" % b)
            assert_close(ks[b, :, :c_hi], r["oks"][b, :, :c_hi], 2e-2 if wl.dtype == "bf16" else 1e-5,
                         5e-3, what="k' seq %d" % b)


def test_decode_ignores_unwritten_rows(hils):
    """Cache rows past each position hold NaN: the step must read only rows <= pos."""
    wl = wk.custom(name="d4", kind="decode", dtype="bf16", B=2, Hq=8, Hkv=2, d=128, T=1500, S=64,
                   k=4, W=192)
    say("decode with NaN past the written rows")
    run_decode(hils, wl, [1500, 1473], 70, seed=12, poison=True)

