"""Parity at the full workload sizes, in the launch configuration the benchmark
times: the 128K prefill (B=1, 32/8 heads, d=128, S=64, k=32, W=1024, per-head
scales), 512K decode (B=4, k=32) and 4M decode (B=1, k=64, 8 planted needles).

The GPU runs the whole path through the C ABI on device-drawn inputs; the fp64
oracle reads back the exact device bytes and evaluates a seeded sample of query
rows (every KV group of each sampled position), so the comparison is element
by element on those rows.  Properties that hold for every row (ids ascending,
in range, padded; finite outputs) are checked on the full outputs.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from hils_testlib import (TAU_E2E_BF16, TAU_STAGE, assert_close, check_rank_keys, check_selection,
                          f64, gather_rows, gpu_rank_keys, kprime_rank_bound, rows_layout, tol_lse,
                          tol_out)

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


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_idx_all_rows(idx, T, S, W, k):
    """Every row: min(k, |C_i|) ids, strictly ascending, in [0, |C_i|), then -1 pads."""
    i = torch.arange(T, device=idx.device, dtype=torch.int64)
    a = i - W + 1
    lw = torch.where(a > 0, torch.div(a, S, rounding_mode="floor") * S, torch.zeros_like(a))
    nc = lw // S                                           # |C_i|
    nsel = torch.clamp(nc, max=k)
    slot = torch.arange(k, device=idx.device)
    want_valid = slot[None, :] < nsel[:, None]             # [T, k]
    x = idx.to(torch.int64)                                # [B, Hkv, T, k]
    valid = x >= 0
    assert torch.equal(valid, want_valid.expand_as(valid)), "valid-slot pattern"
    assert bool((x[~valid] == -1).all()), "pads must be -1"
    assert bool((x < nc[None, None, :, None]).all()), "ids beyond the candidate set"
    inc = x[..., 1:] > x[..., :-1]
    both = valid[..., 1:]
    assert bool(inc[both].all()), "ids not strictly ascending"


def test_prefill_128k_sampled(hils):
    wl = wk.CONFIGS["128k"]
    B, Hq, Hkv, d, S, W, k, T = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T
    say("128k: drawing inputs on the device")
    x = wk.make_prefill(wl, seed=0, device=DEV)
    NC = T // S
    shape = hils.Shape.make(B, Hq, Hkv, d, S, W, k, T, torch.bfloat16)
    k_sum = torch.empty((B, Hq, NC, d), dtype=torch.bfloat16, device=DEV)
    b_sum = torch.empty((B, Hq, NC), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, T, k), dtype=torch.int32, device=DEV)
    ssel = torch.empty((B, Hq, T, k), dtype=torch.float32, device=DEV)
    out = torch.empty_like(x["q"])
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)
    ws_sel = hils.workspace(shape, hils.OP_SELECT, DEV)
    ws_att = hils.workspace(shape, hils.OP_ATTEND_FUSE, DEV)
    say("128k: GPU path")
    hils.hils_summarize(x["k"], x["q_land"], k_sum, b_sum, shape)
    hils.hils_select(x["q_hat"], k_sum, b_sum, idx, ssel, shape, ws_sel)
    hils.hils_attend_fuse(x["q"], x["k"], x["v"], idx, ssel, out, lse, shape, ws_att)
    torch.cuda.synchronize()
    _check_idx_all_rows(idx, T, S, W, k)
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())

    rng = np.random.Generator(np.random.PCG64(128))
    pos = sorted(set([0, 1, 1023, 1086, 1087, 1088, 4095, 65535, 65536, 131070, T - 1]
                     + rng.integers(1087, T, size=21).tolist()))
    say("128k: oracle on %d positions x %d groups" % (len(pos), Hkv))
    k_h, v_h, ql_h = x["k"].cpu(), x["v"].cpu(), x["q_land"].cpu()
    oks, obs = oracle.summarize(k_h, ql_h, S, Hq, ks_round=oracle.ks_round_for("bf16"))
    # k' and b' of every chunk
    assert_close(b_sum.cpu(), obs, 1e-5, what="b'")
    assert_close(k_sum.cpu(), oks, 2e-2, 5e-3, what="k'")
    q_rows = x["q"][:, :, pos].cpu()
    qh_rows = x["q_hat"][:, :, pos].cpu()
    rb, rg, rq = rows_layout(B, Hkv, range(len(pos)))
    ri = np.asarray(pos, np.int64)[rq]
    orc = oracle.rows(rb, rg, ri, rq, q_rows, qh_rows, k_h, v_h, oks, obs, S=S, W=W, topk=k,
                      want_r=True)
    gi = gather_rows(idx, rb, rg, ri, 1)[:, 0].astype(np.int64)
    res = check_selection(gi, orc, k, TAU_E2E_BF16)
    say("  decided %d undecided %d differ %d" % (res["decided"], res["undecided"], res["differ"].sum()))
    # rank keys of the GPU's choice rebuilt from its outputs (s_hat on the choice,
    # each head's L_h from the select workspace) vs the oracle on the same summaries
    G = wl.G
    gs_all = gather_rows(ssel, rb, rg, ri, G)
    gL = gather_rows(hils.select_lse(ws_sel, shape), rb, rg, ri, G)
    rgpu = gpu_rank_keys(gs_all, gL, G)
    orc_g = oracle.rows(rb, rg, ri, rq, q_rows, qh_rows, k_h, v_h, f64(k_sum), f64(b_sum), S=S,
                        W=W, topk=k, want_r=True)
    rk = check_rank_keys(gi, rgpu, orc_g, k, TAU_STAGE / 4, "rank keys (same summaries)")
    qh64 = qh_rows.to(torch.float64).numpy()
    qh_r = np.stack([qh64[b_, g_ * G:(g_ + 1) * G, rq_] for b_, g_, rq_ in zip(rb, rg, rq)])
    kb = kprime_rank_bound(k_sum, oks, qh_r, rb, rg, G, 1.0 / np.sqrt(d))
    rk2 = check_rank_keys(gi, rgpu, orc, k, TAU_STAGE / 4 + kb, "rank keys (oracle k')")
    say("  rank keys: same summaries max err %.3g on %d keys; vs oracle k' %.3g (k' bound %.3g)"
        % (rk["max_err"], rk["keys"], rk2["max_err"], kb))
    want_out, want_lse = orc["out"].copy(), orc["lse"].copy()
    dm = res["differ"]
    if dm.any():
        alt = oracle.rows(rb[dm], rg[dm], ri[dm], rq[dm], q_rows, qh_rows, k_h, v_h, oks, obs, S=S,
                          W=W, topk=k, forced_idx=gi[dm])
        want_out[dm], want_lse[dm] = alt["out"], alt["lse"]
    t = tol_out(torch.bfloat16)
    assert_close(gather_rows(out, rb, rg, ri, wl.G), want_out, t["max_abs"], t["rel_l2"], what="out")
    assert_close(gather_rows(lse, rb, rg, ri, wl.G), want_lse, tol_lse(torch.bfloat16), what="lse")
    # each head's score on the chosen chunks, where the selection agrees
    same = ~dm
    gs = gather_rows(ssel, rb, rg, ri, wl.G)
    osel = orc["ssel"]
    fin = np.isfinite(osel) & same[:, None, None]
    assert np.array_equal(np.isfinite(gs) & same[:, None, None], fin)
    assert_close(gs[fin], osel[fin], 1e-4, what="s_hat on the selection")
    del x, k_sum, b_sum, idx, ssel, out, lse, ws_sel, ws_att
    _free()


def _decode_run(hils, wl, seed, nsteps, check_steps, needles=False):
    """Run nsteps decode steps from the workload's cache length; compare every
    (b, g) row with the oracle at check_steps.  Returns per-step GPU ids."""
    B, Hq, Hkv, d, S, W, k = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k
    say("%s: drawing the cache on the device" % wl.name)
    cache = wk.make_decode_cache(wl, seed=seed, device=DEV)
    L0, cap = cache["length"], cache["capacity"]
    NCcap = cap // S
    shape = hils.Shape.make(B, Hq, Hkv, d, S, W, k, cap, torch.bfloat16)
    ks = torch.empty((B, Hq, NCcap, d), dtype=torch.bfloat16, device=DEV)
    bs = torch.empty((B, Hq, NCcap), dtype=torch.float32, device=DEV)
    hils.hils_summarize(cache["k_cache"], cache["q_land"], ks, bs, shape, 0, L0 // S)
    ws = hils.workspace(shape, hils.OP_DECODE, DEV)
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    say("%s: host copies and oracle summaries" % wl.name)
    kc_h, vc_h, ql_h = cache["k_cache"].cpu(), cache["v_cache"].cpu(), cache["q_land"].cpu()
    ksr = oracle.ks_round_for("bf16")
    oks = np.zeros((B, Hq, NCcap, d))
    obs = np.zeros((B, Hq, NCcap))
    oracle.summarize(kc_h, ql_h, S, Hq, ks_round=ksr, c0=0, nc=L0 // S, ks_NC=NCcap, ksum=oks,
                     bsum=obs)
    dirs = cache["meta"].get("needle_dirs") if needles else None
    hist = []
    n_dec = n_und = 0
    for st in range(nsteps):
        p = L0 + st
        x = wk.make_decode_step(wl, st, seed=seed, needle_dirs=dirs)
        xd = {n_: v_.to(DEV) for n_, v_ in x.items()}
        hils.hils_decode_step([p] * B, xd["q"], xd["q_hat"], xd["k_new"], xd["v_new"],
                              xd["q_land_new"], cache["k_cache"], cache["v_cache"], ks, bs, out,
                              lse, idx, shape, ws)
        torch.cuda.synchronize()
        kc_h[:, :, p] = x["k_new"]
        vc_h[:, :, p] = x["v_new"]
        gi_all = idx.cpu().numpy().reshape(B * Hkv, k).astype(np.int64)
        hist.append(gi_all)
        if st in check_steps:
            say("%s: oracle at step %d" % (wl.name, st))
            rb = np.repeat(np.arange(B), Hkv).astype(np.int32)
            rg = np.tile(np.arange(Hkv), B).astype(np.int32)
            ri = np.full(B * Hkv, p, np.int64)
            rq = np.zeros_like(ri)
            q4, qh4 = x["q"][:, :, None, :], x["q_hat"][:, :, None, :]
            orc = oracle.rows(rb, rg, ri, rq, q4, qh4, kc_h, vc_h, oks, obs, S=S, W=W, topk=k,
                              want_r=True)
            if needles:   # the planted needles stand clear of the haystack in the oracle
                nd = np.asarray(cache["meta"]["needle_chunks"], np.int64)
                for t_ in range(B * Hkv):
                    r = orc["r"][t_, :orc["ncand"][t_]]
                    hay = np.ones(len(r), bool)
                    hay[nd] = False
                    assert r[nd].min() - r[hay].max() > 1.0, ("needle gap", st, t_)
            res = check_selection(gi_all, orc, k, TAU_E2E_BF16)
            n_dec += res["decided"]
            n_und += res["undecided"]
            want_out, want_lse = orc["out"].copy(), orc["lse"].copy()
            dm = res["differ"]
            if dm.any():
                alt = oracle.rows(rb[dm], rg[dm], ri[dm], rq[dm], q4, qh4, kc_h, vc_h, oks, obs,
                                  S=S, W=W, topk=k, forced_idx=gi_all[dm])
                want_out[dm], want_lse[dm] = alt["out"], alt["lse"]
            G = Hq // Hkv
            got = out.cpu().double().numpy().reshape(B * Hkv, G, d)
            gl = lse.cpu().double().numpy().reshape(B * Hkv, G)
            t = tol_out(torch.bfloat16)
            assert_close(got, want_out, t["max_abs"], t["rel_l2"], what="out step %d" % st)
            assert_close(gl, want_lse, tol_lse(torch.bfloat16), what="lse step %d" % st)
        if (p + 1) % S == 0:      # this step completed chunk p // S: oracle summary too
            c = p // S
            ql_h[:, :, c] = x["q_land_new"]
            oracle.summarize(kc_h, ql_h, S, Hq, ks_round=ksr, c0=c, nc=1, ks_NC=NCcap, ksum=oks,
                             bsum=obs)
            assert_close(bs[:, :, c].cpu(), obs[:, :, c], 1e-5, what="b' of completed chunk")
            assert_close(ks[:, :, c].cpu(), oks[:, :, c], 2e-2, 5e-3, what="k' of completed chunk")
    say("  %s decided %d undecided %d" % (wl.name, n_dec, n_und))
    meta = cache["meta"]
    del cache, ks, bs, ws, out, lse, idx, kc_h, vc_h, oks, obs
    _free()
    return hist, meta


def test_prefill_512k_sampled(hils):
    """The 512K context as one prefill (8192 chunks, 128 rank keys per lane): the
    selection and the chunk pass each run one KV group at a time (workspaces of
    one group's share), sampled rows against the oracle."""
    wl = wk.custom(name="512k_prefill", kind="prefill", dtype="bf16", B=1, Hq=32, Hkv=8, d=128,
                   T=524288, S=64, k=32, W=1024, head_scale=(0.5, 2.0))
    B, Hq, Hkv, d, S, W, k, T = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T
    G = Hq // Hkv
    say("512k prefill: drawing inputs on the device")
    x = wk.make_prefill(wl, seed=5, device=DEV)
    NC = T // S
    shape = hils.Shape.make(B, Hq, Hkv, d, S, W, k, T, torch.bfloat16)
    k_sum = torch.empty((B, Hq, NC, d), dtype=torch.bfloat16, device=DEV)
    b_sum = torch.empty((B, Hq, NC), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Hkv, T, k), dtype=torch.int32, device=DEV)
    ssel = torch.empty((B, Hq, T, k), dtype=torch.float32, device=DEV)
    out = torch.empty_like(x["q"])
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)
    # one (b, group) pair's share of each workspace: the calls make passes
    per_sel = T * 64 * 128 * 4                       # rank keys of one group
    per_att = T * k * G * d * 2                      # partial records of one group
    n_sel = hils.hils_workspace_bytes(shape, hils.OP_SELECT) - (B * Hkv - 1) * per_sel
    n_att = hils.hils_workspace_bytes(shape, hils.OP_ATTEND_FUSE) - (Hkv - 1) * per_att
    say("512k prefill: workspaces %.1f + %.1f GiB" % (n_sel / 2**30, n_att / 2**30))
    ws_sel = torch.empty(n_sel, dtype=torch.uint8, device=DEV)
    ws_att = torch.empty(n_att, dtype=torch.uint8, device=DEV)
    say("512k prefill: GPU path")
    hils.hils_summarize(x["k"], x["q_land"], k_sum, b_sum, shape)
    hils.hils_select(x["q_hat"], k_sum, b_sum, idx, ssel, shape, ws_sel)
    hils.hils_attend_fuse(x["q"], x["k"], x["v"], idx, ssel, out, lse, shape, ws_att)
    torch.cuda.synchronize()
    del ws_sel, ws_att
    _free()
    _check_idx_all_rows(idx, T, S, W, k)
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.Generator(np.random.PCG64(512))
    pos = sorted(set([1087, 131071, 262143, 262144, 393216, T - 1] + rng.integers(1087, T, size=10).tolist()))
    say("512k prefill: oracle on %d positions x %d groups" % (len(pos), Hkv))
    k_h, v_h, ql_h = x["k"].cpu(), x["v"].cpu(), x["q_land"].cpu()
    oks, obs = oracle.summarize(k_h, ql_h, S, Hq, ks_round=oracle.ks_round_for("bf16"))
    assert_close(b_sum.cpu(), obs, 1e-5, what="b'")
    assert_close(k_sum.cpu(), oks, 2e-2, 5e-3, what="k'")
    q_rows = x["q"][:, :, pos].cpu()
    qh_rows = x["q_hat"][:, :, pos].cpu()
    rb, rg, rq = rows_layout(B, Hkv, range(len(pos)))
    ri = np.asarray(pos, np.int64)[rq]
    orc = oracle.rows(rb, rg, ri, rq, q_rows, qh_rows, k_h, v_h, oks, obs, S=S, W=W, topk=k,
                      want_r=True)
    gi = gather_rows(idx, rb, rg, ri, 1)[:, 0].astype(np.int64)
    res = check_selection(gi, orc, k, TAU_E2E_BF16)
    say("  decided %d undecided %d differ %d" % (res["decided"], res["undecided"], res["differ"].sum()))
    assert res["decided"] > 0
    want_out, want_lse = orc["out"].copy(), orc["lse"].copy()
    dm = res["differ"]
    if dm.any():
        alt = oracle.rows(rb[dm], rg[dm], ri[dm], rq[dm], q_rows, qh_rows, k_h, v_h, oks, obs, S=S,
                          W=W, topk=k, forced_idx=gi[dm])
        want_out[dm], want_lse[dm] = alt["out"], alt["lse"]
    t = tol_out(torch.bfloat16)
    assert_close(gather_rows(out, rb, rg, ri, G), want_out, t["max_abs"], t["rel_l2"], what="out")
    assert_close(gather_rows(lse, rb, rg, ri, G), want_lse, tol_lse(torch.bfloat16), what="lse")
    del x, k_sum, b_sum, idx, ssel, out, lse
    _free()


def test_decode_512k_sampled(hils):
    """Four 512K-token sequences, through a chunk completion (step 63)."""
    wl = wk.CONFIGS["512k_decode"]
    _decode_run(hils, wl, seed=1, nsteps=65, check_steps={0, 1, 63, 64})


def test_decode_4m_needles(hils):
    """One 4M-token sequence with 8 planted needle chunks: each step selects all of
    them in every group, and sampled steps match the oracle."""
    wl = wk.CONFIGS["4m_decode"]
    hist, meta = _decode_run(hils, wl, seed=2, nsteps=65, check_steps={0, 64}, needles=True)
    needles = set(int(c) for c in meta["needle_chunks"])
    for st, gi in enumerate(hist):
        for row in gi:
            assert needles <= set(row.tolist()), ("needle missed", st, sorted(needles - set(row.tolist())))
