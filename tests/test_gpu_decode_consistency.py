"""Decode against prefill on the same bytes, and decode resumed from a snapshot.

* A decode step at position i computes the prefill row i of the same
  definitions (summary page, Summary: constant-cost decoding over the summaries
  of completed chunks).  Stepping a sequence through positions t0..T-1 with the
  prefill's own q, q_hat, k, v and landmark queries must give the prefill's
  selections (equal wherever the oracle's rank-key gap at the k-th place is at
  least the tie band), its outputs and LSE within the output tolerance, and,
  since both paths summarise with the same arithmetic, bit-identical summaries
  of the chunks completed along the way.
* Decode state is exactly the caches and the summaries: copying them to the
  host after 128 steps, restoring the copies into fresh device buffers and
  replaying the next steps must reproduce every output bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from hils_testlib import TAU_E2E_BF16, assert_close, tol_lse, tol_out

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


WL = wk.custom(name="dc", dtype="bf16", B=2, Hq=8, Hkv=2, d=128, T=1200, S=64, k=6, W=256)


class Stepper:
    """Decode state for the sequences of one prefill input, cache rows past the
    written length poisoned with NaN."""

    def __init__(self, hils, wl, x, t0):
        self.h, self.wl, self.x = hils, wl, x
        B, Hq, Hkv, d, S = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S
        self.cap = -(-wl.T // S) * S + S
        dt = wl.torch_dtype
        self.kc = torch.full((B, Hkv, self.cap, d), float("nan"), dtype=dt, device=DEV)
        self.vc = torch.full_like(self.kc, float("nan"))
        self.kc[:, :, :t0] = x["k"][:, :, :t0].to(DEV)
        self.vc[:, :, :t0] = x["v"][:, :, :t0].to(DEV)
        NCcap = self.cap // S
        self.ks = torch.zeros((B, Hq, NCcap, d), dtype=dt, device=DEV)
        self.bs = torch.zeros((B, Hq, NCcap), dtype=torch.float32, device=DEV)
        self.shape = hils.Shape.make(B, Hq, Hkv, d, S, wl.W, wl.k, self.cap, dt)
        if t0 // S:
            ql = torch.zeros((B, Hq, NCcap, d), dtype=dt, device=DEV)
            ql[:, :, :wl.NC] = x["q_land"].to(DEV)
            hils.hils_summarize(self.kc, ql, self.ks, self.bs, self.shape, 0, t0 // S)
        self.ws = hils.workspace(self.shape, hils.OP_DECODE, DEV)
        self.out = torch.empty((B, Hq, d), dtype=dt, device=DEV)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((B, Hkv, wl.k), dtype=torch.int32, device=DEV)
        self.zero_ql = torch.zeros((B, Hq, d), dtype=dt, device=DEV)

    def step(self, t):
        x, S = self.x, self.wl.S
        c = t // S
        qln = x["q_land"][:, :, c].contiguous().to(DEV) if (t + 1) % S == 0 else self.zero_ql
        self.h.hils_decode_step([t] * self.wl.B, x["q"][:, :, t].contiguous().to(DEV),
                                x["q_hat"][:, :, t].contiguous().to(DEV),
                                x["k"][:, :, t].contiguous().to(DEV), x["v"][:, :, t].contiguous().to(DEV),
                                qln, self.kc, self.vc, self.ks, self.bs, self.out, self.lse, self.idx,
                                self.shape, self.ws)
        torch.cuda.synchronize()
        return self.out.clone(), self.lse.clone(), self.idx.clone()


def test_decode_row_equals_prefill_row(hils):
    wl = WL
    say("decode rows against prefill rows")
    x = wk.make_prefill(wl, seed=41)
    xd = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    pre = hils.prefill(xd["q"], xd["k"], xd["v"], xd["q_land"], xd["q_hat"], S=wl.S, W=wl.W, topk=wl.k)
    torch.cuda.synchronize()
    t0 = 900
    st = Stepper(hils, wl, x, t0)
    outs, lses, idxs = [], [], []
    for t in range(t0, wl.T):
        o, l_, i_ = st.step(t)
        outs.append(o)
        lses.append(l_)
        idxs.append(i_)
    # summaries of every complete chunk, those completed by the steps included
    NC = wl.NC
    assert torch.equal(st.ks[:, :, :NC], pre["k_sum"]), "k' differs from the prefill's"
    assert torch.equal(st.bs[:, :, :NC], pre["b_sum"]), "b' differs from the prefill's"
    dec_idx = torch.stack(idxs, 2).cpu().numpy()                 # [B, Hkv, T - t0, k]
    pre_idx = pre["idx"][:, :, t0:].cpu().numpy()
    dec_out = torch.stack(outs, 2)                               # [B, Hq, T - t0, d]
    dec_lse = torch.stack(lses, 2)
    # where the two selections differ, the event must be undecided: the oracle's
    # gap between the k-th and (k+1)-th rank key below the tie band
    differ = np.any(dec_idx != pre_idx, axis=-1)                 # [B, Hkv, T - t0]
    G = wl.Hq // wl.Hkv
    if differ.any():
        rb, rg, rt = np.nonzero(differ)
        ri = rt + t0
        oks, obs = oracle.summarize(x["k"], x["q_land"], wl.S, wl.Hq, ks_round=oracle.ks_round_for(wl.dtype))
        orc = oracle.rows(rb, rg, ri, ri, x["q"], x["q_hat"], x["k"], x["v"], oks, obs, S=wl.S, W=wl.W,
                          topk=wl.k, want_r=True)
        assert np.all(orc["ncand"] > wl.k)
        assert np.all(orc["gap"] < TAU_E2E_BF16), float(orc["gap"].max())
    say("    rows %d, selections differing (undecided) %d" % (differ.size, int(differ.sum())))
    same = np.repeat(~differ, G, axis=1)                         # [B, Hq, T - t0]
    po = pre["out"][:, :, t0:].cpu().to(torch.float64).numpy()[same]
    do = dec_out.cpu().to(torch.float64).numpy()[same]
    t = tol_out(wl.torch_dtype)
    assert_close(do, po, t["max_abs"], t["rel_l2"], what="decode out vs prefill out")
    pl = pre["lse"][:, :, t0:].cpu().to(torch.float64).numpy()[same]
    dl = dec_lse.cpu().to(torch.float64).numpy()[same]
    assert_close(dl, pl, tol_lse(wl.torch_dtype), what="decode lse vs prefill lse")


def test_decode_resumes_from_snapshot_bit_for_bit(hils):
    wl = WL
    say("decode snapshot and resume")
    x = wk.make_prefill(wl, seed=42)
    t0, n_snap, n_more = 850, 128, 112         # the resumed steps complete chunks 15 and 16
    a = Stepper(hils, wl, x, t0)
    for t in range(t0, t0 + n_snap):
        a.step(t)
    snap = {n: getattr(a, n).cpu().clone() for n in ("kc", "vc", "ks", "bs")}
    ref = [a.step(t) for t in range(t0 + n_snap, t0 + n_snap + n_more)]
    b = Stepper(hils, wl, x, 0)                 # fresh buffers, state restored from the snapshot
    for n, v_ in snap.items():
        getattr(b, n).copy_(v_.to(DEV))
    for j, t in enumerate(range(t0 + n_snap, t0 + n_snap + n_more)):
        o, l_, i_ = b.step(t)
        assert torch.equal(i_, ref[j][2]), "selection differs at step %d" % t
        assert torch.equal(o, ref[j][0]) and torch.equal(l_, ref[j][1]), "output differs at step %d" % t
    for n in ("kc", "vc", "ks", "bs"):   # as bytes: NaN rows past the written length compare equal
        assert torch.equal(_bits(getattr(a, n)), _bits(getattr(b, n))), n


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)
