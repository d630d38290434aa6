"""GPU parity of the backward calls against the fp64 oracle's prefill_backward.

The GPU runs its own forward (summaries, selection, attention), then
hils_attend_fuse_backward and hils_summarize_backward.  The oracle takes the
GPU's selection as the one held fixed and the GPU's stored summaries as the
forward's k', b' (both are inputs of the backward, not results under test), and
the same input and upstream-gradient bytes.

Tolerances, from the arithmetic: fp32 runs every product in fp32 (errors of a
few ulp per term, sums of at most a few thousand terms), so 2e-5 relative.  In
bf16 the kernels round the attention weights alpha and the logit gradients ds to
bf16 before the matrix products (unit roundoff 2^-9 ~ 2e-3 per term, random in
sign), and D = dout . out uses the forward's bf16 out: each gradient's rel-L2
error is then about 2e-3, and the bound is 1e-2 (max-abs 5e-2 of the largest
magnitude).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from hils_testlib import f64

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


CASES = {
    "tiny": wk.CONFIGS["tiny"],
    "f32_g2_d128_ragged": wk.custom(name="b2", dtype="f32", B=1, Hq=4, Hkv=2, d=128, T=900, S=64,
                                    k=3, W=64),
    "bf16_g4_d128": wk.custom(name="b4", dtype="bf16", B=1, Hq=8, Hkv=2, d=128, T=1600, S=64, k=6,
                              W=128),
    "bf16_g8_d64_ragged": wk.custom(name="b8", dtype="bf16", B=2, Hq=8, Hkv=1, d=64, T=1317, S=64,
                                    k=5, W=100),
    "bf16_g1_d64": wk.custom(name="b1", dtype="bf16", B=1, Hq=2, Hkv=2, d=64, T=1000, S=64, k=4,
                             W=64),
    "bf16_k0": wk.custom(name="bk0", dtype="bf16", B=1, Hq=4, Hkv=1, d=128, T=700, S=64, k=0,
                         W=128),
    "f32_no_chunk": wk.custom(name="bnc", dtype="f32", B=1, Hq=2, Hkv=1, d=64, T=37, S=64, k=3,
                              W=64),
    "bf16_no_candidate": wk.custom(name="bnc2", dtype="bf16", B=1, Hq=4, Hkv=2, d=64, T=150, S=64,
                                   k=3, W=128),
}


def tol(dtype):
    if dtype == torch.bfloat16:
        return {"rel_l2": 1e-2, "max_rel": 5e-2}
    return {"rel_l2": 2e-5, "max_rel": 2e-5}


def grad_close(got, want, t, what):
    got, want = f64(got), f64(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    if want.size == 0:
        return 0.0, 0.0
    scale = max(float(np.abs(want).max()), 1e-30)
    err = np.abs(got - want)
    mr = float(err.max()) / scale
    nw = float(np.linalg.norm(want))
    rl = float(np.linalg.norm(got - want)) / nw if nw > 0 else float(np.linalg.norm(got))
    say("    %-8s rel-L2 %.3g  max-abs/max %.3g" % (what, rl, mr))
    if nw == 0:
        assert float(err.max()) <= 1e-6, (what, float(err.max()))
        return rl, mr
    assert mr <= t["max_rel"], "%s: max-abs %.3g of the largest magnitude > %.3g" % (what, mr, t["max_rel"])
    assert rl <= t["rel_l2"], "%s: rel-L2 %.3g > %.3g" % (what, rl, t["rel_l2"])
    return rl, mr


def run_gpu(hils, wl, xd, dout_d, dlse_d, ws_bytes=None):
    B, Hq, Hkv, T, d = wl.B, wl.Hq, wl.Hkv, wl.T, wl.d
    NC = T // wl.S
    r = hils.prefill(xd["q"], xd["k"], xd["v"], xd["q_land"], xd["q_hat"], S=wl.S, W=wl.W, topk=wl.k)
    sh = r["shape"]
    f = dict(dtype=torch.float32, device=DEV)
    g = {"dq": torch.full((B, Hq, T, d), float("nan"), **f),
         "dq_hat": torch.full((B, Hq, T, d), float("nan"), **f),
         "dk": torch.full((B, Hkv, T, d), float("nan"), **f),
         "dv": torch.full((B, Hkv, T, d), float("nan"), **f),
         "dk_sum": torch.full((B, Hq, NC, d), float("nan"), **f),
         "db_sum": torch.full((B, Hq, NC), float("nan"), **f),
         "dq_land": torch.full((B, Hq, NC, d), float("nan"), **f)}
    full = hils.hils_workspace_bytes(sh, hils.OP_ATTEND_BACKWARD)
    ws = torch.empty(max(full if ws_bytes is None else ws_bytes, 1), dtype=torch.uint8, device=DEV)
    hils.hils_attend_fuse_backward(xd["q"], xd["k"], xd["v"], xd["q_hat"], r["k_sum"], r["idx"],
                                   r["ssel"], r["out"], r["lse"], dout_d, dlse_d, g["dq"], g["dk"],
                                   g["dv"], g["dq_hat"], g["dk_sum"], g["db_sum"], sh, ws)
    if NC > 0:
        hils.hils_summarize_backward(xd["k"], xd["q_land"], g["dk_sum"], g["db_sum"], g["dk"],
                                     g["dq_land"], sh)
    torch.cuda.synchronize()
    return r, g, full


def _data(wl, seed):
    x = wk.make_prefill(wl, seed=seed)
    xd = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    gen = torch.Generator().manual_seed(seed + 1000)
    dout = (torch.randn((wl.B, wl.Hq, wl.T, wl.d), generator=gen) * 0.5).to(wl.torch_dtype)
    dlse = torch.randn((wl.B, wl.Hq, wl.T), generator=gen) * 0.5
    return x, xd, dout, dlse


def check_against_oracle(hils, wl, with_dlse=True, seed=5):
    x, xd, dout, dlse = _data(wl, seed)
    r, g, _ = run_gpu(hils, wl, xd, dout.to(DEV), dlse.to(DEV) if with_dlse else None)
    sel = r["idx"].cpu().numpy() if wl.k > 0 else np.zeros((wl.B, wl.Hkv, wl.T, 0), np.int32)
    NC = wl.T // wl.S
    ks = f64(r["k_sum"]) if NC else np.zeros((wl.B, wl.Hq, 0, wl.d))
    bs = f64(r["b_sum"]) if NC else np.zeros((wl.B, wl.Hq, 0))
    want = oracle.prefill_backward(x, sel, f64(dout), f64(dlse) if with_dlse else None, S=wl.S,
                                   W=wl.W, topk=wl.k, ksum=ks, bsum=bs)
    t = tol(wl.torch_dtype)
    for n in ("dq", "dq_hat", "dk", "dv", "dk_sum", "db_sum", "dq_land"):
        grad_close(g[n], want[n], t, n)
    return r, g


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(hils, name):
    wl = CASES[name]
    say("backward", name)
    check_against_oracle(hils, wl)


def test_backward_without_dlse(hils):
    wl = CASES["bf16_g4_d128"]
    say("backward, dlse NULL")
    check_against_oracle(hils, wl, with_dlse=False, seed=8)


def test_backward_passes_and_determinism(hils):
    """A workspace with room for fewer KV heads' dq parts runs in passes; the
    result is bitwise the same as in one pass, and as a second run."""
    wl = CASES["bf16_g4_d128"]
    say("backward in passes")
    x, xd, dout, dlse = _data(wl, 9)
    _, g1, full = run_gpu(hils, wl, xd, dout.to(DEV), dlse.to(DEV))
    _, g2, _ = run_gpu(hils, wl, xd, dout.to(DEV), dlse.to(DEV), ws_bytes=full - 512)
    _, g3, _ = run_gpu(hils, wl, xd, dout.to(DEV), dlse.to(DEV))
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
        assert torch.equal(g1[n], g3[n]), n


def test_backward_8k(hils):
    """The 8K configuration at full size (bf16, 32 / 8 heads, d 128, k 16, W 512)."""
    wl = wk.CONFIGS["8k"]
    say("backward 8K")
    check_against_oracle(hils, wl, seed=3)
