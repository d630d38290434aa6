"""hils_decode_step_noalloc (the decode step on the library's built-in scratch)
against hils_decode_step (caller workspace), through the C ABI.

Both entry points run the same kernels, so every output must be bitwise equal:
out, lse, the selected ids, the appended cache rows and the summaries of the
chunks the steps complete.  Two calls in a row, the second with a smaller
input, check that the shared scratch needs no clearing between calls.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as wk

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


def _state(hils, wl, start, cap, seed):
    """Caches of `start` tokens and the summaries of their complete chunks."""
    base = wk.make_decode_cache(wl, seed=seed, length=start, capacity=cap)
    kc, vc, ql = base["k_cache"].to(DEV), base["v_cache"].to(DEV), base["q_land"].to(DEV)
    NCcap = cap // wl.S
    ks = torch.zeros((wl.B, wl.Hq, NCcap, wl.d), dtype=wl.torch_dtype, device=DEV)
    bs = torch.zeros((wl.B, wl.Hq, NCcap), dtype=torch.float32, device=DEV)
    shape = hils.Shape.make(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, cap, wl.torch_dtype)
    if start // wl.S:
        hils.hils_summarize(kc, ql, ks, bs, shape, 0, start // wl.S)
    return {"kc": kc, "vc": vc, "ks": ks, "bs": bs, "shape": shape}


def _run(hils, wl, start, cap, nsteps, seed):
    a = _state(hils, wl, start, cap, seed)
    b = {k_: (v_.clone() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in a.items()}
    shape = a["shape"]
    ws = hils.workspace(shape, hils.OP_DECODE, DEV)
    outs = []
    for st in range(nsteps):
        x = {n_: v_.to(DEV) for n_, v_ in wk.make_decode_step(wl, st, seed=seed).items()}
        pos = [start + st] * wl.B
        res = []
        for s_, fn in ((a, "ws"), (b, "noalloc")):
            out = torch.empty((wl.B, wl.Hq, wl.d), dtype=wl.torch_dtype, device=DEV)
            lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=DEV)
            idx = torch.empty((wl.B, wl.Hkv, wl.k), dtype=torch.int32, device=DEV)
            args = (pos, x["q"], x["q_hat"], x["k_new"], x["v_new"], x["q_land_new"], s_["kc"],
                    s_["vc"], s_["ks"], s_["bs"], out, lse, idx, shape)
            if fn == "ws":
                hils.hils_decode_step(*args, ws)
            else:
                hils.hils_decode_step_noalloc(*args)
            res.append((out, lse, idx))
        torch.cuda.synchronize()
        for t0, t1 in zip(res[0], res[1]):
            assert torch.equal(t0, t1), ("step", st)
        outs.append(res[1][0].float().abs().mean().item())
    for key in ("kc", "vc", "ks", "bs"):
        assert torch.equal(a[key], b[key]), key
    return outs


def test_noalloc_matches_workspace_entry_point(hils):
    big = wk.custom(name="na1", kind="decode", dtype="bf16", B=3, Hq=8, Hkv=2, d=128, T=3000,
                    S=64, k=8, W=256)
    say("noalloc: B=3, 3000 tokens, 80 steps (one chunk completion)")
    o1 = _run(hils, big, 3000, 3136, 80, seed=21)
    small = wk.custom(name="na2", kind="decode", dtype="bf16", B=1, Hq=4, Hkv=1, d=64, T=700,
                      S=64, k=3, W=128)
    say("noalloc: then B=1, 700 tokens, 30 steps (one chunk completion)")
    o2 = _run(hils, small, 700, 768, 30, seed=22)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(o2))


def test_noalloc_rejects_a_shape_beyond_its_scratch(hils):
    import ctypes
    L = hils.lib()
    s = hils.Shape.make(64, 32, 8, 128, 64, 1024, 64, 1 << 22, torch.bfloat16)
    assert hils.hils_workspace_bytes(s, hils.OP_DECODE) > (64 << 20)
    pos = (ctypes.c_int64 * 64)(*([5] * 64))
    P = ctypes.c_void_p
    assert L.hils_decode_step_noalloc(ctypes.byref(s), pos, *[P(256)] * 12, None) == -10
