"""Seeded synthetic inputs for the HiLS-Attention forward path.

This module only draws random numbers and places them in memory.  It holds
none of the method's arithmetic: no logits, softmax, summaries, selection or
fusion.  Both the GPU path and the fp64 oracle consume the bytes it produces.

Layout (all tensors head-major and contiguous):
    q, q_hat   [B, Hq,  T, d]   io dtype
    k, v       [B, Hkv, T, d]   io dtype
    q_land     [B, Hq, NC, d]   io dtype, one landmark query per complete chunk
Values are N(0,1) * d**-0.25, rounded to the io dtype (round-to-nearest-even).

Small workloads are drawn on the host with numpy's PCG64 (stable across
machines).  The large ones (the 128K prefill and the decode caches) are drawn
on the device with torch's seeded CUDA generator, since moving gigabytes over
PCIe would dominate the run; the oracle then reads back the exact device
bytes it needs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import numpy as np
import torch

__all__ = [
    "Workload", "CONFIGS", "prefill_config", "decode_config",
    "make_prefill", "make_decode_cache", "make_decode_step", "make_dyadic_select",
]


@dataclass
class Workload:
    """Shape of one workload (prefill: seq_len = T; decode: initial cache length)."""
    name: str
    kind: str              # "prefill" | "decode"
    dtype: str             # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int                 # prefill tokens, or decode initial cache length L
    S: int                 # chunk size
    k: int                 # top-k
    W: int                 # window
    steps: int = 0         # decode steps
    needles: int = 0       # planted needle chunks
    head_scale: tuple | None = None   # per-head scale range U[lo, hi]
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def NC(self) -> int:
        return self.T // self.S

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def as_dict(self) -> dict:
        return asdict(self)


# The five workloads: shapes, value distributions and structure as stated for
# the path's published configurations (tiny fp32, 8K with a needle, 128K with
# per-head scales, 512K decode over 4 sequences, 4M decode with 8 needles).
CONFIGS = {
    "tiny": Workload("tiny", "prefill", "f32", 1, 1, 1, 64, 1024, 64, 4, 64),
    "8k": Workload("8k", "prefill", "bf16", 1, 32, 8, 128, 8192, 64, 16, 512, needles=1),
    "128k": Workload("128k", "prefill", "bf16", 1, 32, 8, 128, 131072, 64, 32, 1024,
                     head_scale=(0.5, 2.0)),
    "512k_decode": Workload("512k_decode", "decode", "bf16", 4, 32, 8, 128, 524288, 64, 32, 1024,
                            steps=256),
    "4m_decode": Workload("4m_decode", "decode", "bf16", 1, 32, 8, 128, 4194304, 64, 64, 1024,
                          steps=256, needles=8),
}

# Needle strengths: key = BETA*u, landmark query = GAMMA*u, retrieval/attention
# query = ALPHA*u (u a random unit vector).  With d = 128 the needle chunk's
# retrieval score then sits about 1.2 above the haystack's.
NEEDLE_ALPHA = 8.0
NEEDLE_BETA = 8.0
NEEDLE_GAMMA = 8.0
# A decode query spreads ALPHA_DECODE over n needles (ALPHA_DECODE/sqrt(n) each,
# along mutually orthogonal directions), so it needs a larger total: with 8
# needles this places every needle chunk's rank key well above the haystack.
NEEDLE_ALPHA_DECODE = 32.0


def prefill_config(name: str) -> Workload:
    return CONFIGS[name]


def decode_config(name: str) -> Workload:
    return CONFIGS[name]


def custom(**kw) -> Workload:
    """A workload of arbitrary (small) shape for tests."""
    base = dict(name="custom", kind="prefill", dtype="f32", B=1, Hq=1, Hkv=1, d=64, T=256,
                S=64, k=4, W=64)
    base.update(kw)
    return Workload(**base)


def _np_normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float64) * scale).astype(np.float32)


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return u / np.linalg.norm(u)


def _to_dtype(x: np.ndarray, wl: Workload, device) -> torch.Tensor:
    # float32 -> bf16 in torch rounds to nearest even.
    return torch.from_numpy(np.ascontiguousarray(x)).to(wl.torch_dtype).to(device)


def make_prefill(wl: Workload | str, seed: int = 0, device="cpu") -> dict:
    """Inputs of one prefill forward: q, k, v, q_land, q_hat (+ needle metadata).

    Host generation (numpy PCG64) for everything but the 128K-scale workloads on
    a CUDA device, which are drawn on the device (torch CUDA generator).
    """
    if isinstance(wl, str):
        wl = CONFIGS[wl]
    dev = torch.device(device)
    big = wl.B * wl.Hq * wl.T * wl.d > (1 << 27)
    if dev.type == "cuda" and big:
        return _make_prefill_device(wl, seed, dev)
    rng = np.random.Generator(np.random.PCG64(seed))
    sc = wl.d ** -0.25
    B, Hq, Hkv, T, d, NC = wl.B, wl.Hq, wl.Hkv, wl.T, wl.d, wl.NC
    k = _np_normal(rng, (B, Hkv, T, d), sc)
    v = _np_normal(rng, (B, Hkv, T, d), sc)
    q = _np_normal(rng, (B, Hq, T, d), sc)
    ql = _np_normal(rng, (B, Hq, NC, d), sc)
    qh = _np_normal(rng, (B, Hq, T, d), sc)
    meta = {}
    if wl.head_scale is not None:
        lo, hi = wl.head_scale
        sq = rng.uniform(lo, hi, size=Hq).astype(np.float32)
        skv = rng.uniform(lo, hi, size=Hkv).astype(np.float32)
        q *= sq[None, :, None, None]
        ql *= sq[None, :, None, None]
        qh *= sq[None, :, None, None]
        k *= skv[None, :, None, None]
        v *= skv[None, :, None, None]
        meta["scale_q"], meta["scale_kv"] = sq, skv
    if wl.needles:
        # One needle: a key in chunk c* = 1 of KV head 0, the landmark query of
        # that chunk and the last query of every head of group 0 aligned to it.
        G = Hq // Hkv
        u = _unit(rng, d).astype(np.float32)
        c_star = 1
        j_star = c_star * wl.S + int(rng.integers(0, wl.S))
        i_star = T - 1
        k[0, 0, j_star, :] = NEEDLE_BETA * u
        for h in range(G):
            ql[0, h, c_star, :] = NEEDLE_GAMMA * u
            q[0, h, i_star, :] = NEEDLE_ALPHA * u
            qh[0, h, i_star, :] = NEEDLE_ALPHA * u
        meta.update(needle_chunk=c_star, needle_token=j_star, needle_query=i_star, needle_group=0)
    out = {n: _to_dtype(a, wl, dev) for n, a in (("q", q), ("k", k), ("v", v), ("q_land", ql),
                                                 ("q_hat", qh))}
    out["meta"] = meta
    out["wl"] = wl
    return out


def _dev_normal(gen, shape, scale, dtype, dev) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32, device=dev)
    t.normal_(0.0, 1.0, generator=gen)
    t.mul_(scale)
    return t.to(dtype)


def _make_prefill_device(wl: Workload, seed: int, dev) -> dict:
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    sc = wl.d ** -0.25
    B, Hq, Hkv, T, d, NC = wl.B, wl.Hq, wl.Hkv, wl.T, wl.d, wl.NC
    dt = wl.torch_dtype
    k = _dev_normal(gen, (B, Hkv, T, d), sc, torch.float32, dev)
    v = _dev_normal(gen, (B, Hkv, T, d), sc, torch.float32, dev)
    q = _dev_normal(gen, (B, Hq, T, d), sc, torch.float32, dev)
    ql = _dev_normal(gen, (B, Hq, NC, d), sc, torch.float32, dev)
    qh = _dev_normal(gen, (B, Hq, T, d), sc, torch.float32, dev)
    meta = {}
    if wl.head_scale is not None:
        lo, hi = wl.head_scale
        sq = torch.empty(Hq, device=dev).uniform_(lo, hi, generator=gen)
        skv = torch.empty(Hkv, device=dev).uniform_(lo, hi, generator=gen)
        for t in (q, ql, qh):
            t.mul_(sq[None, :, None, None])
        for t in (k, v):
            t.mul_(skv[None, :, None, None])
        meta["scale_q"], meta["scale_kv"] = sq.cpu().numpy(), skv.cpu().numpy()
    out = {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "q_land": ql.to(dt), "q_hat": qh.to(dt)}
    del q, k, v, ql, qh
    out["meta"] = meta
    out["wl"] = wl
    return out


def decode_capacity(wl: Workload) -> int:
    """Cache rows per head: initial length plus the decode steps, chunk-rounded."""
    n = wl.T + wl.steps
    return -(-n // wl.S) * wl.S


def make_decode_cache(wl: Workload | str, seed: int = 0, device="cpu", length: int | None = None,
                      capacity: int | None = None) -> dict:
    """KV cache of `length` tokens (default: the workload's L) and landmark queries.

    k_cache, v_cache [B, Hkv, Lcap, d]; q_land [B, Hq, Lcap/S, d].  Rows at and
    beyond `length` are zero.  Needle chunks (if any) are planted at seeded
    depths, uniform without replacement over chunks left of the final window.
    """
    if isinstance(wl, str):
        wl = CONFIGS[wl]
    L = wl.T if length is None else length
    cap = decode_capacity(wl) if capacity is None else capacity
    dev = torch.device(device)
    B, Hq, Hkv, d, S = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S
    G = Hq // Hkv
    sc = d ** -0.25
    dt = wl.torch_dtype
    ncap = cap // S
    meta = {}
    if dev.type == "cuda":
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        kc = torch.zeros((B, Hkv, cap, d), dtype=dt, device=dev)
        vc = torch.zeros((B, Hkv, cap, d), dtype=dt, device=dev)
        # draw per (b, head) slices to bound the fp32 temporary
        for b in range(B):
            for g in range(Hkv):
                kc[b, g, :L] = _dev_normal(gen, (L, d), sc, dt, dev)
                vc[b, g, :L] = _dev_normal(gen, (L, d), sc, dt, dev)
        ql = _dev_normal(gen, (B, Hq, ncap, d), sc, dt, dev)
    else:
        rng = np.random.Generator(np.random.PCG64(seed))
        k = np.zeros((B, Hkv, cap, d), np.float32)
        v = np.zeros((B, Hkv, cap, d), np.float32)
        k[:, :, :L] = _np_normal(rng, (B, Hkv, L, d), sc)
        v[:, :, :L] = _np_normal(rng, (B, Hkv, L, d), sc)
        kc, vc = _to_dtype(k, wl, dev), _to_dtype(v, wl, dev)
        ql = _to_dtype(_np_normal(rng, (B, Hq, ncap, d), sc), wl, dev)
    if wl.needles:
        rng = np.random.Generator(np.random.PCG64(seed + 7919))
        n_far = max(1, (L - wl.W) // S - 1)
        chunks = np.sort(rng.choice(n_far, size=wl.needles, replace=False))
        u = np.stack([[_unit(rng, d) for _ in range(Hkv)] for _ in range(wl.needles)])  # [n, Hkv, d]
        for g in range(Hkv):      # orthonormal needle directions within each KV head
            qm, _ = np.linalg.qr(u[:, g, :].T)
            u[:, g, :] = qm.T[:wl.needles]
        toks = chunks * S + rng.integers(0, S, size=wl.needles)
        for n in range(wl.needles):
            for b in range(B):
                for g in range(Hkv):
                    kc[b, g, int(toks[n])] = torch.from_numpy(NEEDLE_BETA * u[n, g]).to(dt).to(dev)
                    for h in range(g * G, (g + 1) * G):
                        ql[b, h, int(chunks[n])] = torch.from_numpy(NEEDLE_GAMMA * u[n, g]).to(dt).to(dev)
        meta.update(needle_chunks=chunks, needle_tokens=toks, needle_dirs=u.astype(np.float32))
    return {"k_cache": kc, "v_cache": vc, "q_land": ql, "length": L, "capacity": cap,
            "meta": meta, "wl": wl}


def make_decode_step(wl: Workload | str, step: int, seed: int = 0, device="cpu",
                     needle_dirs: np.ndarray | None = None) -> dict:
    """Per-step inputs: q, q_hat [B, Hq, d], k_new, v_new [B, Hkv, d], q_land_new [B, Hq, d].

    With needles, q = q_hat = ALPHA_DECODE * sum_n u_n / sqrt(n) + Gaussian noise.
    """
    if isinstance(wl, str):
        wl = CONFIGS[wl]
    rng = np.random.Generator(np.random.PCG64([seed, 1_000_003 + step]))
    B, Hq, Hkv, d = wl.B, wl.Hq, wl.Hkv, wl.d
    G = Hq // Hkv
    sc = d ** -0.25
    q = _np_normal(rng, (B, Hq, d), sc)
    qh = _np_normal(rng, (B, Hq, d), sc)
    kn = _np_normal(rng, (B, Hkv, d), sc)
    vn = _np_normal(rng, (B, Hkv, d), sc)
    qln = _np_normal(rng, (B, Hq, d), sc)
    if needle_dirs is not None:
        nn = needle_dirs.shape[0]
        for h in range(Hq):
            dirn = NEEDLE_ALPHA_DECODE * needle_dirs[:, h // G, :].sum(0) / math.sqrt(nn)
            q[:, h, :] += dirn
            qh[:, h, :] = q[:, h, :]
    dev = torch.device(device)
    return {n: _to_dtype(a, wl, dev) for n, a in (("q", q), ("q_hat", qh), ("k_new", kn),
                                                 ("v_new", vn), ("q_land_new", qln))}


def make_dyadic_select(B=1, Hq=4, Hkv=1, T=512, d=64, S=16, k=8, W=32, seed=0,
                       identical_heads=True, plant_ties=True) -> dict:
    """Inputs whose retrieval scores are exact in fp32 (and fp64).

    q_hat and k' are small integers times 2**-4 and 2**-3 and b' is a multiple
    of 2**-6, with scale = 2**-3: every product and partial sum is a dyadic
    rational with few significant bits, so any summation order gives the same
    fp32 value.  Exact ties are planted by copying chunk summaries; with
    identical heads in a group the GQA key is the same for every head.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    G = Hq // Hkv
    NC = T // S
    qh = rng.integers(-3, 4, size=(B, Hq, T, d)).astype(np.float32) * 2.0 ** -4
    ks = rng.integers(-3, 4, size=(B, Hq, NC, d)).astype(np.float32) * 2.0 ** -3
    bs = rng.integers(0, 8, size=(B, Hq, NC)).astype(np.float32) * 2.0 ** -6
    if identical_heads:
        for g in range(Hkv):
            for h in range(g * G + 1, (g + 1) * G):
                qh[:, h] = qh[:, g * G]
                ks[:, h] = ks[:, g * G]
                bs[:, h] = bs[:, g * G]
    if plant_ties:
        # every third chunk duplicates its predecessor's summary exactly
        for c in range(1, NC, 3):
            ks[:, :, c] = ks[:, :, c - 1]
            bs[:, :, c] = bs[:, :, c - 1]
    return {"q_hat": torch.from_numpy(qh), "k_sum": torch.from_numpy(ks),
            "b_sum": torch.from_numpy(bs), "scale": 2.0 ** -3,
            "wl": custom(B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, S=S, k=k, W=W)}


def make_qcal(wl: Workload, d_model: int, rank: int, seed: int = 0, device="cpu") -> dict:
    """Hidden states and low-rank calibration weights for q_hat = q + W_up W_down h.

    h ~ N(0,1) [B, T, d_model]; W_down ~ N(0,1)/sqrt(d_model) [rank, d_model] (so
    W_down h has unit-variance entries); W_up ~ N(0,1) d^-1/4 / sqrt(rank)
    [Hq, d, rank] (so the correction has the spread of q itself).  Random weights
    stand in for trained ones.  Host numpy PCG64 (seed) for sizes up to 2^27
    elements of h, else the device generator.
    """
    B, T, Hq, d = wl.B, wl.T, wl.Hq, wl.d
    if B * T * d_model <= (1 << 27):
        rng = np.random.Generator(np.random.PCG64(seed + 7919))
        h = _np_normal(rng, (B, T, d_model), 1.0)
        wd = _np_normal(rng, (rank, d_model), d_model ** -0.5)
        wu = _np_normal(rng, (Hq, d, rank), d ** -0.25 * rank ** -0.5)
        return {n: _to_dtype(a, wl, torch.device(device)) for n, a in (("h", h), ("w_down", wd), ("w_up", wu))}
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 7919)
    dt = wl.torch_dtype
    return {"h": _dev_normal(gen, (B, T, d_model), 1.0, torch.float32, dev).to(dt),
            "w_down": _dev_normal(gen, (rank, d_model), d_model ** -0.5, torch.float32, dev).to(dt),
            "w_up": _dev_normal(gen, (Hq, d, rank), d ** -0.25 * rank ** -0.5, torch.float32, dev).to(dt)}
