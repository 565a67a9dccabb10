"""Seeded synthetic inputs for Falcon fast-weight attention.

This module is shared by the oracle-side tests, the GPU parity tests, ``smoke()``
and ``bench.py``.  It draws random numbers and shapes them; it holds none of the
method's arithmetic (no feature map, no clamp, no step normalisation, no state
update).  Everything it returns is a float32/float64 NumPy array.

Workloads stand in for activations of the 124-130M-parameter language models the
Falcon pages train on FineWeb-Edu (d_model 768 = 12 heads x 64): the pages'
dataset is not used, the inputs are N(0,1) draws of the same layer shape.

Generation order (NumPy PCG64 ``default_rng(seed)``, float32, C order):
q [B,T,H,dk], k, v [B,T,H,dv], beta-logits [B,T,H] (or [B,T,H,dv] for the
per-channel variants), lambda-noise [B,T,H], then -- for the long-context
recipe only -- the floor mask and the floor values.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

VARIANTS = ("F1", "F1A", "F2", "F2A", "F3", "F3A")
PER_CHANNEL = ("F2", "F2A")
WINDOWED = ("F3", "F3A")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seqlen: int
    dk: int
    dv: int
    dtype: str          # "fp32" or "bf16": storage type of q, k, v and o
    chunk: int
    gates: str          # "uniform" | "softplus" | "floor5"
    seed: int
    variants: tuple = ("F1",)
    windows: tuple = (1,)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Sizes are the layer shapes of the pages' 124-130M models
# (12 heads of 64), plus a tiny fp32 case and a long-context case.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 256, 32, 32, "fp32", 16, "uniform", 101,
                          variants=VARIANTS, windows=(1, 2, 4)),
    "layer130m": Workload("layer130m", 8, 12, 2048, 64, 64, "bf16", 64, "softplus", 202,
                          variants=("F1", "F1A")),
    "layer130m_f2": Workload("layer130m_f2", 8, 12, 2048, 64, 64, "bf16", 64, "softplus", 303,
                             variants=("F2",)),
    "window_t4096": Workload("window_t4096", 4, 12, 4096, 64, 64, "bf16", 64, "uniform", 404,
                             variants=("F3", "F3A"), windows=(4, 8)),
    "long_t65536": Workload("long_t65536", 1, 16, 65536, 128, 128, "bf16", 64, "floor5", 505,
                            variants=("F1", "F1A")),
}

EPS_GAMMA = 1e-3
EPS_PHI = 1e-6
EPS_ETA = 1e-6


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Both the oracle and the GPU path consume these rounded values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(a)
    out[nan] = np.nan
    return out


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z):
    return np.logaddexp(0.0, z)


def make_inputs(w: Workload, variant: str = "F1", seed: int | None = None,
                window: int = 1) -> dict:
    """Draw one input set for workload ``w`` and ``variant``.

    Returns q, k, v (float32, already bf16-rounded for bf16 workloads), beta
    (float32 [B,T,H] or [B,T,H,dv]) and log_lambda (float32 [B,T,H]).  The
    gates are raw: log_lambda may lie below log(eps_gamma); clamping is the
    method's job."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant}")
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, T, H, dk, dv = w.batch, w.seqlen, w.heads, w.dk, w.dv
    q = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    k = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    v = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    bshape = (B, T, H, dv) if variant in PER_CHANNEL else (B, T, H)
    beta = _sigmoid(rng.standard_normal(bshape, dtype=np.float32)).astype(np.float32)
    if w.gates == "uniform":
        lam = rng.uniform(0.9, 1.0, size=(B, T, H)).astype(np.float32)
        g = np.log(lam).astype(np.float32)
    elif w.gates in ("softplus", "floor5"):
        z = rng.standard_normal((B, T, H), dtype=np.float32)
        g = (-_softplus(z) * 0.1).astype(np.float32)
        if w.gates == "floor5":
            mask = rng.random((B, T, H)) < 0.05
            u = rng.uniform(0.0, 1.0, size=(B, T, H))
            u = np.maximum(u, 1e-30)
            floor_g = np.log(u * EPS_GAMMA).astype(np.float32)
            g = np.where(mask, floor_g, g).astype(np.float32)
    else:
        raise ValueError(w.gates)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return dict(q=q, k=k, v=v, beta=beta, log_lambda=g)


def make_state(w: Workload, seed: int, window: int = 1, zero: bool = False) -> dict:
    """Draw an initial recurrent state: S ~ N(0,1)/sqrt(dk) (so S x has the scale
    of v), x_prev ~ N(0,1)/sqrt(dk), and the window pairs for window > 1."""
    rng = np.random.default_rng(seed)
    B, H, dk, dv = w.batch, w.heads, w.dk, w.dv
    if zero:
        S = np.zeros((B, H, dv, dk), np.float32)
        xp = np.zeros((B, H, dk), np.float32)
    else:
        S = (rng.standard_normal((B, H, dv, dk), dtype=np.float32) / math.sqrt(dk)).astype(np.float32)
        xp = (rng.standard_normal((B, H, dk), dtype=np.float32) / math.sqrt(dk)).astype(np.float32)
    st = dict(S=S, x_prev=xp)
    if window > 1:
        if zero:
            st["win_x"] = np.zeros((B, H, window - 1, dk), np.float32)
            st["win_v"] = np.zeros((B, H, window - 1, dv), np.float32)
        else:
            st["win_x"] = (rng.standard_normal((B, H, window - 1, dk), dtype=np.float32)
                           / math.sqrt(dk)).astype(np.float32)
            st["win_v"] = rng.standard_normal((B, H, window - 1, dv), dtype=np.float32)
    return st


def make_decode_inputs(batch: int, heads: int, dk: int, dv: int, variant: str, seed: int,
                       window: int = 1, dtype: str = "bf16", gates: str = "floor5") -> dict:
    """One decode step's inputs ([B,H,d] each) plus a random incoming state."""
    w = Workload("decode", batch=batch, heads=heads, seqlen=1, dk=dk, dv=dv, dtype=dtype,
                 chunk=1, gates=gates, seed=seed)
    inp = make_inputs(w, variant, seed)
    out = {n: a[:, 0] for n, a in inp.items()}
    out.update(make_state(w, seed + 7919, window))
    return out


def make_cotangents(w: Workload, seed: int, final: bool = True) -> dict:
    """Output gradients for a backward pass: do ~ N(0,1) [B,T,H,dv] (bf16-rounded
    for bf16 workloads, since it is stored in the input type) and, if ``final``,
    dS_T ~ N(0,1)/sqrt(dk) [B,H,dv,dk] fp32."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = w.batch, w.seqlen, w.heads, w.dk, w.dv
    do = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    if w.dtype == "bf16":
        do = round_bf16(do)
    out = dict(do=do, dS_T=None)
    if final:
        out["dS_T"] = (rng.standard_normal((B, H, dv, dk), dtype=np.float32)
                       / math.sqrt(dk)).astype(np.float32)
    return out
