"""Shared helpers of the GPU parity tests (inputs to the device, rel-L2, oracle slices)."""

import numpy as np

import oracle
import workloads as W

TOL = {"fp32": 1e-4, "bf16": 2e-2}   # rel-L2 bar of the parity tests


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def to_dev(inp, dtype, device="cuda"):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for n, a in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        if n in ("q", "k", "v"):
            t = t.to(tdt)
        out[n] = t.to(device).contiguous()
    return out


def state_to_dev(st, device="cuda"):
    import torch
    return {n: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device) for n, a in st.items()}


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_subset(variant, inp, seqs, window=1, state=None, **kw):
    """Run the oracle on the sequences ``seqs`` = [(b, h), ...] only (they are
    independent), returning per-sequence results."""
    res = []
    for b, h in seqs:
        sub = {n: a[b:b + 1, :, h:h + 1] for n, a in inp.items()}
        st = None
        if state is not None:
            st = {n: a[b:b + 1, h:h + 1] for n, a in state.items()}
        res.append(oracle.recurrent(variant, **sub, window=window, state=st, **kw))
    return res
