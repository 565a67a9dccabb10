"""Shared helpers of the GPU parity tests (inputs to the device, rel-L2, oracle slices)."""

import numpy as np

import oracle
import workloads as W

TOL = {"fp32": 1e-4, "bf16": 2e-2}   # rel-L2 bar of the parity tests

# Largest error seen per (test family, quantity, input dtype) in this session;
# tests/conftest.py prints the table at the end of a run.
MAXIMA = {}


def record(family, errs, dtype):
    for name, e in errs.items():
        key = (family, name, dtype)
        MAXIMA[key] = max(MAXIMA.get(key, 0.0), float(e))


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def seq_errors(got, ref):
    """Per-sequence diagnostics of an output o [B, T, H, dv]: the largest rel-L2
    of one (b, h) sequence, and the largest error of one token row relative to
    the RMS row norm of its sequence.  A whole-tensor rel-L2 dilutes one wrong
    row of a long sequence by sqrt(T); these do not."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.linalg.norm(got - ref, axis=-1)               # [B, T, H]
    rn = np.linalg.norm(ref, axis=-1)
    seq_den = np.sqrt(np.sum(rn ** 2, axis=1))             # [B, H]
    seq_num = np.sqrt(np.sum(err ** 2, axis=1))
    head = np.where(seq_den > 0, seq_num / np.where(seq_den > 0, seq_den, 1.0), seq_num)
    rms = np.sqrt(np.mean(rn ** 2, axis=1, keepdims=True))  # [B, 1, H]
    row = np.where(rms > 0, err / np.where(rms > 0, rms, 1.0), err)
    return float(head.max()), float(row.max())


# a row may be worse than the whole sequence, but not by much: a wrong row is off by ~1
ROW_FACTOR = 5.0


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
