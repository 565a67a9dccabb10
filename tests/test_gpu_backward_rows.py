"""GPU parity of the recurrent-form backward (the shapes the chunk-parallel
backward does not build: Falcon-3 / 3A windows, head dims 32 and 128) against
the oracle's reverse-time adjoint of the recurrence (oracle.recurrent_backward),
through the C ABI.  The forward pass that supplies the per-chunk states is the
library's own (falcon_chunk_fwd), at a chunk it builds for the shape; the oracle
runs from the same seeded inputs.

The scalar is <do, o> + <dS_T, S_T>; every gradient (q, k, v, beta, log-decay,
initial S, x_prev and window) is compared by rel-L2 against the bar of the input
dtype.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import TOL, record, rel_l2, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu

BASE = ("dq", "dk", "dv", "dbeta", "dg", "dS0", "dx_prev0")
WINDOWED = ("F3", "F3A")


def grads_of(variant, window):
    return BASE + (("dwin_x0", "dwin_v0") if variant in WINDOWED and window > 1 else ())


def run_bwd(variant, w, seed, window=1, init=True, final_grad=True, align="prefix", chunk=64):
    import torch
    from recurrent_sequence_models_amd import FalconError, chunk_bwd, chunk_fwd
    win = window if variant in WINDOWED else 1
    inp = W.make_inputs(w, variant, seed=seed, window=win)
    st = W.make_state(w, seed + 1, window=win) if init else None
    cot = W.make_cotangents(w, seed + 2, final=final_grad)
    d = to_dev(inp, w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    do = torch.from_numpy(cot["do"]).to(tdt).cuda()
    dST = torch.from_numpy(cot["dS_T"]).cuda() if final_grad else None
    sd = state_to_dev(st) if st is not None else None
    # the per-chunk states of a forward the library builds for this shape: the
    # requested chunk, else the next smaller one
    for c in [chunk] + [x for x in (32, 16) if x < chunk]:
        try:
            _, _, cs = chunk_fwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=c,
                                 window=win, init=sd, final=False, chunk_states=True, align=align)
            break
        except FalconError:
            continue
    else:
        pytest.skip("no chunked forward for this shape")
    g = chunk_bwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], do, cs, init=sd, dS_T=dST,
                  align=align, chunk=c, window=win)
    torch.cuda.synchronize()
    return {n: to_np(g[n]) for n in grads_of(variant, window)}, inp, st, cot


def check_bwd(variant, w, seed, window=1, init=True, final_grad=True, align="prefix", chunk=64,
              family="backward, recurrent form"):
    print("case", variant, w.name, w.dtype, w.dk, w.seqlen, window, align, chunk, flush=True)
    got, inp, st, cot = run_bwd(variant, w, seed, window, init, final_grad, align, chunk)
    ref = oracle.recurrent_backward(variant, **inp, do=cot["do"], state=st, dS_T=cot["dS_T"], align=align,
                                    window=window if variant in WINDOWED else 1)
    errs = {n: rel_l2(got[n], ref[n]) for n in got}
    print(variant, w.name, w.dtype, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    record(family, errs, w.dtype)
    for n, e in errs.items():
        assert np.all(np.isfinite(got[n])), n
        assert e <= TOL[w.dtype], (n, e)
    return got, ref


def small(T, dtype, d=64, B=2, H=3, gates="floor5"):
    return W.WORKLOADS["layer130m"].replace(name=f"bwdr_T{T}_d{d}", batch=B, heads=H, seqlen=T, dtype=dtype,
                                            dk=d, dv=d, gates=gates)


# (the chunked forward pairs same-step window keys for bf16 inputs only)
WIN_CASES = [(v, bw, dt, al) for v in WINDOWED for bw in (2, 4, 8) for dt, al in
             (("bf16", "prefix"), ("bf16", "same"), ("fp32", "prefix"))]


@pytest.mark.parametrize("variant,window,dtype,align", WIN_CASES)
def test_window_backward(variant, window, dtype, align):
    """Windows of 2, 4 and 8 pairs from a random incoming state (window included),
    with a gradient on S_T; T = 150 ends in a ragged chunk."""
    check_bwd(variant, small(150, dtype), 7 + window, window=window, align=align)


DIM_CASES = [(v, d, dt) for d, dts in ((32, ("fp32", "bf16")), (128, ("bf16",)))
             for v in ("F1", "F1A", "F2", "F2A", "F3", "F3A") for dt in dts]


@pytest.mark.parametrize("variant,d,dtype", DIM_CASES)
def test_head_dims(variant, d, dtype):
    """Head dims 32 and 128, every variant (Falcon-3 / 3A with a window of 4)."""
    check_bwd(variant, small(100, dtype, d=d), 3 + d, window=4)


@pytest.mark.parametrize("variant,d", [("F1", 32), ("F2", 32), ("F3", 128), ("F2A", 128)])
def test_head_dims_same_step(variant, d):
    """The same-step pairing at head dims 32 and 128."""
    check_bwd(variant, small(90, "bf16", d=d), 13, window=2, align="same")


@pytest.mark.parametrize("variant,d,window", [("F3", 64, 4), ("F3A", 64, 8), ("F1", 128, 1), ("F2", 32, 1)])
def test_fresh_no_final_gradient(variant, d, window):
    """Fresh sequences (zero state and window) and no gradient on S_T."""
    check_bwd(variant, small(120, "bf16", d=d), 21, window=window, init=False, final_grad=False)


@pytest.mark.parametrize("variant", WINDOWED)
@pytest.mark.parametrize("T", [1, 3, 8, 9, 17])
def test_window_edge_lengths(variant, T):
    """Sequences shorter than the window of 8, and around one stretch of steps."""
    check_bwd(variant, small(T, "fp32", B=1, H=2), 40 + T, window=8)


@pytest.mark.parametrize("variant,window,d", [("F3", 8, 64), ("F3A", 4, 64), ("F3", 2, 128), ("F1", 1, 32)])
@pytest.mark.parametrize("chunk", [16, 32])
def test_from_smaller_chunks(variant, window, d, chunk):
    """Per-chunk states written by a forward at chunk 16 or 32 are the checkpoints."""
    check_bwd(variant, small(150, "bf16", d=d), 60 + chunk, window=window, chunk=chunk)


@pytest.mark.parametrize("variant,window,d", [("F3", 4, 64), ("F1", 1, 128)])
def test_deterministic(variant, window, d):
    a, *_ = run_bwd(variant, small(200, "bf16", d=d), 9, window=window)
    b, *_ = run_bwd(variant, small(200, "bf16", d=d), 9, window=window)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def sampled(variant, w, window, seed, picks):
    got, inp, st, cot = run_bwd(variant, w, seed, window=window)
    for b, h in picks:
        sub = {n: a[b:b + 1, :, h:h + 1] for n, a in inp.items()}
        sst = {n: a[b:b + 1, h:h + 1] for n, a in st.items()}
        ref = oracle.recurrent_backward(variant, **sub, do=cot["do"][b:b + 1, :, h:h + 1], state=sst,
                                        dS_T=cot["dS_T"][b:b + 1, h:h + 1], window=window)
        for n in got:
            if n in ("dS0", "dx_prev0", "dwin_x0", "dwin_v0"):
                gn = got[n][b:b + 1, h:h + 1]
            else:
                gn = got[n][b:b + 1, :, h:h + 1]
            e = rel_l2(gn, ref[n])
            print(variant, (b, h), n, f"{e:.2e}", flush=True)
            record("backward, recurrent form, full size sampled", {n: e}, w.dtype)
            assert e <= TOL[w.dtype], (b, h, n, e)


@pytest.mark.parametrize("variant", WINDOWED)
def test_window_full_size_sampled(variant):
    """The window workload's shape (B4 H12 T4096 d64, bf16, window 4); the oracle
    checks sampled sequences."""
    sampled(variant, W.WORKLOADS["window_t4096"], 4, 81, [(0, 0), (3, 11)])


def test_head_dim_128_long_sampled():
    """Head dim 128 over 4096 steps at the long-context workload's 16 heads."""
    w = W.WORKLOADS["long_t65536"].replace(name="long_t4096", seqlen=4096)
    sampled("F1", w, 1, 83, [(0, 5)])
