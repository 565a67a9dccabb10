"""GPU parity of the chunked backward pass (falcon_chunk_bwd) against the oracle's
reverse-time adjoint of the recurrence (oracle.recurrent_backward), through the
C ABI.  The forward pass that supplies the per-chunk states is the library's
own (falcon_chunk_fwd); the oracle runs from the same seeded inputs.

The scalar is <do, o> + <dS_T, S_T>; every gradient (q, k, v, beta, log-decay,
initial S and x_prev) is compared by rel-L2 against the bar of the input dtype.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import TOL, record, rel_l2, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dbeta", "dg", "dS0", "dx_prev0")


def run_bwd(variant, w, seed, init=True, final_grad=True, align="prefix", chunk=64):
    import torch
    from recurrent_sequence_models_amd import chunk_bwd, chunk_fwd
    inp = W.make_inputs(w, variant, seed=seed)
    st = W.make_state(w, seed + 1) if init else None
    cot = W.make_cotangents(w, seed + 2, final=final_grad)
    d = to_dev(inp, w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    do = torch.from_numpy(cot["do"]).to(tdt).cuda()
    dST = torch.from_numpy(cot["dS_T"]).cuda() if final_grad else None
    sd = state_to_dev(st) if st is not None else None
    # The library's fp32 forward at d 64 pairs same-step keys at chunk 32 only: take
    # the states at every second boundary of the chunk-32 forward (the chunk-64 ends).
    fc = 32 if (w.dtype == "fp32" and align == "same" and chunk == 64) else chunk
    _, _, cs = chunk_fwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=fc, init=sd,
                         final=False, chunk_states=True, align=align)
    if fc != chunk:
        n32 = cs.shape[2]
        idx = [min(2 * c + 1, n32 - 1) for c in range(-(-w.seqlen // 64))]
        cs = cs[:, :, idx].contiguous()
    g = chunk_bwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], do, cs, init=sd, dS_T=dST,
                  align=align, chunk=chunk)
    torch.cuda.synchronize()
    return {n: to_np(g[n]) for n in GRADS}, inp, st, cot


def check_bwd(variant, w, seed, init=True, final_grad=True, align="prefix", chunk=64):
    got, inp, st, cot = run_bwd(variant, w, seed, init, final_grad, align, chunk)
    ref = oracle.recurrent_backward(variant, **inp, do=cot["do"], state=st, dS_T=cot["dS_T"], align=align)
    errs = {n: rel_l2(got[n], ref[n]) for n in GRADS}
    print(variant, w.name, w.dtype, w.seqlen, align, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    record("backward", errs, w.dtype)
    for n, e in errs.items():
        assert np.all(np.isfinite(got[n])), n
        assert e <= TOL[w.dtype], (n, e)
    return got, ref


def small(T, dtype, B=2, H=3, gates="floor5"):
    return W.WORKLOADS["layer130m"].replace(name=f"bwd_T{T}", batch=B, heads=H, seqlen=T, dtype=dtype, gates=gates)


BWD_VARIANTS = ("F1", "F1A", "F2", "F2A")
CASES = [(v, dt, al) for v in BWD_VARIANTS for dt in ("fp32", "bf16") for al in ("prefix", "same")]


@pytest.mark.parametrize("variant,dtype,align", CASES)
@pytest.mark.parametrize("T", [200, 128])
def test_backward_continued(variant, dtype, align, T):
    """Several chunks with a ragged tail (200) or an exact multiple (128), from a
    random incoming state, with a gradient on S_T."""
    check_bwd(variant, small(T, dtype), 11 + T, init=True, final_grad=True, align=align)


@pytest.mark.parametrize("variant,dtype,align", CASES)
def test_backward_fresh_no_final_gradient(variant, dtype, align):
    """Fresh sequences (zero S and x_prev) and no gradient on S_T."""
    check_bwd(variant, small(100, dtype), 5, init=False, final_grad=False, align=align)


@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
@pytest.mark.parametrize("T", [1, 63, 64, 65])
def test_backward_edge_lengths(variant, T):
    """One step, one step short of a chunk, exactly one chunk, one step past it."""
    check_bwd(variant, small(T, "fp32", B=1, H=2), 31 + T, init=True, final_grad=True)


# The reverse scans hold the next chunks in a ring (four slots for Falcon-1, eight
# for the additive variants) and run whole turns of it, then a tail: chunk counts
# 3, 5, 7, 9 and 11 take the tail after zero, one or two whole turns.
@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
@pytest.mark.parametrize("T,dtype", [(150, "bf16"), (300, "fp32"), (420, "bf16"), (560, "bf16"), (700, "fp32")])
def test_backward_scan_ring_tails(variant, T, dtype):
    """Sequences of 3, 5, 7, 9 and 11 chunks of 64 steps (ragged last chunks)."""
    check_bwd(variant, small(T, dtype, B=1, H=2), 71 + T, init=True, final_grad=True)


@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
def test_backward_gates_clear_of_floor(variant):
    """Decays in (0.67, 1) only (no clamped step): every gate takes a gradient."""
    got, ref = check_bwd(variant, small(150, "fp32", gates="softplus"), 3)
    assert np.count_nonzero(got["dg"]) == got["dg"].size


@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
def test_backward_deterministic(variant):
    a, *_ = run_bwd(variant, small(200, "bf16"), 9)
    b, *_ = run_bwd(variant, small(200, "bf16"), 9)
    for n in GRADS:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
def test_backward_full_size_sampled(variant):
    """The full 130M-layer shape (B8 H12 T2048 d64, bf16, chunk 64); the oracle
    checks sampled sequences (sequences are independent, so their gradients are
    those of the oracle run on each alone)."""
    w = W.WORKLOADS["layer130m"]
    got, inp, st, cot = run_bwd(variant, w, 77, init=True, final_grad=True)
    for b, h in [(0, 0), (3, 7), (7, 11)]:
        sub = {n: a[b:b + 1, :, h:h + 1] for n, a in inp.items()}
        sst = {n: a[b:b + 1, h:h + 1] for n, a in st.items()}
        ref = oracle.recurrent_backward(variant, **sub, do=cot["do"][b:b + 1, :, h:h + 1], state=sst,
                                        dS_T=cot["dS_T"][b:b + 1, h:h + 1])
        for n in GRADS:
            if n in ("dS0", "dx_prev0"):
                gn = got[n][b:b + 1, h:h + 1]
            else:
                gn = got[n][b:b + 1, :, h:h + 1]
            e = rel_l2(gn, ref[n])
            print(variant, (b, h), n, f"{e:.2e}", flush=True)
            record("backward, full size sampled", {n: e}, "bf16")
            assert e <= TOL["bf16"], (b, h, n, e)


@pytest.mark.parametrize("variant", list(BWD_VARIANTS))
@pytest.mark.parametrize("chunk,dtype,align", [(16, "fp32", "prefix"), (32, "bf16", "prefix"), (32, "fp32", "same"),
                                               (16, "bf16", "same")])
def test_backward_from_smaller_chunks(variant, chunk, dtype, align):
    """Per-chunk states written by a forward at chunk 16 or 32: the backward reads
    the ones at 64-step boundaries (T = 150: a ragged last chunk)."""
    check_bwd(variant, small(150, dtype), 51 + chunk, init=True, final_grad=True, align=align, chunk=chunk)
