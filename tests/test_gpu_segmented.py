"""GPU parity of the segment-parallel forward (falcon_chunk_fwd_segmented)
against the oracle's recurrent form, through the C ABI.

Every sequence is cut into nseg segments run at once; the result must be the
recurrent form's over the whole sequence (o, final S, x_prev and window), to
the same rel-L2 bars as the plain chunked forward."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import TOL, record, rel_l2, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu


def run_seg(variant, w, nseg, seed, window=1, init=False, align="prefix", inplace=False):
    import torch
    from recurrent_sequence_models_amd import chunk_fwd_segmented
    inp = W.make_inputs(w, variant, seed=seed)
    st = W.make_state(w, seed + 1000, window) if init else None
    d = to_dev(inp, w.dtype)
    sd = state_to_dev(st) if st is not None else None
    final = sd if (inplace and sd is not None) else True
    o, fin = chunk_fwd_segmented(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], nseg, chunk=w.chunk,
                                 window=window, init=sd, final=final, align=align)
    torch.cuda.synchronize()
    got = {"o": to_np(o)}
    got.update({n: to_np(t) for n, t in fin.items()})
    return got, inp, st


def check_seg(variant, w, nseg, seed, window=1, init=False, align="prefix", inplace=False):
    got, inp, st = run_seg(variant, w, nseg, seed, window, init, align, inplace)
    ref = oracle.recurrent(variant, **inp, window=window, state=st, align=align)
    keys = ("o", "S", "x_prev") + (("win_x", "win_v") if window > 1 else ())
    errs = {k: rel_l2(got[k], ref[k]) for k in keys}
    print(variant, w.name, w.dtype, w.seqlen, nseg, window, align, {k: f"{v:.2e}" for k, v in errs.items()},
          flush=True)
    record("segment-parallel forward", errs, w.dtype)
    for k, e in errs.items():
        assert e <= TOL[w.dtype], (k, e)
    return errs


def shape(T, dtype="bf16", d=64, chunk=64, B=2, H=3, gates="floor5"):
    return W.WORKLOADS["layer130m"].replace(name=f"seg_T{T}", batch=B, heads=H, seqlen=T, dk=d, dv=d, dtype=dtype,
                                            chunk=chunk, gates=gates)


@pytest.mark.parametrize("variant", ["F1", "F1A", "F2A"])
@pytest.mark.parametrize("nseg", [1, 2, 4, 8])
def test_segmented_bf16(variant, nseg):
    check_seg(variant, shape(512), nseg, 3 + nseg, init=True)


@pytest.mark.parametrize("variant,window", [("F3", 4), ("F3A", 4), ("F3", 8), ("F3A", 2)])
@pytest.mark.parametrize("nseg", [2, 8])
def test_segmented_windows(variant, window, nseg):
    check_seg(variant, shape(512), nseg, 7 + nseg, window=window, init=True)


@pytest.mark.parametrize("variant", ["F1", "F1A"])
def test_segmented_fp32(variant):
    check_seg(variant, shape(256, "fp32", d=32, chunk=32), 4, 5, init=True)


@pytest.mark.parametrize("variant", ["F1", "F3"])
def test_segmented_same_step(variant):
    window = 4 if variant == "F3" else 1
    check_seg(variant, shape(512), 4, 9, window=window, init=True, align="same")


def test_segmented_fresh_and_ragged_segments():
    """Fresh sequences; segments that are not a multiple of the chunk (T/nseg = 100)."""
    check_seg("F1", shape(400), 4, 13, init=False)


def test_segmented_in_place():
    check_seg("F1", shape(512), 4, 17, init=True, inplace=True)


def test_segmented_d128():
    check_seg("F1", shape(1024, d=128, B=1, H=2), 8, 19, init=True)


@pytest.mark.parametrize("variant,nseg", [("F3", 8), ("F3A", 4)])
def test_segmented_windows_d128(variant, nseg):
    """Windows at head dim 128: the map passes take two 64-channel slices."""
    check_seg(variant, shape(1024, d=128, B=1, H=2), nseg, 37, window=4, init=True)


def test_segmented_matches_plain_forward():
    """Same function as falcon_chunk_fwd on the same inputs (bf16 outputs: the two
    differ only by rounding)."""
    import torch
    from recurrent_sequence_models_amd import chunk_fwd
    w = shape(1024, B=1, H=4)
    got, inp, st = run_seg("F1", w, 8, 23, init=True)
    d = to_dev(inp, w.dtype)
    o, fin, _ = chunk_fwd("F1", d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=64,
                          init=state_to_dev(st))
    torch.cuda.synchronize()
    assert rel_l2(got["o"], to_np(o)) <= 1e-2
    assert rel_l2(got["S"], to_np(fin["S"])) <= 1e-3


@pytest.mark.parametrize("variant,nseg", [("F1", 8), ("F1A", 8), ("F1", 16)])
def test_segmented_long_sampled(variant, nseg):
    """The long-context shape (B1 H16 T65536 d128, bf16, chunk 64) in 8 segments (the
    benchmark's launch) and 16; the oracle checks two sampled heads over the whole
    sequence."""
    w = W.WORKLOADS["long_t65536"]
    got, inp, _ = run_seg(variant, w, nseg, 29)
    for h in (0, 11):
        sub = {n: a[:, :, h:h + 1] for n, a in inp.items()}
        ref = oracle.recurrent(variant, **sub)
        for k in ("o", "S", "x_prev"):
            g = got[k][:, :, h:h + 1] if k == "o" else got[k][:, h:h + 1]
            e = rel_l2(g, ref[k])
            print(variant, h, k, f"{e:.2e}", flush=True)
            record("segment-parallel forward, long context sampled", {k: e}, "bf16")
            assert e <= TOL["bf16"], (h, k, e)
