"""GPU parity of falcon_recurrent_step (single-token decode) against the oracle."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import TOL, record, rel_l2, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu

CASES = [("F1", 1), ("F1A", 1), ("F2", 1), ("F2A", 1), ("F3", 1), ("F3", 4), ("F3", 8), ("F3A", 4), ("F3A", 8)]


def step_gpu(variant, inp, st, window, dtype):
    import torch
    from recurrent_sequence_models_amd import recurrent_step
    d = to_dev({n: inp[n] for n in ("q", "k", "v", "beta", "log_lambda")}, dtype)
    o = recurrent_step(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], st, window=window)
    torch.cuda.synchronize()
    return to_np(o)


@pytest.mark.parametrize("variant,window", CASES)
@pytest.mark.parametrize("d,dtype", [(32, "fp32"), (64, "fp32"), (64, "bf16"), (128, "bf16")])
def test_decode_steps(variant, window, d, dtype):
    """Ten consecutive steps from a random state; state, window and outputs vs the oracle."""
    inp = W.make_decode_inputs(5, 3, d, d, variant, seed=55, window=window, dtype=dtype)
    st0 = {n: inp[n] for n in ("S", "x_prev", "win_x", "win_v") if n in inp}
    st_dev = state_to_dev(st0)
    st_ref = st0
    rng = np.random.default_rng(3)
    for t in range(10):
        x = {n: inp[n] for n in ("q", "k", "v", "beta", "log_lambda")}
        if t:
            x = {n: (a + 0.1 * rng.standard_normal(a.shape)).astype(np.float32) if n in ("q", "k", "v") else a
                 for n, a in x.items()}
            if dtype == "bf16":
                x = {n: W.round_bf16(a) if n in ("q", "k", "v") else a for n, a in x.items()}
        o = step_gpu(variant, x, st_dev, window, dtype)
        r = oracle.decode_step(variant, x["q"], x["k"], x["v"], x["beta"], x["log_lambda"], st_ref, window=window)
        st_ref = {n: r[n] for n in st0}
        record("decode step (10-step chains)", {"o": rel_l2(o, r["o"])}, dtype)
        assert rel_l2(o, r["o"]) <= TOL[dtype], (t, rel_l2(o, r["o"]))
    for n in st0:
        e = rel_l2(to_np(st_dev[n]), st_ref[n])
        record("decode step (10-step chains)", {n: e}, dtype)
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("variant,window", [("F1", 1), ("F1A", 1), ("F2", 1), ("F2A", 1)])
def test_decode_x_T_equals_chunked(variant, window):
    """T decode steps reproduce the chunked forward pass (GPU vs GPU, and both vs the oracle)."""
    import torch
    from recurrent_sequence_models_amd import chunk_fwd, new_state, recurrent_step
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=40, dtype="fp32")
    inp = W.make_inputs(w, variant, seed=77)
    d = to_dev(inp, "fp32")
    o_chunk, fin, _ = chunk_fwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=16)
    st = new_state(2, 3, 64, 64)
    outs = []
    for t in range(40):
        outs.append(recurrent_step(variant, *(d[n][:, t].contiguous() for n in ("q", "k", "v", "beta", "log_lambda")), st))
    torch.cuda.synchronize()
    o_dec = np.stack([to_np(o) for o in outs], axis=1)
    assert rel_l2(o_dec, to_np(o_chunk)) <= 1e-5
    assert rel_l2(to_np(st["S"]), to_np(fin["S"])) <= 1e-5
    r = oracle.recurrent(variant, **inp)
    assert rel_l2(o_dec, r["o"]) <= TOL["fp32"]


def test_decode_full_size_sampled():
    """Batch 256 x 16 heads x 128x128 fp32 states, bf16 q/k/v, ~5% of decays at the floor;
    the oracle checks a sample of states."""
    import torch
    from recurrent_sequence_models_amd import recurrent_step
    inp = W.make_decode_inputs(256, 16, 128, 128, "F1", seed=505, dtype="bf16")
    st = state_to_dev({n: inp[n] for n in ("S", "x_prev")})
    d = to_dev({n: inp[n] for n in ("q", "k", "v", "beta", "log_lambda")}, "bf16")
    o = recurrent_step("F1", d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], st)
    torch.cuda.synchronize()
    o = to_np(o)
    for b in (0, 100, 255):
        sub = {n: inp[n][b:b + 1] for n in inp}
        r = oracle.decode_step("F1", sub["q"], sub["k"], sub["v"], sub["beta"], sub["log_lambda"],
                               {"S": sub["S"], "x_prev": sub["x_prev"]})
        assert rel_l2(o[b], r["o"][0]) <= TOL["bf16"]
        assert rel_l2(to_np(st["S"][b]), r["S"][0]) <= TOL["bf16"]


@pytest.mark.parametrize("variant,window", CASES)
@pytest.mark.parametrize("d,dtype", [(32, "fp32"), (128, "bf16")])
def test_decode_same_step_pairs(variant, window, d, dtype):
    """Same-step pairs (phi(k_t), v_t): consecutive steps vs the oracle; x_prev is not read."""
    from recurrent_sequence_models_amd import recurrent_step
    import torch
    inp = W.make_decode_inputs(4, 3, d, d, variant, seed=56, window=window, dtype=dtype)
    st0 = {n: inp[n] for n in ("S", "x_prev", "win_x", "win_v") if n in inp}
    st_dev = state_to_dev(st0)
    st_ref = st0
    rng = np.random.default_rng(4)
    for t in range(6):
        x = {n: inp[n] for n in ("q", "k", "v", "beta", "log_lambda")}
        if t:
            x = {n: (a + 0.1 * rng.standard_normal(a.shape)).astype(np.float32) if n in ("q", "k", "v") else a
                 for n, a in x.items()}
            if dtype == "bf16":
                x = {n: W.round_bf16(a) if n in ("q", "k", "v") else a for n, a in x.items()}
        dd = to_dev(x, dtype)
        o = recurrent_step(variant, dd["q"], dd["k"], dd["v"], dd["beta"], dd["log_lambda"], st_dev, window=window,
                           align="same")
        torch.cuda.synchronize()
        r = oracle.decode_step(variant, x["q"], x["k"], x["v"], x["beta"], x["log_lambda"], st_ref, window=window,
                               align="same")
        st_ref = {n: r[n] for n in st0}
        assert rel_l2(to_np(o), r["o"]) <= TOL[dtype], (t, rel_l2(to_np(o), r["o"]))
    for n in st0:
        e = rel_l2(to_np(st_dev[n]), st_ref[n])
        assert e <= TOL[dtype], (n, e)
