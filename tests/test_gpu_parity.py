"""GPU parity of falcon_chunk_fwd against the fp64 oracle (through the C ABI).

Bar: rel-L2 <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs, on the
outputs o and on every state the call writes (S, x_prev, window, chunk states).
"""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import ROW_FACTOR, TOL, oracle_subset, record, rel_l2, seq_errors, state_to_dev, to_dev, to_np

pytestmark = pytest.mark.gpu

ROW_VARIANTS = ("F1", "F1A", "F2", "F2A")


def run_gpu(variant, inp, dtype, chunk, window=1, init=None, chunk_states=False, final=True, workspace=True,
            align="prefix"):
    import torch
    from recurrent_sequence_models_amd import chunk_fwd
    d = to_dev(inp, dtype)
    st = state_to_dev(init) if init is not None else None
    o, fin, cs = chunk_fwd(variant, d["q"], d["k"], d["v"], d["beta"], d["log_lambda"], chunk=chunk,
                           window=window, init=st, final=final, chunk_states=chunk_states, workspace=workspace,
                           align=align)
    torch.cuda.synchronize()
    out = {"o": to_np(o)}
    if fin is not None:
        out.update({n: to_np(t) for n, t in fin.items()})
    if cs is not None:
        out["chunk_states"] = to_np(cs)
    return out


def check(variant, w, seed, window=1, init=False, chunk=None, chunk_states=False, workspace=True, align="prefix"):
    inp = W.make_inputs(w, variant, seed=seed)
    st = W.make_state(w, seed + 1000, window) if init else None
    chunk = chunk or w.chunk
    g = run_gpu(variant, inp, w.dtype, chunk, window, st, chunk_states, workspace=workspace, align=align)
    r = oracle.recurrent(variant, **inp, window=window, state=st, return_states=chunk_states, align=align)
    tol = TOL[w.dtype]
    errs = {"o": rel_l2(g["o"], r["o"]), "S": rel_l2(g["S"], r["S"]), "x_prev": rel_l2(g["x_prev"], r["x_prev"])}
    if window > 1:
        errs["win_x"] = rel_l2(g["win_x"], r["win_x"])
        errs["win_v"] = rel_l2(g["win_v"], r["win_v"])
    if chunk_states:
        T = w.seqlen
        ends = [min(T, c0 + chunk) - 1 for c0 in range(0, T, chunk)]
        ref = np.moveaxis(r["states"][:, ends], 2, 1)           # [B,H,NC,dv,dk]
        errs["chunk_states"] = rel_l2(g["chunk_states"], ref)
    head, row = seq_errors(g["o"], r["o"])
    print(variant, w.name, seed, {k: f"{v:.2e}" for k, v in errs.items()},
          f"o per-head max {head:.2e} row max {row:.2e}", flush=True)
    record("chunked forward", {**errs, "o, worst sequence": head, "o, worst row": row}, w.dtype)
    for k, e in errs.items():
        assert e <= tol, (k, e)
    assert head <= tol, ("o per-head", head)
    assert row <= ROW_FACTOR * tol, ("o per-row", row)
    return errs


TINY = W.WORKLOADS["tiny_fp32"]


@pytest.mark.parametrize("variant", ROW_VARIANTS)
@pytest.mark.parametrize("seed", [101, 102, 103])
def test_tiny_fp32(variant, seed):
    """The tiny fp32 workload (B1 H2 T256 d32, chunk 16): recurrent oracle vs chunked GPU."""
    check(variant, TINY, seed)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_chunks_ragged_with_state(variant, chunk):
    w = TINY.replace(batch=2, heads=3, seqlen=203, dk=64, dv=64, chunk=chunk, gates="softplus")
    check(variant, w, 7, init=True, chunk_states=True)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
@pytest.mark.parametrize("d", [32, 64, 128])
def test_bf16_ragged(variant, d):
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=200, dk=d, dv=d)
    check(variant, w, 11, init=True, chunk_states=True)


# The default calls above take the chunk-parallel path (prep over all chunks +
# state scan) wherever a workspace applies; these run the fused path (no
# workspace) on the same cases, and check that the two paths agree.
@pytest.mark.parametrize("variant", ROW_VARIANTS)
@pytest.mark.parametrize("dtype,d,chunk", [("fp32", 64, 16), ("fp32", 32, 64), ("bf16", 32, 64), ("bf16", 64, 32),
                                           ("bf16", 64, 64)])
def test_fused_path(variant, dtype, d, chunk):
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=203, dk=d, dv=d, chunk=chunk, dtype=dtype)
    check(variant, w, 17, init=True, chunk_states=True, workspace=False)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_fused_and_split_paths_agree(variant):
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=333)
    inp = W.make_inputs(w, variant, seed=19)
    st = W.make_state(w, 1019)
    a = run_gpu(variant, inp, "bf16", 64, init=st, chunk_states=True, workspace=True)
    b = run_gpu(variant, inp, "bf16", 64, init=st, chunk_states=True, workspace=False)
    for k in a:
        e = rel_l2(a[k], b[k])
        assert e <= 5e-3, (k, e)   # same arithmetic up to accumulation order and bf16 rounding of tiles


# The state scan splits the value channels of a sequence over NS workgroups,
# chosen from B*H (smallest split giving >= 128 workgroups among those built);
# when B*H is a multiple of 8 the slices of a sequence share an XCD.  These
# shapes reach every built split and both workgroup mappings.
SPLIT_SHAPES = [
    (64, 8, 16, 130),    # B*H = 128: NS = 1
    (64, 8, 8, 130),     # B*H = 64: NS = 2, XCD-grouped
    (64, 1, 66, 130),    # B*H = 66: NS = 2, plain mapping
    (64, 4, 8, 130),     # B*H = 32: NS = 4 (two-kernel form; the one-pass form takes 2), XCD-grouped
    (64, 1, 5, 130),     # B*H = 5: NS = 4 (one-pass: 2), plain mapping
    (128, 2, 32, 100),   # NS = 2, XCD-grouped
    (128, 4, 8, 100),    # NS = 4
    (128, 1, 6, 100),    # NS = 8, plain mapping
]


@pytest.mark.parametrize("variant", ROW_VARIANTS)
@pytest.mark.parametrize("d,B,H,T", SPLIT_SHAPES)
def test_scan_channel_splits(variant, d, B, H, T):
    w = W.WORKLOADS["layer130m"].replace(batch=B, heads=H, seqlen=T, dk=d, dv=d)
    check(variant, w, 23, init=True, chunk_states=True)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65])
def test_short_sequences(variant, T):
    w = TINY.replace(batch=1, heads=2, seqlen=T, dk=32, dv=32, chunk=16)
    check(variant, w, 13)
    w = W.WORKLOADS["layer130m"].replace(batch=1, heads=2, seqlen=T)
    check(variant, w, 14, init=True)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_floor_decay_long_chunks(variant):
    """~5% of steps below the eps_gamma floor (clamped), d = 128, several chunks."""
    w = W.WORKLOADS["long_t65536"].replace(heads=4, seqlen=640)
    check(variant, w, 505)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_correlated_keys(variant):
    """k_t = k_{t-1} + 0.1 noise: ill-conditioned Gram blocks stress the triangular solve."""
    w = TINY.replace(batch=1, heads=2, seqlen=130, dk=64, dv=64, chunk=64, gates="softplus")
    inp = W.make_inputs(w, variant, seed=21)
    k = inp["k"].copy()
    for t in range(1, k.shape[1]):
        k[:, t] = k[:, t - 1] + 0.1 * inp["k"][:, t]
    inp["k"] = k.astype(np.float32)
    g = run_gpu(variant, inp, "fp32", 64)
    r = oracle.recurrent(variant, **inp)
    assert rel_l2(g["o"], r["o"]) <= TOL["fp32"]
    assert rel_l2(g["S"], r["S"]) <= TOL["fp32"]


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_split_continuation_in_place(variant):
    """Two calls, the second continuing in place from the first one's state."""
    import torch
    from recurrent_sequence_models_amd import chunk_fwd, new_state
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=2, seqlen=300)
    inp = W.make_inputs(w, variant, seed=31)
    d = to_dev(inp, "bf16")
    st = new_state(2, 2, 64, 64)
    o1, _, _ = chunk_fwd(variant, *(d[n][:, :137].contiguous() for n in ("q", "k", "v", "beta", "log_lambda")),
                         init=st, final=st)
    o2, _, _ = chunk_fwd(variant, *(d[n][:, 137:].contiguous() for n in ("q", "k", "v", "beta", "log_lambda")),
                         init=st, final=st)
    torch.cuda.synchronize()
    r = oracle.recurrent(variant, **inp)
    o = np.concatenate([to_np(o1), to_np(o2)], axis=1)
    assert rel_l2(o, r["o"]) <= TOL["bf16"]
    assert rel_l2(to_np(st["S"]), r["S"]) <= TOL["bf16"]
    assert rel_l2(to_np(st["x_prev"]), r["x_prev"]) <= 1e-6


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_deterministic(variant):
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=256)
    inp = W.make_inputs(w, variant, seed=41)
    a = run_gpu(variant, inp, "bf16", 64)
    b = run_gpu(variant, inp, "bf16", 64)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name,variant", [("layer130m", "F1"), ("layer130m", "F1A"), ("layer130m_f2", "F2")])
def test_full_size_sampled(name, variant):
    """The full 130M-layer workload (B8 H12 T2048 d64, bf16, chunk 64) in the launch
    configuration the benchmark times; the oracle checks a sample of sequences."""
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, variant, seed=w.seed)
    g = run_gpu(variant, inp, w.dtype, w.chunk)
    seqs = [(0, 0), (3, 7), (7, 11)]
    refs = oracle_subset(variant, inp, seqs)
    for (b, h), r in zip(seqs, refs):
        eo = rel_l2(g["o"][b, :, h], r["o"][0, :, 0])
        es = rel_l2(g["S"][b, h], r["S"][0, 0])
        print(variant, (b, h), f"o {eo:.2e} S {es:.2e}", flush=True)
        record("full-size workloads, sampled", {"o": eo, "S": es}, "bf16")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.all(np.isfinite(g["o"]))


# ---- one-pass kernel (calls without a workspace) ------------------------------------
# One launch per call: derive waves build each system's Gram / score blocks in LDS
# one system ahead of the state waves.  Shapes reach both channel splits it builds
# (d = 32: 1 or 2 slices; d = 64: 2) and both workgroup mappings, with windows.
ONEPASS_SHAPES = [
    (32, 8, 16, 130, 1),     # B*H = 128: one slice
    (32, 1, 5, 130, 1),      # two slices, plain mapping
    (64, 4, 8, 130, 1),      # two slices, XCD-grouped
    (64, 1, 3, 70, 4),       # window of 4
    (64, 2, 4, 70, 8),       # window of 8
    (32, 1, 2, 33, 2),       # window of 2, short
]


ONEPASS_CASES = [(v, *shape) for shape in ONEPASS_SHAPES
                 for v in (("F3", "F3A") if shape[-1] > 1 else ("F1", "F1A", "F2", "F2A", "F3", "F3A"))]


@pytest.mark.parametrize("variant,d,B,H,T,bw", ONEPASS_CASES)
def test_onepass_shapes(variant, d, B, H, T, bw):
    w = W.WORKLOADS["layer130m"].replace(batch=B, heads=H, seqlen=T, dk=d, dv=d)
    check(variant, w, 71, window=bw, init=True, chunk_states=True, workspace=False)


@pytest.mark.parametrize("variant,bw", [("F1", 1), ("F2", 1), ("F1A", 1), ("F3", 4), ("F3A", 8)])
def test_onepass_continuation_in_place(variant, bw):
    """Calls continuing in place without a workspace: with two channel slices per
    sequence the outgoing x_prev / window goes through the tail kernel."""
    import torch
    from recurrent_sequence_models_amd import chunk_fwd, new_state
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=2, seqlen=300)
    inp = W.make_inputs(w, variant, seed=72)
    d = to_dev(inp, "bf16")
    st = new_state(2, 2, 64, 64, window=bw)
    outs = []
    for sl in (slice(0, 5), slice(5, 141), slice(141, 300)):
        o, _, _ = chunk_fwd(variant, *(d[n][:, sl].contiguous() for n in ("q", "k", "v", "beta", "log_lambda")),
                            window=bw, init=st, final=st, workspace=False)
        outs.append(to_np(o))
    torch.cuda.synchronize()
    r = oracle.recurrent(variant, **inp, window=bw)
    assert rel_l2(np.concatenate(outs, axis=1), r["o"]) <= TOL["bf16"]
    names = ("S", "x_prev", "win_x", "win_v") if bw > 1 else ("S", "x_prev")
    for n in names:
        assert rel_l2(to_np(st[n]), r[n]) <= TOL["bf16"], n


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_onepass_full_size_sampled(variant):
    """The full 130M-layer workloads through the one-pass kernel (the benchmark's
    default path for them); the oracle checks a sample of sequences."""
    w = W.WORKLOADS["layer130m_f2" if variant in ("F2", "F2A") else "layer130m"]
    inp = W.make_inputs(w, variant, seed=w.seed)
    g = run_gpu(variant, inp, w.dtype, w.chunk, workspace=False)
    seqs = [(0, 0), (5, 9)]
    refs = oracle_subset(variant, inp, seqs)
    for (b, h), r in zip(seqs, refs):
        eo = rel_l2(g["o"][b, :, h], r["o"][0, :, 0])
        es = rel_l2(g["S"][b, h], r["S"][0, 0])
        print(variant, (b, h), f"o {eo:.2e} S {es:.2e}", flush=True)
        record("full-size workloads, sampled", {"o": eo, "S": es}, "bf16")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.all(np.isfinite(g["o"]))


# ---- same-step pairs (phi(k_t), v_t): the pages' contrast to the prefix pair -----------
SAME_CASES = [(v, 1) for v in ROW_VARIANTS] + [("F3", 2), ("F3", 4), ("F3", 8), ("F3A", 4), ("F3A", 8)]


SAME_SHAPES = [(v, bw, "bf16", 64, 203, 64) for v, bw in SAME_CASES] + \
              [(v, 1, "fp32", 32, 150, 32) for v in ROW_VARIANTS]


@pytest.mark.parametrize("variant,bw,dtype,d,T,chunk", SAME_SHAPES)
@pytest.mark.parametrize("workspace", [True, False])
def test_same_step_pairs(variant, bw, dtype, d, T, chunk, workspace):
    """Both chunk-parallel forms, carried state (x_prev present but not read), chunk states."""
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=T, dk=d, dv=d, dtype=dtype, chunk=chunk)
    check(variant, w, 81, window=bw, init=True, chunk_states=True, workspace=workspace, align="same")


@pytest.mark.parametrize("variant,bw", [("F1", 1), ("F2", 1), ("F3", 4), ("F3A", 2)])
@pytest.mark.parametrize("d,B,H,T", [(128, 1, 6, 100), (64, 8, 16, 70), (32, 1, 5, 9)])
def test_same_step_splits_and_short(variant, bw, d, B, H, T):
    w = W.WORKLOADS["layer130m"].replace(batch=B, heads=H, seqlen=T, dk=d, dv=d)
    check(variant, w, 82, window=bw, init=True, chunk_states=True, align="same")


@pytest.mark.parametrize("variant,bw,workspace", [("F1", 1, False), ("F1", 1, True), ("F3", 4, True),
                                                  ("F3", 8, False)])
def test_same_step_continuation_in_place(variant, bw, workspace):
    import torch
    from recurrent_sequence_models_amd import chunk_fwd, new_state
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=2, seqlen=300)
    inp = W.make_inputs(w, variant, seed=83)
    d = to_dev(inp, "bf16")
    st = new_state(2, 2, 64, 64, window=bw)
    outs = []
    for sl in (slice(0, 5), slice(5, 141), slice(141, 300)):
        o, _, _ = chunk_fwd(variant, *(d[n][:, sl].contiguous() for n in ("q", "k", "v", "beta", "log_lambda")),
                            window=bw, init=st, final=st, workspace=workspace, align="same")
        outs.append(to_np(o))
    torch.cuda.synchronize()
    r = oracle.recurrent(variant, **inp, window=bw, align="same")
    assert rel_l2(np.concatenate(outs, axis=1), r["o"]) <= TOL["bf16"]
    for n in (("S", "x_prev", "win_x", "win_v") if bw > 1 else ("S", "x_prev")):
        assert rel_l2(to_np(st[n]), r[n]) <= TOL["bf16"], n


# ---- packed sequences of different lengths (cu_seqlens) ---------------------------
def run_varlen(variant, lens, dtype, d, chunk, bw, seed, init=True, in_place=False, align="prefix", workspace=None):
    """Pack len(lens) independent sequences (H = 3), run falcon_chunk_fwd_varlen and
    the oracle per sequence; returns the rel-L2 errors per sequence and name."""
    import torch
    from recurrent_sequence_models_amd import chunk_fwd_varlen, new_state
    H = 3
    seqs, refs, states = [], [], []
    for n, T in enumerate(lens):
        w = W.WORKLOADS["layer130m"].replace(batch=1, heads=H, seqlen=max(T, 1), dk=d, dv=d, dtype=dtype, chunk=chunk)
        inp = W.make_inputs(w, variant, seed=seed + n)
        inp = {k: a[:, :T] for k, a in inp.items()}
        st = W.make_state(w, seed + 100 + n, bw) if init else None
        seqs.append(inp)
        states.append(st)
        refs.append(oracle.recurrent(variant, **inp, window=bw, state=st, align=align) if T > 0 else None)
    cat = {k: np.concatenate([x[k][0] for x in seqs], axis=0) for k in seqs[0]}   # [total, H, ...]
    d_in = to_dev(cat, dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    st_dev = None
    if init:
        st_dev = state_to_dev({k: np.concatenate([s[k] for s in states], axis=0) for k in states[0]})
    fin = st_dev if in_place else True
    o, fin = chunk_fwd_varlen(variant, d_in["q"], d_in["k"], d_in["v"], d_in["beta"], d_in["log_lambda"], cu,
                              chunk=chunk, window=bw, init=st_dev, final=fin, align=align, workspace=workspace)
    torch.cuda.synchronize()
    o = to_np(o)
    fin = {k: to_np(t) for k, t in fin.items()}
    errs = []
    offs = np.concatenate([[0], np.cumsum(lens)])
    for n, r in enumerate(refs):
        if r is None:
            continue
        e = {"o": rel_l2(o[offs[n]:offs[n + 1]], r["o"][0]), "S": rel_l2(fin["S"][n], r["S"][0]),
             "x_prev": rel_l2(fin["x_prev"][n], r["x_prev"][0])}
        if bw > 1:
            e["win_x"] = rel_l2(fin["win_x"][n], r["win_x"][0])
            e["win_v"] = rel_l2(fin["win_v"][n], r["win_v"][0])
        errs.append(e)
    return errs


VARLEN_CASES = [(v, 1) for v in ROW_VARIANTS] + [("F3", 4), ("F3A", 8), ("F3", 2)]


@pytest.mark.parametrize("variant,bw", VARLEN_CASES)
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("workspace", [False, True])
def test_varlen_bf16(variant, bw, in_place, workspace):
    """Without a workspace: the one-pass kernel; with one: prep over every image
    slot of the packed layout, then the state scan."""
    errs = run_varlen(variant, [1, 17, 64, 65, 130, 200, 7], "bf16", 64, 64, bw, 91, in_place=in_place,
                      workspace=workspace)
    for e in errs:
        for k, x in e.items():
            assert x <= TOL["bf16"], (k, x, e)


@pytest.mark.parametrize("variant,bw", VARLEN_CASES)
@pytest.mark.parametrize("in_place", [False, True])
def test_varlen_d128(variant, bw, in_place):
    """bf16 at d = 128, chunk 64 (the decode workload's head dim): packed sequences
    on the chunk-parallel path (with a workspace), an empty one among them."""
    errs = run_varlen(variant, [3, 64, 0, 150, 1, 90], "bf16", 128, 64, bw, 94, in_place=in_place)
    assert len(errs) == 5
    for e in errs:
        for k, x in e.items():
            assert x <= TOL["bf16"], (k, x, e)


@pytest.mark.parametrize("variant,bw", [("F1", 1), ("F3", 4)])
def test_varlen_workspace_same_step_and_small_chunks(variant, bw):
    """Same-step pairs on the packed chunk-parallel path; fp32 at chunk 16 with a workspace."""
    errs = run_varlen(variant, [40, 0, 90, 5], "bf16", 64, 64, bw, 95, align="same", workspace=True)
    errs += run_varlen(variant if bw == 1 else "F1", [3, 50, 33, 1], "fp32", 32, 16, 1, 96, workspace=True)
    for e in errs:
        for k, x in e.items():
            assert x <= TOL["bf16"], (k, x, e)


@pytest.mark.parametrize("variant", ROW_VARIANTS)
def test_varlen_fp32(variant):
    errs = run_varlen(variant, [3, 50, 33, 1], "fp32", 32, 32, 1, 92)
    for e in errs:
        for k, x in e.items():
            assert x <= TOL["fp32"], (k, x, e)


@pytest.mark.parametrize("variant,bw", [("F1", 1), ("F3", 4)])
def test_varlen_empty_and_same_step(variant, bw):
    """A zero-length sequence in the pack is skipped; same-step pairs on packed sequences."""
    errs = run_varlen(variant, [40, 0, 90], "bf16", 64, 64, bw, 93, align="same")
    assert len(errs) == 2
    for e in errs:
        for k, x in e.items():
            assert x <= TOL["bf16"], (k, x, e)


# ---- Falcon-3 / 3A: window of Bw pairs --------------------------------------------
WIN_CASES = [("F3", 2), ("F3", 4), ("F3", 8), ("F3A", 2), ("F3A", 4), ("F3A", 8), ("F3", 1), ("F3A", 1)]


@pytest.mark.parametrize("variant,bw", WIN_CASES)
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_window_fp32(variant, bw, chunk):
    w = TINY.replace(batch=2, heads=2, seqlen=150, chunk=chunk)
    check(variant, w, 61, window=bw, init=True, chunk_states=True)


@pytest.mark.parametrize("variant,bw", WIN_CASES)
def test_window_tiny_workload(variant, bw):
    """The tiny fp32 workload itself (B1 H2 T256 d32, chunk 16), fresh sequences."""
    check(variant, TINY, 101, window=bw)


@pytest.mark.parametrize("variant,bw", WIN_CASES)
@pytest.mark.parametrize("d", [32, 64, 128])
def test_window_bf16(variant, bw, d):
    w = W.WORKLOADS["window_t4096"].replace(batch=2, heads=2, seqlen=203, dk=d, dv=d)
    check(variant, w, 62, window=bw, init=True, chunk_states=True)


@pytest.mark.parametrize("variant,bw", [("F3", 4), ("F3A", 8)])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_window_kernel_bf16(variant, bw, d):
    """The windowed kernel (no workspace) on the shapes the chunk-parallel path also takes."""
    w = W.WORKLOADS["window_t4096"].replace(batch=2, heads=2, seqlen=203, dk=d, dv=d)
    check(variant, w, 66, window=bw, init=True, chunk_states=True, workspace=False)


@pytest.mark.parametrize("variant,bw", [("F3", 2), ("F3", 4), ("F3", 8), ("F3A", 2), ("F3A", 4), ("F3A", 8)])
def test_window_split_and_window_kernel_agree(variant, bw):
    w = W.WORKLOADS["window_t4096"].replace(batch=2, heads=3, seqlen=333)
    inp = W.make_inputs(w, variant, seed=67)
    st = W.make_state(w, 1067, bw)
    a = run_gpu(variant, inp, "bf16", 64, window=bw, init=st, chunk_states=True, workspace=True)
    b = run_gpu(variant, inp, "bf16", 64, window=bw, init=st, chunk_states=True, workspace=False)
    for k in a:
        e = rel_l2(a[k], b[k])
        assert e <= 5e-3, (k, e)   # same arithmetic up to accumulation order and bf16 rounding of tiles


# Windowed systems hold 64 / Bw steps; these shapes reach every built channel
# split of the scan (as for one pair per step) with several windows.
WIN_SPLIT_SHAPES = [
    (64, 8, 16, 70),     # B*H = 128: NS = 1
    (64, 1, 5, 70),      # NS = 2, plain mapping
    (128, 2, 32, 50),    # NS = 2, XCD-grouped
    (128, 4, 8, 50),     # NS = 4
    (128, 1, 6, 50),     # NS = 8, plain mapping
]


@pytest.mark.parametrize("variant,bw", [("F3", 2), ("F3", 8), ("F3A", 4)])
@pytest.mark.parametrize("d,B,H,T", WIN_SPLIT_SHAPES)
def test_window_scan_channel_splits(variant, bw, d, B, H, T):
    w = W.WORKLOADS["window_t4096"].replace(batch=B, heads=H, seqlen=T, dk=d, dv=d)
    check(variant, w, 68, window=bw, init=True, chunk_states=True)


@pytest.mark.parametrize("variant,bw", [("F3", 2), ("F3", 4), ("F3", 8), ("F3A", 4), ("F3A", 8)])
@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 9, 17, 33])
def test_window_short_systems(variant, bw, T):
    """Chunk 64 (systems of 64 / Bw steps) with sequences about the window's
    length: the first system's rows mix carried and new pairs, the last is ragged."""
    w = TINY.replace(batch=1, heads=2, seqlen=T, dk=32, dv=32, chunk=64)
    check(variant, w, 65, window=bw, init=True, chunk_states=True)


@pytest.mark.parametrize("variant,bw", [("F3", 4), ("F3", 8), ("F3A", 8)])
@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 9, 33])
def test_window_short(variant, bw, T):
    """Sequences shorter than the window: the final window mixes carried and new pairs."""
    w = TINY.replace(batch=1, heads=2, seqlen=T, dk=32, dv=32, chunk=16)
    check(variant, w, 63, window=bw, init=True)


@pytest.mark.parametrize("variant,bw", [("F3", 4), ("F3A", 4), ("F3", 8)])
def test_window_split_continuation_in_place(variant, bw):
    import torch
    from recurrent_sequence_models_amd import chunk_fwd, new_state
    w = W.WORKLOADS["window_t4096"].replace(batch=2, heads=2, seqlen=300)
    inp = W.make_inputs(w, variant, seed=64)
    d = to_dev(inp, "bf16")
    st = new_state(2, 2, 64, 64, window=bw)
    outs = []
    for sl in (slice(0, 5), slice(5, 141), slice(141, 300)):
        o, _, _ = chunk_fwd(variant, *(d[n][:, sl].contiguous() for n in ("q", "k", "v", "beta", "log_lambda")),
                            window=bw, init=st, final=st)
        outs.append(to_np(o))
    torch.cuda.synchronize()
    r = oracle.recurrent(variant, **inp, window=bw)
    assert rel_l2(np.concatenate(outs, axis=1), r["o"]) <= TOL["bf16"]
    for n in ("S", "x_prev", "win_x", "win_v"):
        assert rel_l2(to_np(st[n]), r[n]) <= TOL["bf16"], n


@pytest.mark.parametrize("variant,bw", [("F3", 4), ("F3", 8), ("F3A", 4), ("F3A", 8)])
def test_window_full_size_sampled(variant, bw):
    """The full window workload (B4 H12 T4096 d64, bf16, chunk 64); sampled sequences."""
    w = W.WORKLOADS["window_t4096"]
    inp = W.make_inputs(w, variant, seed=w.seed)
    g = run_gpu(variant, inp, w.dtype, w.chunk, window=bw)
    seqs = [(0, 0), (3, 11)]
    refs = oracle_subset(variant, inp, seqs, window=bw)
    for (b, h), r in zip(seqs, refs):
        eo = rel_l2(g["o"][b, :, h], r["o"][0, :, 0])
        es = rel_l2(g["S"][b, h], r["S"][0, 0])
        print(variant, bw, (b, h), f"o {eo:.2e} S {es:.2e}", flush=True)
        record("full-size workloads, sampled", {"o": eo, "S": es}, "bf16")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("workspace", [False, True])
def test_forward_call_reuse(workspace):
    """A ForwardCall validated once and issued again after its input buffers were
    refilled gives what a fresh chunk_fwd call gives on the new contents."""
    import torch
    from recurrent_sequence_models_amd import ForwardCall, chunk_fwd
    w = W.WORKLOADS["layer130m"].replace(batch=2, heads=3, seqlen=150)
    d1 = to_dev(W.make_inputs(w, "F1", seed=201), "bf16")
    d2 = to_dev(W.make_inputs(w, "F1", seed=202), "bf16")
    names = ("q", "k", "v", "beta", "log_lambda")
    buf = {n: d1[n].clone() for n in names}
    call = ForwardCall("F1", *(buf[n] for n in names), chunk_states=True, workspace=workspace)
    for d in (d1, d2, d1):
        for n in names:
            buf[n].copy_(d[n])
        o, fin, cs = call()
        ro, rfin, rcs = chunk_fwd("F1", *(d[n] for n in names), chunk_states=True, workspace=workspace)
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(cs, rcs)
        assert torch.equal(fin["S"], rfin["S"]) and torch.equal(fin["x_prev"], rfin["x_prev"])


# ---- Falcon-3A windows at d = 64, chunk 64: the banded-weight kernels ----------------
# (band_state / band_scan / band_out; the window's earlier pairs enter each chunk as a
# halo block, so sequences shorter than the window and chunk edges are the cases.)
@pytest.mark.parametrize("bw", [2, 4, 8])
@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 9, 63, 64, 65, 130])
@pytest.mark.parametrize("align", ["prefix", "same"])
def test_band_short_and_ragged(bw, T, align):
    w = W.WORKLOADS["window_t4096"].replace(batch=1, heads=3, seqlen=T)
    check("F3A", w, 71, window=bw, init=True, chunk_states=True, align=align)


@pytest.mark.parametrize("bw", [2, 4, 8])
@pytest.mark.parametrize("init", [False, True])
def test_band_fp32(bw, init):
    w = TINY.replace(batch=2, heads=2, seqlen=200, dk=64, dv=64, chunk=64)
    check("F3A", w, 72, window=bw, init=init, chunk_states=True)


@pytest.mark.parametrize("bw", [4, 8])
@pytest.mark.parametrize("gates", ["floor5", "softplus"])
def test_band_decay_regimes(bw, gates):
    """Steps at the eps_gamma floor (a window's weights then span e^{-7 |log eps|})
    and softplus gates, several chunks."""
    w = W.WORKLOADS["window_t4096"].replace(batch=2, heads=2, seqlen=333, gates=gates)
    check("F3A", w, 73, window=bw, init=True, chunk_states=True)
