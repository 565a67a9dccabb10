"""CPU tests of the C ABI: the library loads, exports what include/falcon.h
declares, and rejects invalid calls on the host before any HIP call.

No kernel is launched here.  Every call below is invalid by construction;
pointer arguments that are never dereferenced use a fake aligned address, so
the tests are skipped on a machine that has a GPU (a validation bug must never
be able to launch a kernel on a fake pointer)."""

import ctypes
import os
import re

import pytest

from recurrent_sequence_models_amd import falcon as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "falcon.h")
FAKE = ctypes.c_void_p(0x10000)    # aligned, never dereferenced


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="invalid-call tests run only where no GPU is visible")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(falcon_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    L = F.lib()
    names = declared_functions()
    assert set(names) == set(F.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    L = F.lib()
    assert L.falcon_abi_version() == 4
    for code in range(5):
        s = F.status_string(code)
        assert s.startswith("FALCON_")
    assert "unknown" in F.status_string(99)


def good_shape(**kw):
    d = dict(variant="F1", dtype="bf16", batch=2, seqlen=100, heads=3, dk=64, dv=64, chunk=64, window=1)
    d.update(kw)
    return F.make_shape(**d)


def call_fwd(shape, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, init=None, final=None, o=FAKE,
             cs=None, ws=None, wsb=0):
    L = F.lib()
    return L.falcon_chunk_fwd(ctypes.byref(shape) if shape is not None else None, q, k, v, beta, g,
                              ctypes.byref(init) if init else None, ctypes.byref(final) if final else None,
                              o, cs, ws, wsb, None)


def call_step(shape, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, state=None, o=FAKE):
    L = F.lib()
    return L.falcon_recurrent_step(ctypes.byref(shape) if shape is not None else None, q, k, v, beta, g,
                                   ctypes.byref(state) if state else None, o, None)


def workspace(**kw):
    return F.lib().falcon_chunk_fwd_workspace(ctypes.byref(good_shape(**kw)))


def test_workspace_size():
    """The chunk-parallel path keeps one image per (sequence, system of rows) plus
    one carry block per sequence: the size is a multiple of 16 bytes, linear in
    B*H and, per sequence, affine in the number of systems (ceil(T/C) steps of C
    for one pair per step, ceil(T/(C/Bw)) for a window of Bw pairs).  Fp32 at
    d = 128, windows on chunks other than 64 and invalid shapes need none."""
    w1, w2, w3 = workspace(seqlen=100), workspace(seqlen=200), workspace(seqlen=300)   # 2, 4, 5 systems
    img = w3 - w2
    assert w1 > 0 and w1 % 16 == 0 and img > 0 and img % 16 == 0 and w2 - w1 == 2 * img
    assert workspace(batch=4) == 2 * w1
    assert workspace(variant="F1A") < w1                    # no Gram / T blocks
    assert workspace(variant="F3", window=1) == w1          # a one-pair window is Falcon-1
    assert workspace(dk=128, dv=128) > w1                   # d = 128 (bf16): larger carry block only
    assert workspace(dk=128, dv=128) - w1 < img
    assert workspace(dtype="fp32", dk=128, dv=128) == 0
    assert workspace(batch=0) == 0 and workspace(dk=48, dv=48) == 0
    # windows: systems of 64 / Bw steps
    f4 = [workspace(variant="F3", window=4, seqlen=t) for t in (100, 116, 132)]   # 7, 8, 9 systems
    assert f4[0] > 0 and f4[1] - f4[0] == f4[2] - f4[1] > 0
    assert workspace(variant="F3A", window=4) < f4[0]       # no Gram / T blocks
    w8 = [workspace(variant="F3", window=8, seqlen=t) for t in (100, 108)]       # 13, 14 systems
    assert w8[1] - w8[0] == f4[1] - f4[0]                   # same image size: one 16-row score block
    assert workspace(variant="F3", window=4, chunk=32) == 0   # the windowed kernel, no scratch


@cpu_only
def test_workspace_too_small_or_misaligned():
    need = workspace()
    assert call_fwd(good_shape(), ws=FAKE, wsb=need - 16) == F.ERR_WORKSPACE
    assert call_fwd(good_shape(), ws=ctypes.c_void_p(0x10008), wsb=need) == F.ERR_INVALID_ARG


INVALID_SHAPES = [
    dict(variant=0), dict(variant=7), dict(dtype=2), dict(batch=0), dict(seqlen=0), dict(heads=0),
    dict(dk=0), dict(chunk=0), dict(window=0), dict(variant="F1", window=2),
    dict(eps_gamma=0.0), dict(eps_gamma=1.5), dict(eps_gamma=float("nan")), dict(eps_phi=-1.0),
    dict(eps_eta=0.0), dict(eps_eta=float("inf")), dict(align=2), dict(align=-1),
]
UNSUPPORTED_SHAPES = [
    dict(dk=48, dv=48), dict(dk=64, dv=32), dict(dk=256, dv=256), dict(chunk=8), dict(chunk=128),
    dict(dtype="fp32", dk=128, dv=128), dict(variant="F3", window=3), dict(variant="F3", window=16),
    dict(align="same", variant="F3", window=4, chunk=32),   # same-step pairs: chunk-parallel kernels only
]


@cpu_only
@pytest.mark.parametrize("kw", INVALID_SHAPES)
def test_invalid_shape(kw):
    assert call_fwd(good_shape(**kw)) == F.ERR_INVALID_ARG
    if "seqlen" not in kw and "chunk" not in kw:
        assert call_step(good_shape(**kw), state=F.State(FAKE.value, FAKE.value, None, None)) == F.ERR_INVALID_ARG


@cpu_only
@pytest.mark.parametrize("kw", UNSUPPORTED_SHAPES)
def test_unsupported_shape(kw):
    assert call_fwd(good_shape(**kw)) == F.ERR_UNSUPPORTED


@cpu_only
def test_null_shape_and_pointers():
    assert call_fwd(None) == F.ERR_INVALID_ARG
    for name in ("q", "k", "v", "beta", "g", "o"):
        assert call_fwd(good_shape(), **{name: None}) == F.ERR_INVALID_ARG, name
    assert call_step(good_shape(), state=None) == F.ERR_INVALID_ARG


@cpu_only
def test_misaligned_pointers():
    bad = ctypes.c_void_p(0x10004)
    for name in ("q", "k", "v", "o", "beta"):
        assert call_fwd(good_shape(), **{name: bad}) == F.ERR_INVALID_ARG, name
    assert call_fwd(good_shape(), g=ctypes.c_void_p(0x10002)) == F.ERR_INVALID_ARG
    assert call_fwd(good_shape(), cs=bad) == F.ERR_INVALID_ARG


@cpu_only
def test_incomplete_states():
    half = F.State(FAKE.value, None, None, None)
    assert call_fwd(good_shape(), init=half) == F.ERR_INVALID_ARG
    assert call_fwd(good_shape(), final=half) == F.ERR_INVALID_ARG
    no_window = F.State(FAKE.value, FAKE.value, None, None)
    sh = good_shape(variant="F3", window=4)
    assert call_fwd(sh, init=no_window) == F.ERR_INVALID_ARG
    assert call_step(sh, state=no_window) == F.ERR_INVALID_ARG
    assert call_step(good_shape(), state=F.State(FAKE.value, 0x10008, None, None)) == F.ERR_INVALID_ARG


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(F, "_LIB", None)
    monkeypatch.setattr(F, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        F.lib()


def call_varlen(shape, cu=FAKE, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, init=None, final=None, o=FAKE,
                ws=None, wsb=0):
    L = F.lib()
    return L.falcon_chunk_fwd_varlen(ctypes.byref(shape) if shape is not None else None, cu, q, k, v, beta, g,
                                     ctypes.byref(init) if init else None, ctypes.byref(final) if final else None,
                                     o, ws, wsb, None)


def varlen_workspace(**kw):
    return F.lib().falcon_chunk_fwd_varlen_workspace(ctypes.byref(good_shape(**kw)))


@cpu_only
def test_varlen_rejects_on_host():
    """Packed-sequence calls: the offsets pointer must be present and 4-byte aligned;
    shapes without a one-pass kernel are unsupported; all before any HIP call."""
    assert call_varlen(good_shape(seqlen=500), cu=None) == F.ERR_INVALID_ARG
    assert call_varlen(good_shape(seqlen=500), cu=ctypes.c_void_p(0x10002)) == F.ERR_INVALID_ARG
    assert call_varlen(good_shape(seqlen=500), q=None) == F.ERR_INVALID_ARG
    assert call_varlen(good_shape(seqlen=500, batch=0)) == F.ERR_INVALID_ARG
    # no one-pass kernel and no chunk-parallel path either
    assert call_varlen(good_shape(seqlen=500, dtype="fp32", dk=64, dv=64, chunk=64)) == F.ERR_UNSUPPORTED
    assert call_varlen(good_shape(seqlen=500, variant="F3", window=4, chunk=32)) == F.ERR_UNSUPPORTED
    # bf16 d = 128: only the chunk-parallel path, which needs the workspace
    assert call_varlen(good_shape(seqlen=500, dk=128, dv=128)) == F.ERR_WORKSPACE
    need = varlen_workspace(seqlen=500, dk=128, dv=128)
    assert need > 0
    assert call_varlen(good_shape(seqlen=500, dk=128, dv=128), ws=FAKE, wsb=need - 1) == F.ERR_WORKSPACE
    assert call_varlen(good_shape(seqlen=500, dk=128, dv=128), ws=ctypes.c_void_p(0x10008), wsb=need) == \
        F.ERR_INVALID_ARG


def test_varlen_workspace_size():
    """Per head, one image slot per system the packed sequences can have (at most
    total/C + N + 1), plus one carried-state block per sequence and head."""
    one = varlen_workspace(batch=1, seqlen=64, heads=1)
    assert one > 0
    # N sequences of total tokens: slots grow with total / C + N
    a = varlen_workspace(batch=4, seqlen=1000, heads=3)
    b = varlen_workspace(batch=8, seqlen=1000, heads=3)
    c = varlen_workspace(batch=4, seqlen=2000, heads=3)
    assert a < b and a < c
    assert varlen_workspace(batch=4, seqlen=1000, heads=3, dtype="fp32", dk=64, dv=64, chunk=64) == 0
    # at least the dense layout's size for equal-length sequences (that layout is packed tight)
    assert varlen_workspace(batch=4, seqlen=4 * 256, heads=3) >= workspace(batch=4, seqlen=256, heads=3)


def bwd_workspace(**kw):
    return F.lib().falcon_chunk_bwd_workspace(ctypes.byref(good_shape(**kw)))


def call_bwd(shape, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, init=None, cs=FAKE, do=FAKE, dST=None,
             dq=FAKE, dk=FAKE, dv=FAKE, dbeta=FAKE, dg=FAKE, d_init=None, ws=FAKE, wsb=1 << 40):
    L = F.lib()
    return L.falcon_chunk_bwd(ctypes.byref(shape) if shape is not None else None, q, k, v, beta, g,
                              ctypes.byref(init) if init else None, cs, do, dST, dq, dk, dv, dbeta, dg,
                              ctypes.byref(d_init) if d_init else None, ws, wsb, None)


def test_bwd_workspace_size():
    """Per chunk of 64 steps: the chunk's transition of the reverse recurrence,
    the injected state gradient and the end-of-chunk state gradient (3 x 64 x 64
    fp32) plus the chunk's decay; F1, F1A and F2A at d = 64, chunk 64 only."""
    per_chunk = 3 * 64 * 64 * 4 + 4
    assert bwd_workspace(seqlen=64, batch=1, heads=1) == per_chunk
    assert bwd_workspace(seqlen=100) == 2 * 3 * 2 * per_chunk
    assert bwd_workspace(seqlen=129, variant="F1A", dtype="fp32") == 2 * 3 * 3 * per_chunk
    assert bwd_workspace(seqlen=100, variant="F2A") == 2 * 3 * 2 * per_chunk
    # Falcon-2: keys, A, Zc, G and the per-channel steps (5 x 64 x 64), (c, e^{Lm}) and the decay
    assert bwd_workspace(seqlen=100, variant="F2") == 2 * 3 * 2 * (5 * 64 * 64 + 2 * 64 + 1) * 4
    for kw in (dict(dtype="fp32", dk=128, dv=128), dict(dk=64, dv=32), dict(batch=0)):
        assert bwd_workspace(**kw) == 0, kw
    # the kernels work in 64-step chunks whatever the forward's chunk
    assert bwd_workspace(seqlen=100, chunk=32) == bwd_workspace(seqlen=100, chunk=16) == 2 * 3 * 2 * per_chunk
    # a window of one pair is Falcon-1 / 1A
    assert bwd_workspace(variant="F3") == bwd_workspace(variant="F1")
    assert bwd_workspace(variant="F3A") == bwd_workspace(variant="F1A")


def test_bwd_rows_workspace_size():
    """The recurrent-form backward (windows, head dims 32 and 128): per workgroup
    of 16 value rows, for every token the row sums dqh and dx (d each) and two
    scalars, then d floats per carried window pair of each sequence."""
    bth, bh = 2 * 100 * 3, 2 * 3
    for kw, d, bw in ((dict(variant="F3", window=2), 64, 2), (dict(variant="F3A", window=8), 64, 8),
                      (dict(dk=32, dv=32), 32, 1), (dict(dk=128, dv=128, variant="F2"), 128, 1),
                      (dict(dk=128, dv=128, variant="F3", window=4, chunk=16), 128, 4)):
        assert bwd_workspace(**kw) == (d // 16) * (bth * (2 * d + 2) + bh * (bw - 1) * d) * 4, kw


@cpu_only
def test_bwd_rejects_on_host():
    ok = good_shape()
    assert call_bwd(None) == F.ERR_INVALID_ARG
    for kw in INVALID_SHAPES:
        assert call_bwd(good_shape(**kw)) == F.ERR_INVALID_ARG, kw
    for name in ("q", "k", "v", "beta", "g", "cs", "do", "dq", "dk", "dv", "dbeta", "dg", "ws"):
        assert call_bwd(ok, **{name: None}) == F.ERR_INVALID_ARG, name
    for name in ("q", "k", "v", "do", "cs", "dq", "dk", "dv", "dST", "ws"):
        assert call_bwd(ok, **{name: ctypes.c_void_p(0x10008)}) == F.ERR_INVALID_ARG, name
    for name in ("g", "dbeta", "dg"):
        assert call_bwd(ok, **{name: ctypes.c_void_p(0x10002)}) == F.ERR_INVALID_ARG, name
    assert call_bwd(ok, d_init=F.State(FAKE.value, None, None, None)) == F.ERR_INVALID_ARG
    assert call_bwd(ok, init=F.State(None, FAKE.value, None, None)) == F.ERR_INVALID_ARG
    for kw in (dict(dtype="fp32", dk=128, dv=128), dict(dk=64, dv=32)):
        assert call_bwd(good_shape(**kw)) == F.ERR_UNSUPPORTED, kw
    win = good_shape(variant="F3", window=4)
    assert call_bwd(win, wsb=bwd_workspace(variant="F3", window=4) - 1) == F.ERR_WORKSPACE
    # a window's carried state comes with its pairs
    assert call_bwd(win, init=F.State(FAKE.value, FAKE.value, None, None)) == F.ERR_INVALID_ARG
    assert call_bwd(ok, wsb=bwd_workspace() - 1) == F.ERR_WORKSPACE


def seg_workspace(nseg, **kw):
    return F.lib().falcon_chunk_fwd_segmented_workspace(ctypes.byref(good_shape(**kw)), nseg)


def call_seg(shape, nseg, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=FAKE, init=None, final=None, o=FAKE, ws=FAKE,
             wsb=1 << 40):
    L = F.lib()
    return L.falcon_chunk_fwd_segmented(ctypes.byref(shape) if shape is not None else None, nseg, q, k, v, beta,
                                        g, ctypes.byref(init) if init else None,
                                        ctypes.byref(final) if final else None, o, ws, wsb, None)


def test_segmented_workspace_size():
    """Built where the two-kernel path is, for nseg dividing T with segments of
    at least Bw steps, except F2; grows with the segment count (per-segment states)."""
    w1 = seg_workspace(1, seqlen=512)
    w4 = seg_workspace(4, seqlen=512)
    assert w1 > 0 and w4 > w1 and w4 % 256 == 0
    assert seg_workspace(3, seqlen=512) == 0                       # 3 does not divide 512
    assert seg_workspace(0, seqlen=512) == 0
    assert seg_workspace(4, seqlen=512, variant="F2") == 0         # per-row maps
    assert seg_workspace(4, seqlen=512, variant="F2A") > 0
    assert seg_workspace(4, seqlen=512, variant="F3", window=4) > 0
    assert seg_workspace(128, seqlen=256, variant="F3", window=4) == 0   # segments of 2 < Bw steps
    assert seg_workspace(4, seqlen=512, dtype="fp32", dk=128, dv=128) == 0   # no two-kernel path


@cpu_only
def test_segmented_rejects_on_host():
    ok = good_shape(seqlen=512)
    assert call_seg(None, 4) == F.ERR_INVALID_ARG
    assert call_seg(ok, 0) == F.ERR_INVALID_ARG
    assert call_seg(ok, 3) == F.ERR_INVALID_ARG
    assert call_seg(ok, 4, ws=None) == F.ERR_INVALID_ARG
    assert call_seg(ok, 4, ws=ctypes.c_void_p(0x10008)) == F.ERR_INVALID_ARG
    assert call_seg(ok, 4, o=None) == F.ERR_INVALID_ARG
    assert call_seg(good_shape(seqlen=512, variant="F2"), 4) == F.ERR_UNSUPPORTED
    assert call_seg(ok, 4, wsb=seg_workspace(4, seqlen=512) - 1) == F.ERR_WORKSPACE
    for kw in INVALID_SHAPES:
        assert call_seg(good_shape(**kw), 1) == F.ERR_INVALID_ARG, kw


def _cpu_state(B=2, H=3, dk=64, dv=64, window=1, dtype=None, drop=()):
    import torch
    dt = dtype or torch.float32
    st = dict(S=torch.zeros(B, H, dv, dk, dtype=dt), x_prev=torch.zeros(B, H, dk, dtype=dt))
    if window > 1:
        st["win_x"] = torch.zeros(B, H, window - 1, dk, dtype=dt)
        st["win_v"] = torch.zeros(B, H, window - 1, dv, dtype=dt)
    for k in drop:
        st.pop(k)
    return st


def test_binding_checks_state_shapes():
    """The binding passes raw state pointers, so it checks every state array's
    shape, dtype and presence before the call (the device check comes last, so
    on a CPU tensor of the right shape only the device is refused)."""
    import torch
    dev = torch.device("cuda:0")
    chk = F._check_state
    with pytest.raises(ValueError, match="must live on"):
        chk("init", _cpu_state(), 2, 3, 64, 64, 1, dev)               # right shapes, wrong device
    with pytest.raises(ValueError, match="shape"):
        chk("init", _cpu_state(B=1), 2, 3, 64, 64, 1, dev)            # another batch
    with pytest.raises(ValueError, match="shape"):
        chk("init", _cpu_state(H=4), 2, 3, 64, 64, 1, dev)            # another head count
    with pytest.raises(ValueError, match="shape"):
        chk("init", _cpu_state(dk=32, dv=32), 2, 3, 64, 64, 1, dev)   # another head dim
    with pytest.raises(TypeError, match="dtype"):
        chk("init", _cpu_state(dtype=torch.float64), 2, 3, 64, 64, 1, dev)
    with pytest.raises(ValueError, match="needs 'win_x'"):
        chk("final", _cpu_state(window=4, drop=("win_x",)), 2, 3, 64, 64, 4, dev)
    with pytest.raises(ValueError, match="shape"):
        chk("final", _cpu_state(window=2), 2, 3, 64, 64, 4, dev)      # a window built for Bw = 2
    with pytest.raises(ValueError, match="contiguous|shape"):
        st = _cpu_state()
        st["S"] = torch.zeros(2, 3, 64, 64).transpose(2, 3)
        chk("init", st, 2, 3, 64, 64, 1, dev)
    with pytest.raises(TypeError, match="state dict"):
        chk("init", [1, 2], 2, 3, 64, 64, 1, dev)


def test_bench_reference_counts():
    """bench.py's algorithmic bytes and reference flops reproduce the
    configurations' roofline table (bytes of inputs, outputs and final state; the
    chunked form's fixed flop formula, per WY system of C/Bw steps for Falcon-3)."""
    import bench
    import workloads as W
    c2, c3, c4, c5 = (W.WORKLOADS[n] for n in ("layer130m", "layer130m_f2", "window_t4096", "long_t65536"))
    assert bench.alg_bytes(c2, "F1") / 1e6 == pytest.approx(103.83, abs=0.01)
    assert bench.alg_bytes(c3, "F2") / 1e6 == pytest.approx(153.38, abs=0.01)
    assert bench.alg_bytes(c5, "F1") / 1e6 == pytest.approx(1083.19, abs=0.01)
    assert bench.ref_flops(c2, "F1") / 1e9 == pytest.approx(13.15, abs=0.01)
    assert bench.ref_flops(c2, "F1A") / 1e9 == pytest.approx(6.44, abs=0.01)
    assert bench.ref_flops(c3, "F2") / 1e9 == pytest.approx(10.47, abs=0.01)
    assert bench.ref_flops(c4, "F3", 4) / 1e9 == pytest.approx(38.12, abs=0.01)
    assert bench.ref_flops(c4, "F3", 8) / 1e9 == pytest.approx(71.40, abs=0.01)
    assert bench.ref_flops(c4, "F3A", 4) / 1e9 == pytest.approx(6.44, abs=0.01)
    assert bench.ref_flops(c4, "F3A", 8) == bench.ref_flops(c4, "F3A", 4)
    assert bench.ref_flops(c5, "F1") / 1e9 == pytest.approx(190.41, abs=0.01)
    assert bench.ref_flops(c5, "F1A") / 1e9 == pytest.approx(103.08, abs=0.01)
    # Falcon-3 with one pair per step is Falcon-1
    assert bench.ref_flops(c4, "F3", 1) == bench.ref_flops(c4, "F1")
