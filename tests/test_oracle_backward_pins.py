"""Pins of the oracle's backward pass (reverse-time adjoint of the recurrence).

The expected values come from a different route: central finite differences of
the forward oracle, which is itself pinned against the masked-parallel form and
the closed forms in ``test_oracle_pins``.  The scalar is <do, o> + <dS_T, S_T>.
Directional derivatives along random directions cover every input at once
(a dropped term, a wrong sign or a transposed operand in any gradient moves
them); full element-wise differences on a tiny case check each entry.
"""

import numpy as np
import pytest

import oracle
import workloads as W

BWD_VARS = ("F1", "F1A", "F2", "F2A")
ALIGNS = ("prefix", "same")


def setup(variant, T=9, dk=4, dv=3, B=1, H=2, gates="floor5", seed=3, carry=True, window=1):
    w = W.WORKLOADS["tiny_fp32"].replace(batch=B, heads=H, seqlen=T, dk=dk, dv=dv, gates=gates)
    inp = {n: a.astype(np.float64) for n, a in W.make_inputs(w, variant, seed=seed).items()}
    st = W.make_state(w, seed + 1, window=window) if carry else None
    if st is not None:
        st = {n: a.astype(np.float64) for n, a in st.items()}
    cot = W.make_cotangents(w, seed + 2)
    return inp, st, cot


def scalar(variant, inp, st, cot, align, window=1):
    r = oracle.recurrent(variant, **inp, state=st, align=align, window=window)
    return float(np.sum(r["o"] * cot["do"]) + np.sum(r["S"] * cot["dS_T"]))


def grads(variant, inp, st, cot, align, window=1):
    return oracle.recurrent_backward(variant, **inp, do=cot["do"], state=st, dS_T=cot["dS_T"],
                                     align=align, window=window)


# The inputs and the name of their gradient.
WRT = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("log_lambda", "dg")]
WRT_STATE = [("S", "dS0"), ("x_prev", "dx_prev0")]


@pytest.mark.parametrize("variant", BWD_VARS)
@pytest.mark.parametrize("align", ALIGNS)
def test_directional_derivatives(variant, align):
    inp, st, cot = setup(variant)
    g = grads(variant, inp, st, cot, align)
    rng = np.random.default_rng(11)
    h = 1e-6
    for name, gname in WRT + WRT_STATE:
        src = st if name in ("S", "x_prev") else inp
        d = rng.standard_normal(src[name].shape)
        if name == "log_lambda":
            # keep clamped gates clamped and the others clear of the floor
            d = np.where(np.exp(src[name]) > 1e-3, d, 0.0)
        plus = {**src, name: src[name] + h * d}
        minus = {**src, name: src[name] - h * d}
        if src is st:
            fp = scalar(variant, inp, plus, cot, align)
            fm = scalar(variant, inp, minus, cot, align)
        else:
            fp = scalar(variant, plus, st, cot, align)
            fm = scalar(variant, minus, st, cot, align)
        fd = (fp - fm) / (2 * h)
        an = float(np.sum(g[gname] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("variant", BWD_VARS)
@pytest.mark.parametrize("align", ALIGNS)
def test_elementwise_differences(variant, align):
    inp, st, cot = setup(variant, T=5, dk=3, dv=2, H=1, gates="softplus")
    g = grads(variant, inp, st, cot, align)
    h = 1e-6
    for name, gname in WRT + WRT_STATE:
        src = st if name in ("S", "x_prev") else inp
        fd = np.zeros(src[name].shape)
        for idx in np.ndindex(src[name].shape):
            a = src[name].copy()
            a[idx] += h
            b = src[name].copy()
            b[idx] -= h
            if src is st:
                fd[idx] = (scalar(variant, inp, {**st, name: a}, cot, align)
                           - scalar(variant, inp, {**st, name: b}, cot, align)) / (2 * h)
            else:
                fd[idx] = (scalar(variant, {**inp, name: a}, st, cot, align)
                           - scalar(variant, {**inp, name: b}, st, cot, align)) / (2 * h)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("variant", BWD_VARS)
def test_clamped_decay_has_no_gate_gradient(variant):
    """Below the floor the decay is the constant eps_gamma ([P2] 正衰减钳制)."""
    inp, st, cot = setup(variant, gates="floor5", T=40, seed=7)
    clamped = np.exp(inp["log_lambda"]) <= 1e-3
    assert clamped.any()
    g = grads(variant, inp, st, cot, "prefix")
    assert np.all(g["dg"][clamped] == 0.0)
    assert np.all(g["dg"][~clamped] != 0.0)


def test_same_step_ignores_carried_key():
    """With the same-step pairing the carried x_prev is never read: zero gradient."""
    inp, st, cot = setup("F1")
    g = grads("F1", inp, st, cot, "same")
    assert np.all(g["dx_prev0"] == 0.0)


def test_prefix_last_key_has_no_gradient():
    """Under the prefix pairing k_T only feeds the outgoing x_prev (no gradient taken)."""
    inp, st, cot = setup("F1")
    g = grads("F1", inp, st, cot, "prefix")
    assert np.all(g["dk"][:, -1] == 0.0)


def test_additive_value_gradient_closed_form():
    """F1A at unit decay and unit key norm: o_t = sum_{s<=t} eta_s (x_s . qh_t) v_s, so
    dv_s = eta_s sum_{t>=s} (x_s . qh_t) do_t + eta_s dS_T x_s (linear attention's adjoint)."""
    inp, st, cot = setup("F1A", T=8, carry=False)
    inp["log_lambda"][:] = 0.0
    g = grads("F1A", inp, None, cot, "same")
    qh = oracle.phi(inp["q"])
    x = oracle.phi(inp["k"])
    eta = inp["beta"] / (1e-6 + np.sum(x * x, -1))
    B, T, H, _ = x.shape
    ref = np.zeros_like(inp["v"])
    for b in range(B):
        for hh in range(H):
            for s in range(T):
                acc = cot["dS_T"][b, hh] @ x[b, s, hh]
                for t in range(s, T):
                    acc = acc + (x[b, s, hh] @ qh[b, t, hh]) * cot["do"][b, t, hh]
                ref[b, s, hh] = eta[b, s, hh] * acc
    np.testing.assert_allclose(g["dv"], ref, rtol=1e-12, atol=1e-12)


# ---- windows (Falcon-3 / 3A) -------------------------------------------------------
# The same finite-difference routes, with the carried window among the inputs.
WIN_CASES = [("F3", 2), ("F3", 3), ("F3A", 2), ("F3A", 3)]
WRT_WIN = WRT_STATE + [("win_x", "dwin_x0"), ("win_v", "dwin_v0")]


@pytest.mark.parametrize("variant,window", WIN_CASES)
@pytest.mark.parametrize("align", ALIGNS)
def test_window_directional_derivatives(variant, window, align):
    inp, st, cot = setup(variant, window=window, T=11)
    g = grads(variant, inp, st, cot, align, window)
    rng = np.random.default_rng(17)
    h = 1e-6
    for name, gname in WRT + WRT_WIN:
        src = st if name in st else inp
        d = rng.standard_normal(src[name].shape)
        if name == "log_lambda":
            d = np.where(np.exp(src[name]) > 1e-3, d, 0.0)
        plus = {**src, name: src[name] + h * d}
        minus = {**src, name: src[name] - h * d}
        if src is st:
            fp = scalar(variant, inp, plus, cot, align, window)
            fm = scalar(variant, inp, minus, cot, align, window)
        else:
            fp = scalar(variant, plus, st, cot, align, window)
            fm = scalar(variant, minus, st, cot, align, window)
        fd = (fp - fm) / (2 * h)
        an = float(np.sum(g[gname] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("variant,window", [("F3", 3), ("F3A", 2)])
def test_window_elementwise_differences(variant, window):
    inp, st, cot = setup(variant, T=5, dk=3, dv=2, H=1, gates="softplus", window=window)
    g = grads(variant, inp, st, cot, "prefix", window)
    h = 1e-6
    for name, gname in WRT + WRT_WIN:
        src = st if name in st else inp
        fd = np.zeros(src[name].shape)
        for idx in np.ndindex(src[name].shape):
            a = src[name].copy()
            a[idx] += h
            b = src[name].copy()
            b[idx] -= h
            if src is st:
                fd[idx] = (scalar(variant, inp, {**st, name: a}, cot, "prefix", window)
                           - scalar(variant, inp, {**st, name: b}, cot, "prefix", window)) / (2 * h)
            else:
                fd[idx] = (scalar(variant, {**inp, name: a}, st, cot, "prefix", window)
                           - scalar(variant, {**inp, name: b}, st, cot, "prefix", window)) / (2 * h)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("base", ["F1", "F1A"])
def test_one_pair_window_is_falcon1(base):
    """A window of one pair is the one-pair step ([P1] Falcon家族): identical gradients."""
    inp, st, cot = setup(base, T=12)
    g1 = grads(base, inp, st, cot, "prefix")
    g3 = grads(base.replace("1", "3"), inp, st, cot, "prefix", 1)
    for key in g1:
        np.testing.assert_allclose(g3[key], g1[key], rtol=1e-13, atol=1e-14, err_msg=key)
