"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests re-calls the oracle's own arithmetic as the expected value:
each compares it with a different route to the same number (a whole-sequence
linear solve, a finite-difference gradient, a textbook closed form, a reduction
to another variant, an invariant).  Page keys [P1] [P2] [P3] as in ``oracle``.
"""

import math

import numpy as np
import pytest

import oracle
import workloads as W

VARS = oracle.VARIANTS


def small(T=13, dk=5, dv=3, B=2, H=2, gates="uniform", seed=0, variant="F1"):
    w = W.WORKLOADS["tiny_fp32"].replace(batch=B, heads=H, seqlen=T, dk=dk, dv=dv, gates=gates)
    return w, W.make_inputs(w, variant, seed=seed)


def windows_for(v):
    return (1, 2, 4) if v in ("F3", "F3A") else (1,)


def unit(a, eps=1e-6):
    a = np.asarray(a, np.float64)
    return a / np.sqrt((a * a).sum(-1, keepdims=True) + eps)


CASES = [(v, bw) for v in VARS for bw in windows_for(v)]


# -- P1: recurrent == masked-parallel ([P1] 三种等价形式, Fig. 4; [P2] 三种视角) -------
@pytest.mark.parametrize("variant,bw", CASES)
@pytest.mark.parametrize("carry", [False, True])
def test_p1_recurrent_equals_masked_parallel(variant, bw, carry):
    w, inp = small(T=17, variant=variant, gates="softplus")
    st = W.make_state(w, 3, bw) if carry else None
    r = oracle.recurrent(variant, **inp, window=bw, state=st)
    m = oracle.masked_parallel(variant, **inp, window=bw, state=st)
    for key in ("o", "S", "x_prev") + (("win_x", "win_v") if bw > 1 else ()):
        np.testing.assert_allclose(r[key], m[key], rtol=0, atol=1e-12, err_msg=key)


# -- P2: F1A at lam = 1 is denominator-free causal linear attention ([P1] 三种等价形式)
def test_p2_f1a_is_linear_attention():
    w, inp = small(T=11, dk=4, dv=3, variant="F1A")
    inp["log_lambda"][:] = 0.0
    r = oracle.recurrent("F1A", **inp)
    qh, kh = unit(inp["q"]), unit(inp["k"])
    B, T, H, _ = qh.shape
    ref = np.zeros(r["o"].shape)
    for b in range(B):
        for h in range(H):
            # strict-causal attention on the original keys, values shifted by one step
            for t in range(T):
                for i in range(t):
                    eta = inp["beta"][b, i + 1, h] / (1e-6 + kh[b, i, h] @ kh[b, i, h])
                    ref[b, t, h] += (qh[b, t, h] @ kh[b, i, h]) * eta * inp["v"][b, i + 1, h]
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


def test_p2_f1a_with_decay_is_decayed_linear_attention():
    w, inp = small(T=9, dk=4, dv=3, variant="F1A")
    r = oracle.recurrent("F1A", **inp)
    qh, kh = unit(inp["q"]), unit(inp["k"])
    lam = np.exp(inp["log_lambda"].astype(np.float64))
    B, T, H, _ = qh.shape
    ref = np.zeros(r["o"].shape)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                for j in range(1, t + 1):             # pair j = (phi(k_{j-1}), v_j)
                    decay = np.prod(lam[b, j + 1:t + 1, h])
                    x = kh[b, j - 1, h]
                    eta = inp["beta"][b, j, h] / (1e-6 + x @ x)
                    ref[b, t, h] += decay * (qh[b, t, h] @ x) * eta * inp["v"][b, j, h]
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


# -- P3: Falcon-3 with a window of one pair is Falcon-1 ([P1] Falcon家族; [P2] 六个变体)
@pytest.mark.parametrize("pair", [("F3", "F1"), ("F3A", "F1A")])
def test_p3_window_one_reduces(pair):
    w, inp = small(T=15, variant="F1")
    st = W.make_state(w, 4, 1)
    a = oracle.recurrent(pair[0], **inp, window=1, state=st)
    b = oracle.recurrent(pair[1], **inp, window=1, state=st)
    np.testing.assert_allclose(a["o"], b["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a["S"], b["S"], rtol=0, atol=1e-14)


# -- P4: window average keeps the write magnitude independent of B ([P2] 六个变体) --
@pytest.mark.parametrize("bw", [2, 3, 5, 8])
@pytest.mark.parametrize("pair", [("F3", "F1"), ("F3A", "F1A")])
def test_p4_identical_pairs_any_window(bw, pair):
    w, inp = small(T=10, dk=4, dv=3, variant="F1")
    inp["k"][:] = inp["k"][:, :1]             # every key the same
    inp["v"][:] = inp["v"][:, :1]             # every value the same
    x0 = unit(inp["k"][:, 0])                 # [B,H,dk]
    S0 = W.make_state(w, 6, 1)["S"]
    st1 = dict(S=S0, x_prev=x0)
    stw = dict(S=S0, x_prev=x0,
               win_x=np.repeat(x0[:, :, None], bw - 1, axis=2),
               win_v=np.repeat(inp["v"][:, 0][:, :, None], bw - 1, axis=2))
    a = oracle.recurrent(pair[0], **inp, window=bw, state=stw)
    b = oracle.recurrent(pair[1], **inp, window=1, state=st1)
    np.testing.assert_allclose(a["o"], b["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["S"], b["S"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("bw", [2, 4, 8])
def test_p4_write_bounded_by_largest_pair(bw):
    """|S_t - lam_t S_{t-1}|_F <= eta_t max_j |e_j| |x_j| for random windows: an
    average, never a sum, of the window's rank-one writes."""
    w, inp = small(T=12, dk=6, dv=4, variant="F3")
    st = W.make_state(w, 8, bw)
    r = oracle.recurrent("F3", **inp, window=bw, state=st, return_states=True)
    S = r["states"]
    lam = np.maximum(np.exp(inp["log_lambda"].astype(np.float64)), 1e-3)
    kh = unit(inp["k"])
    B, T, H = lam.shape
    ratio_max = 0.0
    for b in range(B):
        for h in range(H):
            pairs_x = list(st["win_x"][b, h].astype(np.float64))
            pairs_v = list(st["win_v"][b, h].astype(np.float64))
            Sprev = st["S"][b, h].astype(np.float64)
            xp = st["x_prev"][b, h].astype(np.float64)
            for t in range(T):
                x = xp
                pairs_x.append(x)
                pairs_v.append(inp["v"][b, t, h].astype(np.float64))
                wx, wv = pairs_x[-bw:], pairs_v[-bw:]
                eta = inp["beta"][b, t, h] / (1e-6 + x @ x)
                bound = eta * max(np.linalg.norm(vj - Sprev @ xj) * np.linalg.norm(xj)
                                  for xj, vj in zip(wx, wv))
                delta = np.linalg.norm(S[b, t, h] - lam[b, t, h] * Sprev)
                assert delta <= bound * (1 + 1e-12)
                ratio_max = max(ratio_max, delta / bound)
                Sprev = S[b, t, h]
                xp = kh[b, t, h]
    assert ratio_max > 0.05      # the bound is not vacuous


# -- P5: each step is one gradient step on the instantaneous ridge loss, and the
# loss does not increase for an admissible step ([P2] 梯度下降) -----------------------
def _loss(variant, S, xs, vs, rho):
    """Instantaneous loss at the state S for the window pairs (xs, vs).
    Regression: mean_j 1/2 |v_j - S x_j|^2; inner product: -mean_j <v_j, S x_j>;
    plus the ridge term rho/2 |S|^2 (rho may be per row for F2/F2A).
    Returned per row of S (value channel) so F2's per-channel steps can be used."""
    per_row = np.zeros(S.shape[0])
    for xj, vj in zip(xs, vs):
        pred = np.array([sum(S[i, c] * xj[c] for c in range(S.shape[1])) for i in range(S.shape[0])])
        if variant in ("F1", "F2", "F3"):
            per_row += 0.5 * (vj - pred) ** 2 / len(xs)
        else:
            per_row += -(vj * pred) / len(xs)
    return per_row + 0.5 * rho * np.sum(S * S, axis=1)


@pytest.mark.parametrize("variant,bw", CASES)
def test_p5_step_is_gradient_step(variant, bw):
    w, inp = small(T=4, dk=4, dv=3, B=1, H=1, variant=variant)
    st = W.make_state(w, 11, bw)
    r = oracle.recurrent(variant, **inp, window=bw, state=st, return_states=True)
    kh = unit(inp["k"])
    pairs_x = list(st["win_x"][0, 0].astype(np.float64)) if bw > 1 else []
    pairs_v = list(st["win_v"][0, 0].astype(np.float64)) if bw > 1 else []
    Sprev = st["S"][0, 0].astype(np.float64)
    xp = st["x_prev"][0, 0].astype(np.float64)
    h = 1e-5
    for t in range(4):
        x = xp
        pairs_x.append(x)
        pairs_v.append(inp["v"][0, t, 0].astype(np.float64))
        xs, vs = pairs_x[-bw:], pairs_v[-bw:]
        lam = max(math.exp(float(inp["log_lambda"][0, t, 0])), 1e-3)
        beta = np.asarray(inp["beta"][0, t, 0], np.float64)
        eta = beta / (1e-6 + x @ x) * np.ones(Sprev.shape[0])     # per row
        rho = (1 - lam) / eta
        grad = np.zeros_like(Sprev)
        for i in range(Sprev.shape[0]):
            for c in range(Sprev.shape[1]):
                Sp, Sm = Sprev.copy(), Sprev.copy()
                Sp[i, c] += h
                Sm[i, c] -= h
                grad[i, c] = (_loss(variant, Sp, xs, vs, rho)[i] - _loss(variant, Sm, xs, vs, rho)[i]) / (2 * h)
        expect = Sprev - eta[:, None] * grad
        np.testing.assert_allclose(r["states"][0, t, 0], expect, rtol=0, atol=1e-8)
        # A gradient step on a quadratic decreases it when eta * lambda_max(Hessian) <= 2;
        # the Hessian is mean_j x_j x_j^T + rho I.
        hess_top = np.linalg.eigvalsh(sum(np.outer(xj, xj) for xj in xs) / len(xs))[-1]
        if variant in ("F1", "F2", "F3") and np.all(eta * (hess_top + rho) <= 2):
            assert np.all(_loss(variant, r["states"][0, t, 0], xs, vs, rho)
                          <= _loss(variant, Sprev, xs, vs, rho) + 1e-12)
        Sprev = r["states"][0, t, 0]
        xp = kh[0, t, 0]


def test_p5_unit_decay_loss_contracts_exactly():
    """At lam = 1, l(S_t) = (1 - eta |x|^2)^2 l(S_{t-1}) for l = 1/2 |v_t - S x_t|^2."""
    w, inp = small(T=8, dk=5, dv=3, variant="F1")
    inp["log_lambda"][:] = 0.0
    st = W.make_state(w, 12, 1)
    r = oracle.recurrent("F1", **inp, state=st, return_states=True)
    kh = unit(inp["k"])
    for b in range(2):
        for h in range(2):
            Sprev = st["S"][b, h].astype(np.float64)
            x = st["x_prev"][b, h].astype(np.float64)
            for t in range(8):
                vt = inp["v"][b, t, h]
                eta = inp["beta"][b, t, h] / (1e-6 + x @ x)
                before = 0.5 * np.sum((vt - Sprev @ x) ** 2)
                after = 0.5 * np.sum((vt - r["states"][b, t, h] @ x) ** 2)
                assert after == pytest.approx((1 - eta * (x @ x)) ** 2 * before, rel=1e-10, abs=1e-14)
                Sprev, x = r["states"][b, t, h], kh[b, t, h]


# -- P6: delta-rule storage closed forms ([P1] Falcon家族; [P2] 梯度下降, NLMS) ------
def test_p6_repeated_pair():
    w, inp = small(T=9, dk=4, dv=3, variant="F1")
    inp["log_lambda"][:] = 0.0
    inp["k"][:] = inp["k"][:, :1]
    inp["v"][:] = inp["v"][:, :1]
    inp["beta"][:] = inp["beta"][:, :1]
    x = unit(inp["k"][:, 0])
    st = dict(S=np.zeros((2, 2, 3, 4)), x_prev=x)
    r = oracle.recurrent("F1", **inp, state=st)
    a = inp["beta"][:, 0] * np.sum(x * x, -1) / (1e-6 + np.sum(x * x, -1))    # eta |x|^2
    n = 9
    got = np.einsum("bhij,bhj->bhi", r["S"], x)
    expect = (1 - (1 - a) ** n)[..., None] * inp["v"][:, 0]
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-13)


def test_p6_orthonormal_keys():
    """With orthonormal keys every residual equals its value, so F1 == F1A and
    S_T x_j = eta_j prod_{s>j} lam_s v_j."""
    dk, T = 8, 7
    w, inp = small(T=T, dk=dk, dv=3, B=1, H=1, variant="F1")
    Qm, _ = np.linalg.qr(np.random.default_rng(1).standard_normal((dk, dk)))
    inp["k"] = Qm[None, :T, None, :]                       # k_0..k_{T-1}: orthonormal rows
    xs = np.concatenate([Qm[T:T + 1], Qm[:T - 1]])         # pair keys x_j = phi(k_{j-1}), x_0 carried
    st = dict(S=np.zeros((1, 1, 3, dk)), x_prev=Qm[None, None, T])
    a = oracle.recurrent("F1", **inp, state=st, eps_phi=0.0, eps_eta=0.0)
    b = oracle.recurrent("F1A", **inp, state=st, eps_phi=0.0, eps_eta=0.0)
    np.testing.assert_allclose(a["o"], b["o"], rtol=0, atol=1e-14)
    lam = np.exp(inp["log_lambda"][0, :, 0].astype(np.float64))
    for j in range(T):
        got = a["S"][0, 0] @ xs[j]
        expect = inp["beta"][0, j, 0] * np.prod(lam[j + 1:]) * inp["v"][0, j, 0]
        np.testing.assert_allclose(got, expect, rtol=0, atol=1e-14)


# -- P7: per-channel step reductions ([P1] Falcon家族; [P2] 六个变体) ---------------
def test_p7_f2_equal_channels_is_f1():
    w, inp = small(T=14, dk=5, dv=4, variant="F1")
    st = W.make_state(w, 2, 1)
    a = oracle.recurrent("F1", **inp, state=st)
    inp2 = dict(inp, beta=np.repeat(inp["beta"][..., None], 4, axis=-1))
    b = oracle.recurrent("F2", **inp2, state=st)
    np.testing.assert_allclose(a["o"], b["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a["S"], b["S"], rtol=0, atol=1e-14)


def test_p7_f2a_is_f1a_with_scaled_values():
    w, inp = small(T=14, dk=5, dv=4, variant="F2A")
    st = W.make_state(w, 2, 1)
    a = oracle.recurrent("F2A", **inp, state=st)
    inp2 = dict(inp, v=inp["v"].astype(np.float64) * inp["beta"], beta=np.ones(inp["log_lambda"].shape))
    b = oracle.recurrent("F1A", **inp2, state=st)
    np.testing.assert_allclose(a["o"], b["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a["S"], b["S"], rtol=0, atol=1e-13)


# -- P8: chunk-size invariance, split continuation, decode x T ([P1] 三种等价形式) ---
@pytest.mark.parametrize("variant,bw", CASES)
def test_p8_chunk_invariance(variant, bw):
    w, inp = small(T=19, variant=variant, gates="softplus")
    st = W.make_state(w, 5, bw)
    ref = oracle.recurrent(variant, **inp, window=bw, state=st)
    for C in (1, 2, 3, 7, 16, 19, 40):
        c = oracle.chunked(variant, **inp, window=bw, state=st, chunk=C)
        np.testing.assert_allclose(c["o"], ref["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(c["S"], ref["S"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant,bw", CASES)
def test_p8_split_continuation(variant, bw):
    w, inp = small(T=16, variant=variant)
    whole = oracle.recurrent(variant, **inp, window=bw)
    first = oracle.recurrent(variant, **{n: a[:, :7] for n, a in inp.items()}, window=bw)
    st = {n: first[n] for n in ("S", "x_prev", "win_x", "win_v") if n in first}
    second = oracle.masked_parallel(variant, **{n: a[:, 7:] for n, a in inp.items()}, window=bw, state=st)
    np.testing.assert_allclose(np.concatenate([first["o"], second["o"]], 1), whole["o"], rtol=0, atol=1e-12)
    for key in st:
        np.testing.assert_allclose(second[key], whole[key], rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant,bw", CASES)
def test_p8_decode_steps(variant, bw):
    w, inp = small(T=9, variant=variant)
    st0 = W.make_state(w, 7, bw)
    whole = oracle.recurrent(variant, **inp, window=bw, state=st0)
    st = st0
    for t in range(9):
        r = oracle.decode_step(variant, *(inp[n][:, t] for n in ("q", "k", "v", "beta", "log_lambda")),
                               state=st, window=bw)
        np.testing.assert_allclose(r["o"], whole["o"][:, t], rtol=0, atol=1e-13)
        st = {n: r[n] for n in ("S", "x_prev", "win_x", "win_v") if n in r}
    np.testing.assert_allclose(st["S"], whole["S"], rtol=0, atol=1e-13)


# -- P9: positive-decay clamp ([P1] 三种等价形式; [P2] 正衰减钳制) ------------------
@pytest.mark.parametrize("variant", VARS)
def test_p9_clamp(variant):
    w, inp = small(T=10, variant=variant)
    outs = []
    for g in (-np.inf, -50.0, math.log(1e-3) - 1.0, math.log(1e-3)):
        x = dict(inp)
        x["log_lambda"] = inp["log_lambda"].astype(np.float64).copy()
        x["log_lambda"][:, 3:6] = g
        outs.append(oracle.recurrent(variant, **x, window=1))
    for o in outs[1:3]:
        np.testing.assert_array_equal(o["o"], outs[0]["o"])
    np.testing.assert_allclose(outs[3]["o"], outs[0]["o"], rtol=1e-14, atol=1e-15)
    # above the floor the decay is not touched
    y = dict(inp)
    y["log_lambda"] = inp["log_lambda"].astype(np.float64).copy()
    y["log_lambda"][:, 3:6] = math.log(2e-3)
    assert not np.allclose(oracle.recurrent(variant, **y)["o"], outs[0]["o"])


def test_p9_floor_value():
    """Below the floor the state decays by exactly eps_gamma per step."""
    w, inp = small(T=3, dk=4, dv=3, variant="F1A")
    inp["beta"][:] = 0.0
    inp["log_lambda"][:] = -np.inf
    st = W.make_state(w, 3, 1)
    r = oracle.recurrent("F1A", **inp, state=st)
    np.testing.assert_allclose(r["S"], st["S"].astype(np.float64) * 1e-9, rtol=1e-14)


# -- P10: a fresh sequence by hand ([P1] 本质; [P2] 一个被忽略的时间差) ------------------
@pytest.mark.parametrize("variant", VARS)
def test_p10_fresh_sequence_by_hand(variant):
    bw = 3 if variant in ("F3", "F3A") else 1
    w, inp = small(T=2, dk=4, dv=3, B=1, H=1, variant=variant)
    r = oracle.recurrent(variant, **inp, window=bw, return_states=True)
    assert np.all(r["o"][0, 0, 0] == 0.0)             # x_1 = 0: nothing written, nothing read
    assert np.all(r["states"][0, 0, 0] == 0.0)
    k1 = inp["k"][0, 0, 0].astype(np.float64)
    x2 = k1 / math.sqrt(float(k1 @ k1) + 1e-6)
    q2 = inp["q"][0, 1, 0].astype(np.float64)
    qh2 = q2 / math.sqrt(float(q2 @ q2) + 1e-6)
    beta2 = np.asarray(inp["beta"][0, 1, 0], np.float64)
    eta2 = beta2 / (1e-6 + x2 @ x2)
    v2 = inp["v"][0, 1, 0].astype(np.float64)
    S2 = (eta2 * v2)[:, None] * x2[None, :] / bw      # S_1 = 0; window pairs before t=1 are zero
    np.testing.assert_allclose(r["states"][0, 1, 0], S2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["o"][0, 1, 0], (x2 @ qh2) * eta2 * v2 / bw, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r["x_prev"][0, 0], unit(inp["k"][0, 1, 0]), rtol=1e-15)


# -- P11: same-step alignment, the pages' contrast to the prefix pair ([P1] 本质;
# [P2] 一个被忽略的时间差): x_t = phi(k_t) ------------------------------------------------
@pytest.mark.parametrize("variant,bw", CASES)
@pytest.mark.parametrize("carry", [False, True])
def test_p11_same_step_recurrent_equals_masked_parallel(variant, bw, carry):
    w, inp = small(T=17, variant=variant, gates="softplus")
    st = W.make_state(w, 3, bw) if carry else None
    r = oracle.recurrent(variant, **inp, window=bw, state=st, align="same")
    m = oracle.masked_parallel(variant, **inp, window=bw, state=st, align="same")
    for key in ("o", "S", "x_prev") + (("win_x", "win_v") if bw > 1 else ()):
        np.testing.assert_allclose(r[key], m[key], rtol=0, atol=1e-12, err_msg=key)


@pytest.mark.parametrize("variant,bw", CASES)
def test_p11_same_step_is_prefix_on_keys_one_step_ahead(variant, bw):
    """Writing (phi(k_t), v_t) at step t is the prefix rule fed the keys one step
    ahead (k'_{t-1} = k_t), with phi(k_1) as the carried feature."""
    w, inp = small(T=15, variant=variant, gates="softplus")
    st = W.make_state(w, 4, bw)
    same = oracle.recurrent(variant, **inp, window=bw, state=st, align="same")
    shifted = dict(inp)
    k = np.asarray(inp["k"])
    shifted["k"] = np.concatenate([k[:, 1:], k[:, -1:]], axis=1)   # the last key only feeds x_prev
    st2 = dict(st)
    st2["x_prev"] = unit(k[:, 0])
    pre = oracle.recurrent(variant, **shifted, window=bw, state=st2)
    np.testing.assert_allclose(same["o"], pre["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(same["S"], pre["S"], rtol=0, atol=1e-12)
    if bw > 1:
        np.testing.assert_allclose(same["win_x"], pre["win_x"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(same["win_v"], pre["win_v"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant", VARS)
def test_p11_same_step_first_write_by_hand(variant):
    bw = 3 if variant in ("F3", "F3A") else 1
    w, inp = small(T=1, dk=4, dv=3, B=1, H=1, variant=variant)
    r = oracle.recurrent(variant, **inp, window=bw, align="same")
    x1 = unit(inp["k"][0, 0, 0])
    qh1 = unit(inp["q"][0, 0, 0])
    beta1 = np.asarray(inp["beta"][0, 0, 0], np.float64)
    eta1 = beta1 / (1e-6 + x1 @ x1)
    v1 = inp["v"][0, 0, 0].astype(np.float64)
    S1 = (eta1 * v1)[:, None] * x1[None, :] / bw       # from S_0 = 0 the decay has nothing to act on
    np.testing.assert_allclose(r["S"][0, 0], S1, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["o"][0, 0, 0], S1 @ qh1, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("variant,bw", CASES)
def test_p11_same_step_chunk_invariance(variant, bw):
    w, inp = small(T=19, variant=variant, gates="softplus")
    st = W.make_state(w, 5, bw)
    ref = oracle.recurrent(variant, **inp, window=bw, state=st, align="same")
    for C in (1, 3, 16, 40):
        c = oracle.chunked(variant, **inp, window=bw, state=st, chunk=C, align="same")
        np.testing.assert_allclose(c["o"], ref["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(c["S"], ref["S"], rtol=0, atol=1e-12)
