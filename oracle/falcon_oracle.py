"""Plain fp64 oracle of Falcon fast-weight attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP path.

What is computed (page keys [P1] [P2] [P3] are defined in ``oracle/__init__``):

* Prefix alignment -- [P1] 本质, [P2] 一个被忽略的时间差, [P3] 核心方法: the
  training pair written at step t is (phi(k_{t-1}), v_t); the read at step t
  happens after that write.  x_t = phi(k_{t-1}); for a fresh sequence x_1 = 0.
* One online gradient step on an instantaneous loss -- [P2] 梯度下降: for the
  regression family the loss is the ridge loss of the state used as a linear
  predictor of v_t from x_t; one step at S_{t-1} gives
      S_t = lam_t S_{t-1} + eta_t (v_t - S_{t-1} x_t) x_t^T
  with the residual taken against the un-decayed S_{t-1}.
* NLMS step -- [P1] Falcon家族, [P2] 梯度下降: eta_t = beta_t / (eps_eta + |x_t|^2).
* Family -- [P1] Falcon家族, [P2] 六个变体:
    F1  scalar eta_t;  F2  per-value-channel eta_t (a vector over rows of S);
    F3  residuals of the last B_w pairs, each against the same S_{t-1},
        averaged (divided by B_w, not summed);
    F1A/F2A/F3A  inner-product objective: the write is additive, v_t x_t^T
        (no residual), with the same alignment and the same step.
* Positive-decay clamp -- [P1] 三种等价形式, [P2] 正衰减钳制:
  lam_t = max(exp(g_t), eps_gamma) for the input log-decay g_t.
* Read -- o_t = S_t phi(q_t) (read after write), phi(a) = a / sqrt(|a|^2 + eps_phi).
* Same-step alignment (``align="same"``) -- the contrast the pages draw against
  prefix alignment ([P1] 本质, [P2] 一个被忽略的时间差): the pair written at step t
  is (phi(k_t), v_t), i.e. x_t = phi(k_t); the carried x_prev is not read, and
  window pairs are (phi(k_j), v_j).  The outgoing x_prev is phi(k_T) either way.

Readings where the pages are silent (also listed in the design notes):
  R3 x_1 = 0 for a fresh sequence (o_1 = 0); a continued sequence passes x_prev.
  R4/R5 eps_phi = eps_eta = 1e-6.
  R6 floor only, lam <= 1 assumed.
  R8 F3 residuals against the current S_{t-1}.
  R9 F3 pairs before the sequence start are zero (or the carried window); the
     divisor stays B_w.
  R10 F3 uses the newest key's eta_t for the whole window.
  R11 F2 keeps a scalar decay; only eta is per channel.

Array conventions: q, k [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H] (or [B,T,H,dv] for
F2/F2A); log_lambda [B,T,H]; S [B,H,dv,dk] (row i = value channel i); x_prev
[B,H,dk]; win_x [B,H,Bw-1,dk] and win_v [B,H,Bw-1,dv], oldest first.
"""

from __future__ import annotations

import numpy as np

VARIANTS = ("F1", "F1A", "F2", "F2A", "F3", "F3A")
_DELTA = ("F1", "F2", "F3")          # regression family: residual-driven write
_VECTOR_ETA = ("F2", "F2A")
_WINDOWED = ("F3", "F3A")


def phi(a, eps_phi=1e-6):
    """L2-normalised identity feature map, [P1] 三种等价形式 (phi on Q and K)."""
    a = np.asarray(a, dtype=np.float64)
    return a / np.sqrt(np.sum(a * a, axis=-1, keepdims=True) + eps_phi)


ALIGNS = ("prefix", "same")


def _check(variant, window, align="prefix"):
    if align not in ALIGNS:
        raise ValueError(f"unknown alignment {align!r}")
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if window < 1:
        raise ValueError("window must be >= 1")
    if variant not in _WINDOWED and window != 1:
        raise ValueError("window > 1 only for F3/F3A")


def _to_seq(a):
    """[B,T,H,...] -> [B*H, T, ...] float64."""
    a = np.asarray(a, dtype=np.float64)
    B, T, H = a.shape[:3]
    return np.moveaxis(a, 2, 1).reshape((B * H, T) + a.shape[3:])


def _from_seq(a, B, H):
    """[B*H, T, ...] -> [B,T,H,...]."""
    T = a.shape[1]
    return np.moveaxis(a.reshape((B, H, T) + a.shape[2:]), 1, 2)


def _initial(state, N, B, H, dk, dv, window):
    S = np.zeros((N, dv, dk))
    xp = np.zeros((N, dk))
    wx = np.zeros((N, window - 1, dk))
    wv = np.zeros((N, window - 1, dv))
    if state is not None:
        if state.get("S") is not None:
            S = np.asarray(state["S"], np.float64).reshape(N, dv, dk).copy()
        if state.get("x_prev") is not None:
            xp = np.asarray(state["x_prev"], np.float64).reshape(N, dk).copy()
        if window > 1 and state.get("win_x") is not None:
            wx = np.asarray(state["win_x"], np.float64).reshape(N, window - 1, dk).copy()
            wv = np.asarray(state["win_v"], np.float64).reshape(N, window - 1, dv).copy()
    return S, xp, wx, wv


def _step(variant, window, S, x, v, beta, g, qh, wx, wv, eps_gamma, eps_eta):
    """One step of the recurrent form for all N sequences at once.

    S [N,dv,dk], x [N,dk] (= phi(k_{t-1})), v [N,dv], beta [N] or [N,dv], g [N],
    qh [N,dk] (= phi(q_t)), wx/wv the carried window (oldest first).
    Returns the new S and the output o_t = S_t qh."""
    lam = np.maximum(np.exp(g), eps_gamma)                 # positive-decay clamp
    energy = np.sum(x * x, axis=-1)                        # |x_t|^2
    if variant in _VECTOR_ETA:
        eta = beta / (eps_eta + energy)[:, None]           # [N,dv]   NLMS, per channel
    else:
        eta = beta / (eps_eta + energy)                    # [N]      NLMS, scalar
    if variant in _WINDOWED:
        keys = np.concatenate([wx, x[:, None, :]], axis=1)        # [N,Bw,dk], pairs t-Bw+1..t
        vals = np.concatenate([wv, v[:, None, :]], axis=1)        # [N,Bw,dv]
        if variant == "F3":
            resid = vals - np.einsum("nij,nbj->nbi", S, keys)     # v_j - S_{t-1} x_j
        else:
            resid = vals
        write = np.einsum("nbi,nbj->nij", resid, keys) * (eta / window)[:, None, None]
    else:
        if variant in ("F1", "F2"):
            resid = v - np.einsum("nij,nj->ni", S, x)             # v_t - S_{t-1} x_t
        else:
            resid = v
        if variant in _VECTOR_ETA:
            write = (eta * resid)[:, :, None] * x[:, None, :]     # diag(eta) r x^T
        else:
            write = (eta[:, None] * resid)[:, :, None] * x[:, None, :]
    S = lam[:, None, None] * S + write
    o = np.einsum("nij,nj->ni", S, qh)                            # read after write
    return S, o


def recurrent(variant, q, k, v, beta, log_lambda, *, window=1, state=None,
              eps_gamma=1e-3, eps_phi=1e-6, eps_eta=1e-6, return_states=False, align="prefix"):
    """Recurrent form, one step at a time ([P1] 三种等价形式 form A; [P2] 三种视角).

    Returns dict(o [B,T,H,dv], S, x_prev, win_x, win_v) and, if requested,
    ``states`` [B,T,H,dv,dk] = S_t after every step."""
    _check(variant, window, align)
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = B * H
    Q, K, V = _to_seq(q), _to_seq(k), _to_seq(v)
    Bt, G = _to_seq(beta), _to_seq(log_lambda)
    S, xp, wx, wv = _initial(state, N, B, H, dk, dv, window)
    O = np.zeros((N, T, dv))
    states = np.zeros((N, T, dv, dk)) if return_states else None
    for t in range(T):
        x = xp if align == "prefix" else phi(K[:, t], eps_phi)
        S, O[:, t] = _step(variant, window, S, x, V[:, t], Bt[:, t], G[:, t],
                           phi(Q[:, t], eps_phi), wx, wv, eps_gamma, eps_eta)
        if states is not None:
            states[:, t] = S
        if window > 1:
            wx = np.concatenate([wx[:, 1:], x[:, None]], axis=1)
            wv = np.concatenate([wv[:, 1:], V[:, t][:, None]], axis=1)
        xp = phi(K[:, t], eps_phi)
    out = dict(o=_from_seq(O, B, H), S=S.reshape(B, H, dv, dk), x_prev=xp.reshape(B, H, dk))
    if window > 1:
        out["win_x"] = wx.reshape(B, H, window - 1, dk)
        out["win_v"] = wv.reshape(B, H, window - 1, dv)
    if states is not None:
        out["states"] = _from_seq(states, B, H)
    return out


def decode_step(variant, q, k, v, beta, log_lambda, state, *, window=1,
                eps_gamma=1e-3, eps_phi=1e-6, eps_eta=1e-6, align="prefix"):
    """One token of the recurrent form for a batch of sequences.

    q, k [B,H,dk], v [B,H,dv], beta [B,H] or [B,H,dv], log_lambda [B,H];
    ``state`` holds S, x_prev (and the window for F3/F3A).  Returns o [B,H,dv]
    and the new state (x_prev becomes phi(k))."""
    ins = [np.asarray(a)[:, None] for a in (q, k, v, beta, log_lambda)]
    r = recurrent(variant, *ins, window=window, state=state, eps_gamma=eps_gamma, align=align,
                  eps_phi=eps_phi, eps_eta=eps_eta)
    r["o"] = r["o"][:, 0]
    return r


# ---------------------------------------------------------------------------
# Masked-parallel form: the whole sequence as one lower-triangular linear system
# ([P1] 三种等价形式 form B and Figure 4-B "WY representation + TriSolve";
# [P2] 三种视角).  Built from the unrolled recurrence, with numpy.linalg.solve
# doing the triangular solve; independent of the step loop above.
# ---------------------------------------------------------------------------

def _pairs_for_sequence(X, V, wx, wv, window):
    """Key/value of every pair index j = -(Bw-1) .. T-1 (carried window first)."""
    return np.concatenate([wx, X], axis=0), np.concatenate([wv, V], axis=0)


def _masked_parallel_one(variant, window, Qh, X, V, beta, g, S0, wx, wv,
                         eps_gamma, eps_eta):
    """One sequence.  Qh, X [T,dk]; V [T,dv]; beta [T] or [T,dv]; g [T].

    Virtual rows r = (s, j): step s in 0..T-1 and pair j in s-Bw+1..s
    (Bw = 1 for F1/F2/F1A/F2A, so r = s).  Unrolling the recurrence from S0:
      S_s   = e^{L_s} S0 + sum_{r: s(r) <= s} e^{L_s - L_{s(r)}} w_r e_r x_{j(r)}^T
      e_r   = v_{j(r)} - S_{s(r)-1} x_{j(r)}                 (regression family)
            = v_{j(r)}                                        (A variants)
    so the residuals solve (I + A diag(w)) E = V_r - diag(e^{L_{s-1}}) X_r S0^T with
      A[r, r'] = e^{L_{s(r)-1} - L_{s(r')}} <x_{j(r)}, x_{j(r')}>  for s(r') < s(r).
    L is the inclusive cumulative sum of log(lam); L_{-1} = 0."""
    T, dk = X.shape
    dv = V.shape[1]
    lam = np.maximum(np.exp(g), eps_gamma)
    L = np.cumsum(np.log(lam))
    Lprev = L - np.log(lam)
    energy = np.sum(X * X, axis=1)
    eta = beta / (eps_eta + energy)[:, None] if beta.ndim == 2 else beta / (eps_eta + energy)
    Bw = window
    PX, PV = _pairs_for_sequence(X, V, wx, wv, Bw)          # pair j lives at index j + Bw - 1
    steps = np.repeat(np.arange(T), Bw)                      # s(r)
    pj = (np.arange(T)[:, None] + np.arange(-Bw + 1, 1)[None, :]).reshape(-1)   # j(r)
    Xr = PX[pj + Bw - 1]
    Vr = PV[pj + Bw - 1]
    R = len(steps)
    if eta.ndim == 2:
        w = eta[steps] / Bw                                  # [R, dv]
    else:
        w = eta[steps] / Bw                                  # [R]
    earlier = steps[None, :] < steps[:, None]                # s(r') < s(r)
    A = np.where(earlier, np.exp(Lprev[steps][:, None] - L[steps][None, :]) * (Xr @ Xr.T), 0.0)
    rhs = Vr - np.exp(Lprev[steps])[:, None] * (Xr @ S0.T)
    if variant in _DELTA:
        if w.ndim == 2:                                      # F2: one solve per value channel
            E = np.empty((R, dv))
            for c in range(dv):
                E[:, c] = np.linalg.solve(np.eye(R) + A * w[None, :, c], rhs[:, c])
        else:
            E = np.linalg.solve(np.eye(R) + A * w[None, :], rhs)
    else:
        E = Vr.copy()
    WE = E * (w if w.ndim == 2 else w[:, None])              # w_r e_r
    upto = steps[None, :] <= np.arange(T)[:, None]           # s(r) <= s
    D = np.where(upto, np.exp(L[:, None] - L[steps][None, :]), 0.0)
    O = np.exp(L)[:, None] * (Qh @ S0.T) + (D * (Qh @ Xr.T)) @ WE
    ST = np.exp(L[-1]) * S0 + (np.exp(L[-1] - L[steps])[:, None] * WE).T @ Xr
    return O, ST, PX, PV


def masked_parallel(variant, q, k, v, beta, log_lambda, *, window=1, state=None,
                    eps_gamma=1e-3, eps_phi=1e-6, eps_eta=1e-6, align="prefix"):
    """Masked-parallel form over the whole sequence (quadratic; small T only)."""
    _check(variant, window, align)
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = B * H
    Qh = phi(_to_seq(q), eps_phi)
    Kf = phi(_to_seq(k), eps_phi)
    V, Bt, G = _to_seq(v), _to_seq(beta), _to_seq(log_lambda)
    S, xp, wx, wv = _initial(state, N, B, H, dk, dv, window)
    O = np.zeros((N, T, dv))
    ST = np.zeros((N, dv, dk))
    nwx = np.zeros_like(wx)
    nwv = np.zeros_like(wv)
    for n in range(N):
        if align == "prefix":
            X = np.concatenate([xp[n][None], Kf[n, :-1]], axis=0)  # x_t = phi(k_{t-1})
        else:
            X = Kf[n]                                               # x_t = phi(k_t)
        O[n], ST[n], PX, PV = _masked_parallel_one(variant, window, Qh[n], X, V[n], Bt[n], G[n],
                                                   S[n], wx[n], wv[n], eps_gamma, eps_eta)
        if window > 1:
            nwx[n] = PX[-(window - 1):]
            nwv[n] = PV[-(window - 1):]
    out = dict(o=_from_seq(O, B, H), S=ST.reshape(B, H, dv, dk),
               x_prev=Kf[:, -1].reshape(B, H, dk))
    if window > 1:
        out["win_x"] = nwx.reshape(B, H, window - 1, dk)
        out["win_v"] = nwv.reshape(B, H, window - 1, dv)
    return out


def chunked(variant, q, k, v, beta, log_lambda, *, chunk, window=1, state=None,
            eps_gamma=1e-3, eps_phi=1e-6, eps_eta=1e-6, align="prefix"):
    """Chunked form ([P1] 三种等价形式 form C, [P2] 三种视角): the masked-parallel
    form applied chunk by chunk, with the state (S, x_prev, window) handed from
    one chunk to the next.  chunk = 1 is the recurrent form, chunk >= T the
    masked-parallel form."""
    T = np.asarray(q).shape[1]
    st = None if state is None else dict(state)
    outs = []
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(T, c0 + chunk))
        r = masked_parallel(variant, q[:, sl], k[:, sl], v[:, sl], beta[:, sl],
                            log_lambda[:, sl], window=window, state=st, align=align,
                            eps_gamma=eps_gamma, eps_phi=eps_phi, eps_eta=eps_eta)
        outs.append(r["o"])
        st = {n: r[n] for n in ("S", "x_prev", "win_x", "win_v") if n in r}
    res = dict(st)
    res["o"] = np.concatenate(outs, axis=1)
    return res


_BACKWARD_VARIANTS = VARIANTS


def _phi_backward(a, da, eps_phi):
    """Adjoint of phi(a) = a / n, n = sqrt(|a|^2 + eps_phi): J^T da = da/n - a (a.da)/n^3."""
    n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True) + eps_phi)
    return da / n - a * np.sum(a * da, axis=-1, keepdims=True) / n ** 3


def recurrent_backward(variant, q, k, v, beta, log_lambda, do, *, window=1, state=None, dS_T=None,
                       eps_gamma=1e-3, eps_phi=1e-6, eps_eta=1e-6, align="prefix"):
    """Gradients of the recurrent form by reverse-time accumulation (the adjoint of
    the step written out), for the chunked form's use in training ([P1] 三种等价形式:
    the chunk-parallel form is the one a training framework runs).

    The scalar being differentiated is <do, o> + <dS_T, S_T> for the forward of
    :func:`recurrent` from ``state`` (S, x_prev; zeros when absent).  The outgoing
    x_prev takes no gradient.  Differentiation conventions (readings):
      * lam = max(exp(g), eps_gamma): dg = dlam * lam where exp(g) > eps_gamma,
        else 0 (at the floor the decay does not depend on g);
      * eta = beta / (eps_eta + |x|^2) depends on x through |x|^2;
      * phi is differentiated as written (with eps_phi inside the root).

    Per step t, going backwards, with G the gradient of the scalar w.r.t. S_t:
        G += do_t qh_t^T;  dqh_t = S_t^T do_t;  dlam_t = <G, S_{t-1}>;  u = G x_t
        regression (F1/F2): e = v_t - S_{t-1} x_t, deta = e * u, dv_t = eta * u,
            dx_t = G^T (eta e) - S_{t-1}^T (eta u),  G <- lam G - (eta u) x_t^T
        additive (F1A/F2A): e = v_t, same deta/dv_t, dx_t = G^T (eta v_t),  G <- lam G
    (``eta * u`` is a scalar times a vector for F1/F1A and elementwise for F2/F2A.)
    Windows (F3/F3A, [P1] Falcon家族, [P2] 六个变体): the step writes the B_w pairs
    j of its window with weight w = eta_t / B_w, so every pair j gets
        u_j = G x_j,  e_j = v_j - S_{t-1} x_j (F3) or v_j (F3A),  dv_j += w u_j,
        dx_j += w (G^T e_j - S_{t-1}^T u_j) (the second term F3 only),
    deta_t = sum_j <e_j, u_j> / B_w and G <- lam G - w sum_j u_j x_j^T (F3) or lam G;
    pairs before the sequence start are the carried window, whose gradients are
    dwin_x0 / dwin_v0.
    Then dx_t gains -2 x_t sum(deta * eta)/(eps_eta + |x_t|^2), dbeta_t = deta/(eps_eta + |x_t|^2),
    and dx_t flows through phi to k_{t-1} (prefix; x_1 of the prefix form is the
    carried x_prev, so its gradient is dx_prev0) or to k_t (same step).

    Returns dict(dq, dk, dv [B,T,H,d], dbeta (shape of beta), dg [B,T,H],
    dS0 [B,H,dv,dk], dx_prev0 [B,H,dk]) and, for windows of B_w > 1,
    dwin_x0 [B,H,B_w-1,dk] and dwin_v0 [B,H,B_w-1,dv]."""
    _check(variant, window, align)
    if variant not in _BACKWARD_VARIANTS:
        raise ValueError(f"no backward for {variant}")
    if variant in _WINDOWED:
        return _window_backward(variant, q, k, v, beta, log_lambda, do, window=window, state=state,
                                dS_T=dS_T, eps_gamma=eps_gamma, eps_phi=eps_phi, eps_eta=eps_eta,
                                align=align)
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = B * H
    Q, K, V = _to_seq(q), _to_seq(k), _to_seq(v)
    Bt, G_in, dO = _to_seq(beta), _to_seq(log_lambda), _to_seq(do)
    S0, xp0, _, _ = _initial(state, N, B, H, dk, dv, 1)
    delta = variant in _DELTA
    vector = variant in _VECTOR_ETA

    # Forward pass, keeping every state and every x_t.
    fwd = recurrent(variant, q, k, v, beta, log_lambda, state=state, eps_gamma=eps_gamma,
                    eps_phi=eps_phi, eps_eta=eps_eta, return_states=True, align=align)
    states = _to_seq(fwd["states"])                                     # [N,T,dv,dk], S_t
    Kh = phi(K, eps_phi)
    Qh = phi(Q, eps_phi)
    if align == "prefix":
        X = np.concatenate([xp0[:, None, :], Kh[:, :-1]], axis=1)      # x_t = phi(k_{t-1})
    else:
        X = Kh.copy()

    dQh = np.zeros_like(Qh)
    dX = np.zeros_like(X)
    dV = np.zeros_like(V)
    dBt = np.zeros_like(Bt)
    dGl = np.zeros((N, T))
    G = np.zeros((N, dv, dk)) if dS_T is None else np.asarray(dS_T, np.float64).reshape(N, dv, dk).copy()
    for t in range(T - 1, -1, -1):
        S_prev = states[:, t - 1] if t > 0 else S0
        S_t = states[:, t]
        x = X[:, t]
        energy = eps_eta + np.sum(x * x, axis=-1)                       # [N]
        b = Bt[:, t]
        eta = b / energy[:, None] if vector else b / energy              # [N,dv] or [N]
        lam = np.maximum(np.exp(G_in[:, t]), eps_gamma)
        G = G + dO[:, t][:, :, None] * Qh[:, t][:, None, :]
        dQh[:, t] = np.einsum("nij,ni->nj", S_t, dO[:, t])
        dlam = np.einsum("nij,nij->n", G, S_prev)
        u = np.einsum("nij,nj->ni", G, x)                               # G x_t
        e = V[:, t] - np.einsum("nij,nj->ni", S_prev, x) if delta else V[:, t]
        eta_v = eta if vector else eta[:, None]                          # broadcast over rows
        deta_rows = e * u                                                # per value channel
        dV[:, t] = eta_v * u
        dx = np.einsum("nij,ni->nj", G, eta_v * e)
        if delta:
            dx = dx - np.einsum("nij,ni->nj", S_prev, eta_v * u)
            G = lam[:, None, None] * G - (eta_v * u)[:, :, None] * x[:, None, :]
        else:
            G = lam[:, None, None] * G
        if vector:
            deta = deta_rows                                             # [N,dv]
            dBt[:, t] = deta / energy[:, None]
            denergy = -np.sum(deta * eta, axis=-1) / energy
        else:
            deta = np.sum(deta_rows, axis=-1)                            # [N]
            dBt[:, t] = deta / energy
            denergy = -deta * eta / energy
        dX[:, t] = dx + 2.0 * denergy[:, None] * x
        dGl[:, t] = np.where(np.exp(G_in[:, t]) > eps_gamma, dlam * lam, 0.0)

    dQ = _phi_backward(Q, dQh, eps_phi)
    dK = np.zeros_like(K)
    dxp0 = np.zeros((N, dk))
    if align == "prefix":
        dK[:, :-1] = _phi_backward(K[:, :-1], dX[:, 1:], eps_phi)
        dxp0 = dX[:, 0]
    else:
        dK = _phi_backward(K, dX, eps_phi)
    out = dict(dq=_from_seq(dQ, B, H), dk=_from_seq(dK, B, H), dv=_from_seq(dV, B, H),
               dbeta=_from_seq(dBt, B, H), dg=_from_seq(dGl, B, H),
               dS0=G.reshape(B, H, dv, dk), dx_prev0=dxp0.reshape(B, H, dk))
    return out


def _window_backward(variant, q, k, v, beta, log_lambda, do, *, window, state, dS_T, eps_gamma,
                     eps_phi, eps_eta, align):
    """recurrent_backward for F3/F3A: the reverse-time adjoint of the window step
    (see there), one step at a time."""
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = B * H
    Bw = window
    Q, K, V = _to_seq(q), _to_seq(k), _to_seq(v)
    Bt, G_in, dO = _to_seq(beta), _to_seq(log_lambda), _to_seq(do)
    S0, xp0, wx0, wv0 = _initial(state, N, B, H, dk, dv, Bw)
    fwd = recurrent(variant, q, k, v, beta, log_lambda, window=Bw, state=state, eps_gamma=eps_gamma,
                    eps_phi=eps_phi, eps_eta=eps_eta, return_states=True, align=align)
    states = _to_seq(fwd["states"])
    Kh = phi(K, eps_phi)
    Qh = phi(Q, eps_phi)
    if align == "prefix":
        X = np.concatenate([xp0[:, None, :], Kh[:, :-1]], axis=1)
    else:
        X = Kh.copy()
    # every pair of the sequence, the carried window first: pair j sits at j + Bw - 1
    XA = np.concatenate([wx0, X], axis=1)
    VA = np.concatenate([wv0, V], axis=1)
    dXA = np.zeros_like(XA)
    dVA = np.zeros_like(VA)
    dQh = np.zeros_like(Qh)
    dBt = np.zeros_like(Bt)
    dGl = np.zeros((N, T))
    G = np.zeros((N, dv, dk)) if dS_T is None else np.asarray(dS_T, np.float64).reshape(N, dv, dk).copy()
    for t in range(T - 1, -1, -1):
        S_prev = states[:, t - 1] if t > 0 else S0
        S_t = states[:, t]
        x = X[:, t]
        energy = eps_eta + np.sum(x * x, axis=-1)
        eta = Bt[:, t] / energy
        w = eta / Bw
        lam = np.maximum(np.exp(G_in[:, t]), eps_gamma)
        keys = XA[:, t:t + Bw]                                            # pairs t-Bw+1 .. t
        vals = VA[:, t:t + Bw]
        G = G + dO[:, t][:, :, None] * Qh[:, t][:, None, :]
        dQh[:, t] = np.einsum("nij,ni->nj", S_t, dO[:, t])
        dlam = np.einsum("nij,nij->n", G, S_prev)
        U = np.einsum("nij,nbj->nbi", G, keys)                            # G x_j
        if variant == "F3":
            E = vals - np.einsum("nij,nbj->nbi", S_prev, keys)            # v_j - S_{t-1} x_j
        else:
            E = vals
        dVA[:, t:t + Bw] += w[:, None, None] * U
        dXA[:, t:t + Bw] += w[:, None, None] * np.einsum("nij,nbi->nbj", G, E)
        if variant == "F3":
            dXA[:, t:t + Bw] -= w[:, None, None] * np.einsum("nij,nbi->nbj", S_prev, U)
            G = lam[:, None, None] * G - w[:, None, None] * np.einsum("nbi,nbj->nij", U, keys)
        else:
            G = lam[:, None, None] * G
        deta = np.sum(E * U, axis=(1, 2)) / Bw
        dBt[:, t] = deta / energy
        dXA[:, t + Bw - 1] += 2.0 * (-deta * eta / energy)[:, None] * x
        dGl[:, t] = np.where(np.exp(G_in[:, t]) > eps_gamma, dlam * lam, 0.0)

    dX = dXA[:, Bw - 1:]
    dQ = _phi_backward(Q, dQh, eps_phi)
    dK = np.zeros_like(K)
    dxp0 = np.zeros((N, dk))
    if align == "prefix":
        dK[:, :-1] = _phi_backward(K[:, :-1], dX[:, 1:], eps_phi)
        dxp0 = dX[:, 0]
    else:
        dK = _phi_backward(K, dX, eps_phi)
    out = dict(dq=_from_seq(dQ, B, H), dk=_from_seq(dK, B, H), dv=_from_seq(dVA[:, Bw - 1:], B, H),
               dbeta=_from_seq(dBt, B, H), dg=_from_seq(dGl, B, H),
               dS0=G.reshape(B, H, dv, dk), dx_prev0=dxp0.reshape(B, H, dk))
    if Bw > 1:
        out["dwin_x0"] = dXA[:, :Bw - 1].reshape(B, H, Bw - 1, dk)
        out["dwin_v0"] = dVA[:, :Bw - 1].reshape(B, H, Bw - 1, dv)
    return out
