"""CPU oracle of the scan's backward pass: plain, slow, fp64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module; the GPU library never
does, and it shares no code with the HIP kernels.

Sources (web pages, cited by title and section):

[D]   "Diagonal Equivalence in State Space Models: Characterization,
      Retrieval Rank, and Selective Extensions" (paperpeel.com).
      - Section 2.5 "Parallel scan and gradients": the adjoint (reverse)
        recurrence of an affine state update; the state sensitivity runs
        backward through the transposed transition, the transition's gradient
        pairs that sensitivity with the previous state, the initial state's
        gradient is the sensitivity left at the start, and a sensitivity that
        arrives for the final state (from a later segment) is added to the
        terminal condition.  Parameter and input gradients follow by the
        chain rule through the coefficient maps.
      - Section 5.5 and Appendix C.2: every carry (state, phase, previous
        write) is differentiable, so gradients flow through the initial and
        the final carry.
      - Appendix C.5: the angle gradient is the sensitive one (a reverse sum
        of phase sensitivities).
[M3]  "Mamba-3: Improved Sequence Modeling using State Space Principles"
      (intuitivepapers.ai explainer): the forward recurrence differentiated
      here (see ``ref.scan_seq``).

What is differentiated: ``ref.scan_seq``, token by token, for one scalar loss
    loss = sum(dy * y) + <dfinal.h, h_L> + <dfinal.phi, phi_L>
           + <dfinal.B_prev, B_prev_L> + <dfinal.x_prev, x_prev_L>
(the returned phase taken before its reduction into [0, 2 pi), whose
derivative is one).  The reverse sweep below is the plain adjoint of that
loop: it replays the forward recurrence storing every state, then walks back.
"""
import math

import numpy as np

from . import ref


def heavy_tail_rate_grad(u):
    """d A / d u of ``ref.heavy_tail_rate``: -1 for u >= 0, -1/(1-u)^2 for
    u < 0, and 0 where the clamp at -1e-4 holds."""
    u = np.asarray(u, dtype=np.float64)
    ht = np.where(u >= 0.0, 1.0 + u, 1.0 / (1.0 - np.minimum(u, 0.0)))
    d = np.where(u >= 0.0, 1.0, 1.0 / (1.0 - np.minimum(u, 0.0)) ** 2)
    return np.where(-ht < -1e-4, -d, 0.0)


def _rot_grad(dv, v_rot, phi):
    """Adjoint of v_rot = rot(v, phi) for one token: (d v, d phi).

    The transpose of a rotation by phi is the rotation by -phi; the angle's
    derivative of pair i is (-v_rot[2i+1], v_rot[2i]) (the rotated pair turned
    by a further quarter turn), summed over the leading (rank) axis.
    """
    npairs = np.shape(phi)[-1] if np.ndim(phi) else 0
    dv_in = ref.rot(dv, -np.asarray(phi)) if npairs else np.array(dv, dtype=np.float64)
    if npairs == 0:
        return dv_in, np.zeros(0)
    e, o = v_rot[..., 0:2 * npairs:2], v_rot[..., 1:2 * npairs:2]
    de, do = dv[..., 0:2 * npairs:2], dv[..., 1:2 * npairs:2]
    dphi = np.sum(-de * o + do * e, axis=tuple(range(np.ndim(dv) - 1)))
    return dv_in, dphi


def scan_bwd(inp, dy, dfinal=None):
    """Gradients of the loss above with respect to every input of the scan.

    inp: the dict of ``ref.scan_seq``; dy [b,L,H,R,P]; dfinal: dict with h
    [b,H,P,N], phi [b,H,np], B_prev [b,H,R,N], x_prev [b,H,R,P] (any may be
    None) or None.

    Returns a dict: x [b,L,H,R,P]; B, C [b,L,G,R,N] (summed over the heads of
    a group); dt, lam [b,L,H]; theta [b,L,H,np]; A_log [H] (static rate law)
    or A_raw [b,L,H] (per-token rates); B_bias, C_bias [H,R,N]; init (dict h,
    phi, B_prev, x_prev, as the carry).
    """
    b, L, H, G, R, P, N, npairs = ref._dims(inp)
    f64 = lambda a: None if a is None else np.asarray(a, dtype=np.float64)  # noqa: E731
    dy = f64(dy)
    dfinal = dfinal or {}
    heavy = inp.get("A_raw") is not None
    out = {"x": np.zeros((b, L, H, R, P)), "B": np.zeros((b, L, G, R, N)), "C": np.zeros((b, L, G, R, N)),
           "dt": np.zeros((b, L, H)), "lam": np.zeros((b, L, H)), "theta": np.zeros((b, L, H, npairs)),
           "B_bias": np.zeros((H, R, N)), "C_bias": np.zeros((H, R, N)),
           "init": {"h": np.zeros((b, H, P, N)), "phi": np.zeros((b, H, npairs)),
                    "B_prev": np.zeros((b, H, R, N)), "x_prev": np.zeros((b, H, R, P))}}
    if heavy:
        out["A_raw"] = np.zeros((b, L, H))
    else:
        out["A_log"] = np.zeros(H)
    for bi in range(b):
        for h in range(H):
            g = h * G // H
            s = ref._stream(inp, bi, h)
            a = s["a"]                                           # A_t = -a_t
            # forward replay, keeping every state, angle and turned B, C
            Hs = [s["H0"].copy()]
            phis, Bts, Cts = [], [], []
            alpha, beta, gamma = np.zeros(L), np.zeros(L), np.zeros(L)
            phi, Bp, Xp = s["phi0"].copy(), s["Bp0"].copy(), s["xp0"].copy()
            Xps, Bps = [], []
            for t in range(L):
                dt, lam = s["dt"][t], s["lam"][t]
                alpha[t] = math.exp(-dt * a[t])
                beta[t] = alpha[t] * dt * (1.0 - lam)
                gamma[t] = lam * dt
                phi = phi + dt * s["theta"][t]
                Bt, Ct = ref.rot(s["B"][t], phi), ref.rot(s["C"][t], phi)
                Xps.append(Xp)
                Bps.append(Bp)
                Hs.append(alpha[t] * Hs[-1] + beta[t] * (Xp.T @ Bp) + gamma[t] * (s["x"][t].T @ Bt))
                phis.append(phi.copy())
                Bts.append(Bt)
                Cts.append(Ct)
                Bp, Xp = Bt, s["x"][t]
            # terminal conditions: the final carry's sensitivities
            dfh = f64(dfinal.get("h"))
            Gs = dfh[bi, h].copy() if dfh is not None else np.zeros((P, N))   # d loss / d H_t
            dfp = f64(dfinal.get("phi"))
            Phi = dfp[bi, h].copy() if dfp is not None else np.zeros(npairs)  # d loss / d phi_t
            dfb, dfx = f64(dfinal.get("B_prev")), f64(dfinal.get("x_prev"))
            dB_next = dfb[bi, h].copy() if dfb is not None else np.zeros((R, N))  # d loss / d (B~_t) via later use
            dX_next = dfx[bi, h].copy() if dfx is not None else np.zeros((R, P))
            dA_sum = 0.0
            for t in range(L - 1, -1, -1):
                dt, lam, X = s["dt"][t], s["lam"][t], s["x"][t]
                Bt, Ct = Bts[t], Cts[t]
                # readout y_t[r] = H_t C~_t[r]
                Gs = Gs + dy[bi, t, h].T @ Ct                    # P x N: sum_r dy_r (x) C~_r
                dCt = dy[bi, t, h] @ Hs[t + 1]                   # R x N: H_t^T dy_r
                # update H_t = alpha H_{t-1} + beta Xp^T Bp + gamma X^T B~
                d_alpha = float(np.sum(Gs * Hs[t]))
                d_beta = float(np.sum(Gs * (Xps[t].T @ Bps[t])))
                d_gamma = float(np.sum(Gs * (X.T @ Bt)))
                dX = gamma[t] * (Bt @ Gs.T) + dX_next           # R x P
                dBt = gamma[t] * (X @ Gs) + dB_next             # R x N
                dX_next = beta[t] * (Bps[t] @ Gs.T)             # to the previous token (or the carry)
                dB_next = beta[t] * (Xps[t] @ Gs)
                Gs = alpha[t] * Gs
                # scalar maps: alpha = exp(-dt a), beta = alpha dt (1 - lam), gamma = lam dt
                d_alpha_tot = d_alpha + d_beta * dt * (1.0 - lam)
                d_dt = d_alpha_tot * alpha[t] * (-a[t]) + d_beta * alpha[t] * (1.0 - lam) + d_gamma * lam
                d_lam = -d_beta * alpha[t] * dt + d_gamma * dt
                d_A = d_alpha_tot * alpha[t] * dt                # d loss / d A_t (A_t = -a_t)
                # rotations of B and C by phi_t
                dBh, dphiB = _rot_grad(dBt, Bt, phis[t])
                dCh, dphiC = _rot_grad(dCt, Ct, phis[t])
                # phi_t = phi_{t-1} + dt theta_t: Phi collects d loss / d phi_t
                Phi = Phi + dphiB + dphiC
                if npairs:
                    out["theta"][bi, t, h] = dt * Phi
                    d_dt += float(np.dot(s["theta"][t], Phi))
                out["x"][bi, t, h] = dX
                out["B"][bi, t, g] += dBh
                out["C"][bi, t, g] += dCh
                out["B_bias"][h] += dBh
                out["C_bias"][h] += dCh
                out["dt"][bi, t, h] = d_dt
                out["lam"][bi, t, h] = d_lam
                if heavy:
                    out["A_raw"][bi, t, h] = d_A * float(heavy_tail_rate_grad(inp["A_raw"][bi, t, h]))
                else:
                    dA_sum += d_A
            if not heavy:
                # A = -exp(A_log): dA / dA_log = A
                out["A_log"][h] += dA_sum * (-math.exp(float(inp["A_log"][h])))
            out["init"]["h"][bi, h] = Gs
            out["init"]["phi"][bi, h] = Phi
            out["init"]["B_prev"][bi, h] = dB_next
            out["init"]["x_prev"][bi, h] = dX_next
    return out


def loss(inp, dy, dfinal=None):
    """The scalar differentiated by ``scan_bwd`` (used by its finite-difference
    pins): the unreduced final phase is phi0 + sum_t dt_t theta_t."""
    y, fin = ref.scan_seq(inp)
    v = float(np.sum(np.asarray(dy, np.float64) * y))
    if dfinal:
        b, L, H, G, R, P, N, npairs = ref._dims(inp)
        if dfinal.get("h") is not None:
            v += float(np.sum(np.asarray(dfinal["h"], np.float64) * fin["h"]))
        if dfinal.get("B_prev") is not None:
            v += float(np.sum(np.asarray(dfinal["B_prev"], np.float64) * fin["B_prev"]))
        if dfinal.get("x_prev") is not None:
            v += float(np.sum(np.asarray(dfinal["x_prev"], np.float64) * fin["x_prev"]))
        if dfinal.get("phi") is not None and npairs:
            phi = np.zeros((b, H, npairs)) if inp.get("init") is None else np.asarray(inp["init"]["phi"], np.float64)
            phi = phi + np.einsum("blh,blhi->bhi", np.asarray(inp["dt"], np.float64),
                                  np.asarray(inp["theta"], np.float64))
            v += float(np.sum(np.asarray(dfinal["phi"], np.float64) * phi))
    return v
