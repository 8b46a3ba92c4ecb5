"""CPU oracle for the Mamba-3 selective scan: plain, slow, fp64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module; the GPU library never
does, and it shares no code with the HIP kernels.

Sources (web pages, cited by title and section):

[M3]  "Mamba-3: Improved Sequence Modeling using State Space Principles"
      (intuitivepapers.ai explainer).
      - "How the exponential-trapezoidal update works": the three-term update
        h_t = a_t h_{t-1} + b_t B_{t-1} x_{t-1} + g_t B_t x_t with
        a_t = exp(dt_t A_t), b_t = a_t dt_t (1 - lam_t), g_t = lam_t dt_t, and
        the worked example with x = (1, 0, 0).
      - "The trapezoid term as a two-tap filter": the masked matrix form
        Y = (L o C B^T) X, with L the decay mask times a bidiagonal band.
      - "Computing the rotation as a data-dependent RoPE": the running angle
        phi_t = phi_{t-1} + dt_t theta_t, B and C rotated by the accumulated
        angle instead of rotating the state, the lagged term keeping the
        previous token's rotation, and the decode-step listing (carried h,
        phi, B_prev, x_prev).
      - "MIMO: a rank-4 state update for the same state size": x_t is P x R,
        B_t is N x R, R writes share one decay and are summed into one state,
        which is read R times.
      - The remarks after the decode listing on the layer's remaining
        nonlinearities: the rate activation the code calls heavy_tail, 1 + u
        for u >= 0 and 1 / (1 - u) for u < 0, negated and clamped at -1e-4
        (the per-token rate A_t = -heavy_tail(A_r) of the listing).
[D]   "Diagonal Equivalence in State Space Models: Characterization,
      Retrieval Rank, and Selective Extensions" (paperpeel.com).
      - Section 2.4: chunked evaluation with chunk-local cumulative
        log-decays and carried boundary states.
      - Appendix C.2: initial/final carries (state, phase, previous write).

Conventions where the pages leave a choice (each is a reading, not a fact):
  * The state H is P x N; a write is X^T B (sum over the R ranks of the outer
    products x_r (x) B_r); readout r is H @ C_r (P numbers).
  * Rotation pairs are adjacent dims (2i, 2i+1), i < npairs; dims from
    2*npairs on do not rotate.  rot(v, phi) turns each pair counter-clockwise
    by phi_i; B and C are turned by the same rule.
  * theta is the activated angular rate; each token adds dt_t * theta_t.
  * The per-head bias is added to B and C before the rotation.
  * B/C groups: head h reads group h * G // H.
  * The carried B_prev is the biased and rotated B of the previous token.
  * The returned phase is reduced into [0, 2 pi).

All functions take the dict produced by ``m3inputs.make_scan_inputs`` (float32
arrays of storage-exact values) and compute in float64.
"""
import math

import numpy as np

TWO_PI = 2.0 * math.pi


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def rot(v, phi):
    """Rotate adjacent pairs of the last axis of ``v`` by the angles ``phi``.

    [M3] "Computing the rotation as a data-dependent RoPE": a complex channel
    is a 2 x 2 rotation acting on a pair of real state entries.  Pair i is
    (2i, 2i+1); ``phi`` has one angle per pair and may broadcast against the
    leading axes of ``v``.
    """
    v = np.array(v, dtype=np.float64, copy=True)
    npairs = np.shape(phi)[-1] if np.ndim(phi) else 0
    if npairs == 0:
        return v
    c, s = np.cos(phi), np.sin(phi)
    e = v[..., 0:2 * npairs:2].copy()
    o = v[..., 1:2 * npairs:2].copy()
    v[..., 0:2 * npairs:2] = e * c - o * s
    v[..., 1:2 * npairs:2] = e * s + o * c
    return v


def heavy_tail_rate(u):
    """Per-token decay rate A_t (< 0) from the rate input u (float or array).

    [M3] remarks after the decode listing: heavy_tail(u) is 1 + u for u >= 0
    and 1 / (1 - u) for u < 0; the rate is its negation, clamped at -1e-4.
    """
    u = np.asarray(u, dtype=np.float64)
    ht = np.where(u >= 0.0, 1.0 + u, 1.0 / (1.0 - np.minimum(u, 0.0)))
    return np.minimum(-ht, -1e-4)


def _rate_mag(inp, bi, h, L):
    """a_t = -A_t > 0 for the L tokens of stream (bi, h): exp(A_log[h]) for the
    static law, or -heavy_tail_rate(A_raw[bi, t, h]) for per-token rates."""
    if inp.get("A_raw") is not None:
        return -heavy_tail_rate(inp["A_raw"][bi, :, h])
    return np.full(L, math.exp(float(inp["A_log"][h])))


def _dims(inp):
    b, L, H, R, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[4]
    npairs = 0 if inp.get("theta") is None else inp["theta"].shape[3]
    return b, L, H, G, R, P, N, npairs


def _stream(inp, bi, h):
    """fp64 views of one (batch, head) stream, with the bias folded into B, C."""
    b, L, H, G, R, P, N, npairs = _dims(inp)
    g = h * G // H
    f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    x = f(inp["x"][bi, :, h])                       # [L,R,P]
    Bh = f(inp["B"][bi, :, g])                      # [L,R,N]
    Ch = f(inp["C"][bi, :, g])
    if inp.get("B_bias") is not None:
        Bh = Bh + f(inp["B_bias"][h])
    if inp.get("C_bias") is not None:
        Ch = Ch + f(inp["C_bias"][h])
    dt = f(inp["dt"][bi, :, h])
    lam = f(inp["lam"][bi, :, h])
    th = f(inp["theta"][bi, :, h]) if npairs else np.zeros((L, 0))
    a = _rate_mag(inp, bi, h, L)                     # [L]: A_t = -a_t
    init = inp.get("init")
    if init is not None:
        H0 = f(init["h"][bi, h])
        phi0 = f(init["phi"][bi, h])
        Bp0 = f(init["B_prev"][bi, h])
        xp0 = f(init["x_prev"][bi, h])
    else:
        H0, phi0 = np.zeros((P, N)), np.zeros(npairs)
        Bp0, xp0 = np.zeros((R, N)), np.zeros((R, P))
    return dict(x=x, B=Bh, C=Ch, dt=dt, lam=lam, theta=th, a=a,
                H0=H0, phi0=phi0, Bp0=Bp0, xp0=xp0, L=L, R=R, P=P, N=N)


def _alloc(inp):
    b, L, H, G, R, P, N, npairs = _dims(inp)
    y = np.zeros((b, L, H, R, P))
    fin = {"h": np.zeros((b, H, P, N)), "phi": np.zeros((b, H, npairs)),
           "B_prev": np.zeros((b, H, R, N)), "x_prev": np.zeros((b, H, R, P))}
    return y, fin


def _store(fin, bi, h, H_, phi, Bp, Xp):
    fin["h"][bi, h] = H_
    fin["phi"][bi, h] = np.mod(phi, TWO_PI)
    fin["B_prev"][bi, h] = Bp
    fin["x_prev"][bi, h] = Xp


# ----------------------------------------------------------------------------
# 1. the sequential recurrence (the definition)
# ----------------------------------------------------------------------------
def scan_seq(inp):
    """Token-by-token recurrence; returns (y [b,L,H,R,P], final carry dict).

    [M3] "How the exponential-trapezoidal update works" (three-term update),
    "Computing the rotation as a data-dependent RoPE" (rotated B, C and the
    lagged term carrying the previous rotation), "MIMO: a rank-4 state update"
    (rank-R write, R readouts).
    """
    b, L, H, G, R, P, N, npairs = _dims(inp)
    y, fin = _alloc(inp)
    for bi in range(b):
        for h in range(H):
            s = _stream(inp, bi, h)
            Hs, phi, Bp, Xp = s["H0"].copy(), s["phi0"].copy(), s["Bp0"].copy(), s["xp0"].copy()
            for t in range(L):
                dt, lam = s["dt"][t], s["lam"][t]
                alpha = math.exp(-dt * s["a"][t])
                beta = alpha * dt * (1.0 - lam)
                gamma = lam * dt
                phi = phi + dt * s["theta"][t]
                Bt = rot(s["B"][t], phi)                 # R x N
                Ct = rot(s["C"][t], phi)
                X = s["x"][t]                            # R x P
                Hs = alpha * Hs + beta * (Xp.T @ Bp) + gamma * (X.T @ Bt)
                y[bi, t, h] = Ct @ Hs.T                  # y[r,:] = H @ C_r
                Bp, Xp = Bt, X
            _store(fin, bi, h, Hs, phi, Bp, Xp)
    return y, fin


# ----------------------------------------------------------------------------
# 2. one decode step (the page's listing, restricted to the scan core)
# ----------------------------------------------------------------------------
def decode_step(carry, x, B, C, dt, lam, theta, A_log, B_bias=None, C_bias=None, A_raw=None):
    """One token for every (batch, head); returns (y [b,H,R,P], new carry).

    [M3] "Computing the rotation as a data-dependent RoPE", decode listing:
    step size, decay, trapezoid weights, biased B/C, phase update, rotation,
    three-term state update, readout, cache of the previous write.  The
    projections, activations, D skip and gate around it are outside the scan.

    carry: dict h [b,H,P,N], phi [b,H,np], B_prev [b,H,R,N], x_prev [b,H,R,P]
    x [b,H,R,P]; B, C [b,G,R,N]; dt, lam [b,H]; theta [b,H,np] or None;
    A_raw [b,H] per-token rate inputs (heavy-tail law) or None (A = -exp(A_log)).
    """
    f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    h, phi = f(carry["h"]), f(carry["phi"])
    Bp, Xp = f(carry["B_prev"]), f(carry["x_prev"])
    b, H, R, P = np.shape(x)
    G = np.shape(B)[1]
    y = np.zeros((b, H, R, P))
    new = {"h": np.zeros_like(h), "phi": np.zeros_like(phi),
           "B_prev": np.zeros_like(Bp), "x_prev": np.zeros((b, H, R, P))}
    for bi in range(b):
        for hh in range(H):
            g = hh * G // H
            d = float(dt[bi, hh])
            rate = (float(heavy_tail_rate(A_raw[bi, hh])) if A_raw is not None
                    else -math.exp(float(A_log[hh])))
            alpha = math.exp(d * rate)
            lm = float(lam[bi, hh])
            beta = alpha * d * (1.0 - lm)
            gamma = lm * d
            Bv = f(B[bi, g]) + (0.0 if B_bias is None else f(B_bias[hh]))
            Cv = f(C[bi, g]) + (0.0 if C_bias is None else f(C_bias[hh]))
            ph = phi[bi, hh] + (d * f(theta[bi, hh]) if theta is not None else 0.0)
            Bv, Cv = rot(Bv, ph), rot(Cv, ph)
            xv = f(x[bi, hh])
            hn = alpha * h[bi, hh] + beta * (Xp[bi, hh].T @ Bp[bi, hh]) + gamma * (xv.T @ Bv)
            for r in range(R):
                y[bi, hh, r] = hn @ Cv[r]
            new["h"][bi, hh] = hn
            new["phi"][bi, hh] = np.mod(ph, TWO_PI)
            new["B_prev"][bi, hh] = Bv
            new["x_prev"][bi, hh] = xv
    return y, new


# ----------------------------------------------------------------------------
# 3. the quadratic (masked matrix) form, brute force
# ----------------------------------------------------------------------------
def scan_quadratic(inp):
    """Whole-sequence masked form Y = (L o C B^T) X plus the carry term.

    [M3] "The trapezoid term as a two-tap filter": the mask is the decay mask
    (entry (t, s) the product of the decays after s up to t) times a matrix
    with gamma on the diagonal and beta one below it.  Written out, entry
    (t, s) of the product is prod_{k=s+1..t} a_k * (g_s + [t > s] d_{s+1})
    with d_u = dt_u (1 - lam_u) (the a_{s+1} inside b_{s+1} completes the
    decay product).  [M3] "MIMO": every write (s, r') reaches every read
    (t, r).  The decays are multiplied out explicitly (no log-sums), so this
    route is independent of the chunked one.  For tiny L only.
    """
    b, L, H, G, R, P, N, npairs = _dims(inp)
    y, fin = _alloc(inp)
    for bi in range(b):
        for h in range(H):
            s = _stream(inp, bi, h)
            dt, lam = s["dt"], s["lam"]
            alpha = np.exp(-dt * s["a"])
            gamma = lam * dt
            delta = dt * (1.0 - lam)
            phi = s["phi0"] + np.cumsum(dt[:, None] * s["theta"], axis=0)   # [L,np]
            Bt = np.stack([rot(s["B"][t], phi[t]) for t in range(L)])      # [L,R,N]
            Ct = np.stack([rot(s["C"][t], phi[t]) for t in range(L)])
            X = s["x"]
            Wm = np.zeros((L, L))
            for t in range(L):
                for u in range(t + 1):
                    band = gamma[u] + (delta[u + 1] if t > u else 0.0)
                    Wm[t, u] = np.prod(alpha[u + 1:t + 1]) * band
            S = Ct.reshape(L * R, N) @ Bt.reshape(L * R, N).T        # [(t,r),(s,r')]
            Wx = np.kron(Wm, np.ones((R, R)))
            yflat = (Wx * S) @ X.reshape(L * R, P)
            Hin = s["H0"] + delta[0] * (s["xp0"].T @ s["Bp0"])
            carry_decay = np.array([np.prod(alpha[:t + 1]) for t in range(L)])
            yflat += np.repeat(carry_decay, R)[:, None] * (Ct.reshape(L * R, N) @ Hin.T)
            y[bi, :, h] = yflat.reshape(L, R, P)
            Hf = np.prod(alpha) * Hin
            for u in range(L):
                band = gamma[u] + (delta[u + 1] if u < L - 1 else 0.0)
                Hf = Hf + np.prod(alpha[u + 1:]) * band * (X[u].T @ Bt[u])
            _store(fin, bi, h, Hf, phi[-1] if L else s["phi0"], Bt[-1], X[-1])
    return y, fin


# ----------------------------------------------------------------------------
# 4. the chunked form
# ----------------------------------------------------------------------------
def scan_chunked(inp, chunk):
    """Chunked evaluation: quadratic inside a chunk, carried state between.

    [D] Section 2.4: chunk-local cumulative log-decays l_t (sum of log a_k
    from the chunk start to t) so that decays are exp(l_t - l_s) differences;
    [M3] "The trapezoid term as a two-tap filter" for the in-chunk mask.
    For chunk [c0, c1) with incoming state H_in and carried previous write
    u = X_prev^T B_prev:
      y_t   = exp(l_t) (H_in + d_c0 u) C_t
              + sum_{c0<=s<=t} exp(l_t - l_s)(g_s + [s<t] d_{s+1}) (C_t . B_s) x_s
      H_out = exp(l_e) (H_in + d_c0 u)
              + sum_s exp(l_e - l_s)(g_s + [s<e] d_{s+1}) X_s^T B_s,   e = c1 - 1
    and the previous write becomes token e's.
    """
    b, L, H, G, R, P, N, npairs = _dims(inp)
    y, fin = _alloc(inp)
    for bi in range(b):
        for h in range(H):
            s = _stream(inp, bi, h)
            dt, lam = s["dt"], s["lam"]
            loga = -dt * s["a"]
            gamma = lam * dt
            delta = dt * (1.0 - lam)
            Hs, phi, Bp, Xp = s["H0"].copy(), s["phi0"].copy(), s["Bp0"].copy(), s["xp0"].copy()
            for c0 in range(0, L, chunk):
                c1 = min(c0 + chunk, L)
                n = c1 - c0
                ell = np.cumsum(loga[c0:c1])
                phis = phi + np.cumsum(dt[c0:c1, None] * s["theta"][c0:c1], axis=0)
                Bt = np.stack([rot(s["B"][c0 + i], phis[i]) for i in range(n)])
                Ct = np.stack([rot(s["C"][c0 + i], phis[i]) for i in range(n)])
                X = s["x"][c0:c1]
                Hin = Hs + delta[c0] * (Xp.T @ Bp)
                for i in range(n):
                    t = c0 + i
                    acc = math.exp(ell[i]) * (Ct[i] @ Hin.T)          # R x P
                    for j in range(i + 1):
                        w = math.exp(ell[i] - ell[j]) * (gamma[c0 + j] + (delta[c0 + j + 1] if j < i else 0.0))
                        acc += w * ((Ct[i] @ Bt[j].T) @ X[j])
                    y[bi, t, h] = acc
                Hn = math.exp(ell[-1]) * Hin
                for j in range(n):
                    w = math.exp(ell[-1] - ell[j]) * (gamma[c0 + j] + (delta[c0 + j + 1] if j < n - 1 else 0.0))
                    Hn = Hn + w * (X[j].T @ Bt[j])
                Hs, phi, Bp, Xp = Hn, phis[-1], Bt[-1], X[-1]
            _store(fin, bi, h, Hs, phi, Bp, Xp)
    return y, fin


# ----------------------------------------------------------------------------
# 5. the unrotated-state form
# ----------------------------------------------------------------------------
def _rot_state(Hm, ang):
    """Rotate the state's N axis (each row of P x N) by per-pair angles."""
    return rot(Hm, ang)


def scan_seq_unrotated(inp):
    """Recurrence with the rotation applied to the state instead of B and C.

    [M3] "Computing the rotation as a data-dependent RoPE": before the change
    of variables the state itself is turned each step and B, C enter raw; the
    rotated state is the unrotated one turned back by the running rotation.
    With B_rot = rot(B, phi_t) the unrotated state obeys
      H'_t = rot_N(a_t H'_{t-1} + b_t X_{t-1}^T B_{t-1}, -dt_t theta_t) + g_t X_t^T B_t
    with raw (biased, unrotated) B and C, and y_t = H'_t C_t.  The carry is
    mapped into this frame by turning it back through -phi0.
    """
    b, L, H, G, R, P, N, npairs = _dims(inp)
    y, fin = _alloc(inp)
    for bi in range(b):
        for h in range(H):
            s = _stream(inp, bi, h)
            Hs = _rot_state(s["H0"], -s["phi0"])
            Bp = rot(s["Bp0"], -s["phi0"])
            Xp = s["xp0"].copy()
            phi = s["phi0"].copy()
            for t in range(L):
                dt, lam = s["dt"][t], s["lam"][t]
                alpha = math.exp(-dt * s["a"][t])
                beta = alpha * dt * (1.0 - lam)
                gamma = lam * dt
                step = dt * s["theta"][t]
                phi = phi + step
                Hs = _rot_state(alpha * Hs + beta * (Xp.T @ Bp), -step) + gamma * (s["x"][t].T @ s["B"][t])
                y[bi, t, h] = s["C"][t] @ Hs.T
                Bp, Xp = s["B"][t], s["x"][t]
            # report the carry in the rotated frame, as the scan does
            _store(fin, bi, h, _rot_state(Hs, phi), phi, rot(Bp, phi), Xp)
    return y, fin


# ----------------------------------------------------------------------------
# 6. an instrumented decode step that counts arithmetic operations
# ----------------------------------------------------------------------------
class _Ops:
    def __init__(self):
        self.n = 0

    def mul(self, a, b):
        self.n += 1
        return a * b

    def add(self, a, b):
        self.n += 1
        return a + b


def counted_decode_step(h, x, B, C, alpha, gamma):
    """Decode step with lambda = 1 and no rotation, counting every operation.

    [M3] "Why a recurrent model's decode step is memory-bound" and "MIMO":
    the page counts a step as one scaling of the state, the rank-R outer
    product added into it, and the R readouts.  gamma is folded into x before
    the count (a per-channel pre-multiply, which the page's count leaves out).
    h [P,N], x [R,P], B, C [R,N].  Returns (h_new, y [R,P], op count).
    """
    P, N = len(h), len(h[0])
    R = len(x)
    ops = _Ops()
    xg = [[gamma * x[r][p] for p in range(P)] for r in range(R)]       # not counted
    hn = [[0.0] * N for _ in range(P)]
    for p in range(P):
        for n in range(N):
            v = ops.mul(alpha, h[p][n])
            for r in range(R):
                v = ops.add(v, ops.mul(xg[r][p], B[r][n]))
            hn[p][n] = v
    y = [[0.0] * P for _ in range(R)]
    for r in range(R):
        for p in range(P):
            acc = ops.mul(hn[p][0], C[r][0])
            for n in range(1, N):
                acc = ops.add(acc, ops.mul(hn[p][n], C[r][n]))
            y[r][p] = acc
    return hn, y, ops.n
