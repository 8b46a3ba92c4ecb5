"""CPU oracle of the per-coordinate selective scan (the Mamba 1 preset): plain,
slow, fp64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module; the GPU library never
does, and it shares no code with the HIP kernels.

Sources (web pages, cited by title and section):

[D]   "Diagonal Equivalence in State Space Models: Characterization,
      Retrieval Rank, and Selective Extensions" (paperpeel.com).
      - Section 5.1, "Per-coordinate scan": diagonal transitions that vary
        across every state coordinate; the scan covers the Mamba 1 preset,
        whose log decay is one static coordinate coefficient times a step.
      - The table of copied-weight presets (Mamba 1 row): real static
        per-coordinate decay with the exponential-Euler write.
      - The related-work paragraph on Mamba 1: one diagonal single-input,
        single-output core per channel, input-dependent steps and B, C.
      - Section 5.5: the scan is an associative recurrence (prefix
        combination of (decay, write) pairs).
[M3]  "Mamba-3: Improved Sequence Modeling using State Space Principles"
      (intuitivepapers.ai explainer), section "How Mamba gets its recurrence
      from a differential equation": the decay exp(dt A) with A frozen at the
      step, and the deployed gain dt (the rectangle rule, exponential-Euler).

What is computed, for every batch b and channel d (group g = d G / D of the
shared B, C), each of the N state coordinates n separately:

    a[d, n]      = -exp(A_log[d, n])                 (static, < 0)
    alpha_t[n]   = exp(dt[b, t, d] a[d, n])
    h[n]        <- alpha_t[n] h[n] + dt[b, t, d] B[b, t, g, n] x[b, t, d]
    y[b, t, d]   = sum_n C[b, t, g, n] h[n]

with the state h [b, D, N] carried in and out.  Nothing here is an
approximation: the oracle is the recurrence itself, evaluated in fp64 on the
inputs' stored values.
"""
import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _dims(inp):
    x = np.asarray(inp["x"])
    b, L, D = x.shape
    G, N = np.asarray(inp["B"]).shape[2:4]
    assert D % G == 0
    return b, L, D, G, N


def decay_rates(A_log):
    """a = -exp(A_log): the static per-coordinate rates [D, N]."""
    return -np.exp(_f64(A_log))


def scan_seq(inp, h0=None):
    """The recurrence token by token (the definition).

    inp: x [b, L, D], dt [b, L, D], A_log [D, N], B, C [b, L, G, N]; h0 [b, D, N]
    or None (zero).  Returns (y [b, L, D], h_final [b, D, N]), fp64.
    """
    b, L, D, G, N = _dims(inp)
    x, dt, B, C = _f64(inp["x"]), _f64(inp["dt"]), _f64(inp["B"]), _f64(inp["C"])
    a = decay_rates(inp["A_log"])                           # [D, N]
    gidx = (np.arange(D) * G) // D                          # group of each channel
    h = np.zeros((b, D, N)) if h0 is None else _f64(h0).copy()
    y = np.zeros((b, L, D))
    for t in range(L):
        Bt = B[:, t][:, gidx]                               # [b, D, N]
        Ct = C[:, t][:, gidx]
        d = dt[:, t][:, :, None]                            # [b, D, 1]
        h = np.exp(d * a[None]) * h + d * Bt * x[:, t][:, :, None]
        y[:, t] = np.sum(Ct * h, axis=2)
    return y, h


def scan_quadratic(inp, h0=None):
    """The same function as a sum over token pairs (masked attention with one
    decay mask per coordinate, [D] section 5.1):

        y_t = sum_n C_t[n] ( prod_{k<=t} alpha_k[n] h0[n]
                             + sum_{s<=t} (prod_{s<k<=t} alpha_k[n]) dt_s B_s[n] x_s )

    with the products taken as exponentials of sums of dt a.  Slow; for small
    inputs only."""
    b, L, D, G, N = _dims(inp)
    x, dt, B, C = _f64(inp["x"]), _f64(inp["dt"]), _f64(inp["B"]), _f64(inp["C"])
    a = decay_rates(inp["A_log"])
    gidx = (np.arange(D) * G) // D
    cum = np.cumsum(dt, axis=1)                              # [b, L, D]: sum_{k<=t} dt_k
    y = np.zeros((b, L, D))
    for t in range(L):
        for s in range(t + 1):
            # sum_{s<k<=t} dt_k = cum_t - cum_s
            w = np.exp((cum[:, t] - cum[:, s])[:, :, None] * a[None])     # [b, D, N]
            term = w * (dt[:, s][:, :, None] * B[:, s][:, gidx] * x[:, s][:, :, None])
            y[:, t] += np.sum(C[:, t][:, gidx] * term, axis=2)
        if h0 is not None:
            w0 = np.exp(cum[:, t][:, :, None] * a[None])
            y[:, t] += np.sum(C[:, t][:, gidx] * w0 * _f64(h0), axis=2)
    return y


def combine(first, second):
    """Composition of two affine per-coordinate steps h -> A h + W (first, then
    second): (A1, W1) then (A2, W2) is (A2 A1, A2 W1 + W2).  The associative
    operator of the prefix scan ([D] section 5.5)."""
    A1, W1 = first
    A2, W2 = second
    return A2 * A1, A2 * W1 + W2


def scan_assoc(inp, h0=None):
    """The recurrence as an inclusive prefix of ``combine`` over the tokens (a
    plain left fold of the associative operator), then the readout: the same
    function as ``scan_seq`` by associativity."""
    b, L, D, G, N = _dims(inp)
    x, dt, B, C = _f64(inp["x"]), _f64(inp["dt"]), _f64(inp["B"]), _f64(inp["C"])
    a = decay_rates(inp["A_log"])
    gidx = (np.arange(D) * G) // D
    steps = [(np.exp(dt[:, t][:, :, None] * a[None]), dt[:, t][:, :, None] * B[:, t][:, gidx] * x[:, t][:, :, None])
             for t in range(L)]
    h_init = np.zeros((b, D, N)) if h0 is None else _f64(h0)
    y = np.zeros((b, L, D))
    acc = None
    for t in range(L):
        acc = steps[t] if acc is None else combine(acc, steps[t])
        h = acc[0] * h_init + acc[1]
        y[:, t] = np.sum(C[:, t][:, gidx] * h, axis=2)
    h_fin = h_init if acc is None else acc[0] * h_init + acc[1]
    return y, h_fin
