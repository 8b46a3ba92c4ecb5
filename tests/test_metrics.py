"""CPU checks of the error metrics the parity tests use."""
import numpy as np

from tests._util import ROW_TOL, pooled_signed, rel_l2, row_errors


def test_row_bound_catches_one_wrong_row():
    """One corrupted (token, rank) row of a long output hides under the
    whole-tensor bound but not under the per-row bound (a planted error in
    oracle-shaped data)."""
    rng = np.random.default_rng(5)
    r = rng.standard_normal((2048, 4, 64))
    g = r * (1 + 3e-3 * rng.standard_normal(r.shape))
    assert row_errors(g, r).max() < ROW_TOL
    g[1000, 2] = rng.standard_normal(64)
    assert rel_l2(g, r) <= 2e-2                      # hidden from the tensor norm
    assert row_errors(g, r).max() > 10 * ROW_TOL     # caught per row


def test_row_bound_floor_near_zero():
    """Rows whose exact value is near zero are judged against a tenth of the RMS
    row norm, so rounding noise there is not amplified without bound."""
    rng = np.random.default_rng(6)
    r = rng.standard_normal((100, 64))
    r[7] *= 1e-9
    g = r + 1e-3 * rng.standard_normal(r.shape)
    e = row_errors(g, r)
    assert e.max() < 2e-2


def test_pooled_signed_sees_a_bias():
    rng = np.random.default_rng(7)
    r = np.abs(rng.standard_normal(1000)) + 0.5
    assert abs(pooled_signed(r * (1 + 1e-3 * rng.standard_normal(1000)), r)) < 1e-3
    assert pooled_signed(r * 1.01, r) > 9e-3
