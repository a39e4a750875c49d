"""Pins of the SSD error budget (tests/_ssd_bound.py) against the SSD
oracle, on the CPU.  The budget sums magnitudes of the terms that the
kernel rounds; with inputs of one sign those sums are the outputs
themselves, and in general they bound them (triangle inequality):
  * x, B, C > 0, no initial state:  E1 = y - D x exactly (every pair (t, s)
    with s <= t contributes w_ts (C_t . B_s) x_s > 0), and 0 = E2 in the
    first chunk of 64 tokens, 0 < E2 <= E1 after it;
  * x = 0, C > 0, initial state > 0:  E2 = y (the output is the readout of
    the decayed initial state, chunk by chunk);
  * x, B > 0, no initial state:  S_last = the final state;
  * any signs:  |y - D x| <= E1 + E2 and |h_L - e^(lam_L) h0| <= S_last.
A dropped step size, a wrong decay sign, a transposed operand or a chunk
boundary off by one in the budget fails one of these."""
import numpy as np
import pytest

import oracle
from tests._ssd_bound import _softplus, ssd_budget


def problem(seed, batch=2, L=150, H=3, P=8, N=16, G=1, positive=False, zero_x=False, h0=True):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    x, B, C = f(batch, L, H, P), f(batch, L, G, N), f(batch, L, G, N)
    if positive:
        x, B, C = np.abs(x), np.abs(B), np.abs(C)
    if zero_x:
        x = np.zeros_like(x)
    dt = (0.5 * f(batch, L, H)).astype(np.float32)
    bias = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), H)))).astype(np.float32)
    A = (-rng.uniform(1.0, 16.0, H)).astype(np.float32)
    hh = f(batch, H, P, N) if h0 else None
    if hh is not None and positive:
        hh = np.abs(hh)
    return dict(x=x, dt=dt, A=A, B=B, C=C, dt_bias=bias, h0=hh)


def run(pr, D=None):
    y, last = oracle.ssd_scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], D=D, z=None,
                              dt_bias=pr["dt_bias"], h0=pr["h0"])
    E1, E2, Sl = ssd_budget(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], dt_bias=pr["dt_bias"],
                            h0=pr["h0"])
    return y, last, E1, E2, Sl


@pytest.mark.parametrize("G", [1, 3])
def test_positive_inputs_E1_is_the_output(G):
    pr = problem(1, H=3, G=G, positive=True, h0=False)
    y, last, E1, E2, Sl = run(pr)
    np.testing.assert_allclose(E1, y, rtol=1e-12, atol=1e-300)
    # the readout of the state entering a chunk is part of the output: none in
    # the first chunk, and never more than the whole
    np.testing.assert_array_equal(E2[:, :64], 0.0)
    assert np.all(E2[:, 64:] > 0) and np.all(E2 <= E1 * (1 + 1e-12))
    np.testing.assert_allclose(Sl, last, rtol=1e-12)


def test_zero_input_E2_is_the_readout_of_the_initial_state():
    pr = problem(2, positive=True, zero_x=True, h0=True, L=200)
    y, last, E1, E2, Sl = run(pr)
    np.testing.assert_array_equal(E1, 0.0)
    np.testing.assert_allclose(E2, y, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_budget_bounds_the_terms(seed):
    pr = problem(seed, L=257, H=2, G=2, h0=True)
    D = np.linspace(0.5, 1.5, pr["A"].shape[0]).astype(np.float32)
    y, last, E1, E2, Sl = run(pr, D=D)
    yd = y - D[None, None, :, None] * pr["x"].astype(np.float64)
    assert np.all(np.abs(yd) <= (E1 + E2) * (1 + 1e-12) + 1e-300)
    # the final state minus the decayed initial state
    d = _softplus(pr["dt"].astype(np.float64) + pr["dt_bias"][None, None, :])
    lamL = np.sum(d * pr["A"][None, None, :], axis=1)  # (batch, H)
    rest = last - np.exp(lamL)[:, :, None, None] * pr["h0"]
    assert np.all(np.abs(rest) <= Sl * (1 + 1e-12) + 1e-12)
    # not vacuous: most elements' budget is well below a tenth of |y - D x|... or
    # at least of the same order (the sums of |terms| exceed |sum| only by
    # cancellation)
    assert np.median((E1 + E2) / np.maximum(np.abs(yd), 1e-300)) < 20
