"""Shared test helpers: tolerances, oracle runs on (sub)problems, comparison."""
import numpy as np
import torch

import oracle

# float32 inputs: rtol 1e-4 / atol 1e-5; bf16 inputs with a float32 state:
# rtol 2e-2 / atol 1e-2 (elementwise |gpu - ref| <= atol + rtol*|ref|)
TOL = {"fp32": (1e-4, 1e-5), "bf16": (2e-2, 1e-2)}


def oracle_for(problem, b_idx=None, d_idx=None, nthreads=None):
    """float64 oracle outputs for a problem, optionally for a subset of batch
    rows and channels (channels are independent, so the subset's outputs are
    the full problem's outputs at those positions)."""
    h = problem.host_f32(b_idx, d_idx)
    return oracle.scan(h["x"], h["delta"], h["A"], h["B"], h["C"], D=h["D"], z=h["z"],
                       delta_bias=h["delta_bias"], delta_softplus=problem.delta_softplus,
                       h0=h["h0"], nthreads=nthreads)


def assert_close(got, ref, rtol, atol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite values" % what
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError("%s: %d of %d elements outside rtol=%g atol=%g; worst at %s: got %r ref %r"
                             % (what, int(bad.sum()), bad.size, rtol, atol, i, got[i], ref[i]))


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()
