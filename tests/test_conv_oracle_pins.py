"""Pins of the float64 convolution oracle (oracle/conv_oracle.c) against
what the pages and the mathematics fix.

The page ("Linear Attention vs Softmax Attention: Can RWKV or Mamba Replace
Transformers?", section "Implementation") runs the main branch through a
depthwise Conv1d padded by kernel_size - 1 and cut to seq_len, then SiLU.
Here that is checked against library routines that compute the same
definition on their own (numpy's correlate and convolve, scipy's FIR filter,
scipy's logistic function), against an impulse response, and against the
structural properties a causal filter with a carried state must have
(split/resume, one-step decoding).  Copies of the oracle with a plausible
slip planted must fail the pins.
"""
import os
import subprocess

import numpy as np
import pytest
import scipy.signal
import scipy.special

import oracle


def case(rng, batch, L, dim, W, state=True, bias=True):
    return dict(x=rng.standard_normal((batch, L, dim)).astype(np.float32),
                w=rng.uniform(-1, 1, (dim, W)).astype(np.float32),
                bias=rng.uniform(-1, 1, dim).astype(np.float32) if bias else None,
                state=rng.standard_normal((batch, dim, W - 1)).astype(np.float32) if state else None)


def reference(c, silu):
    """Per channel: the input with the state in front, correlated with the
    filter ('valid' keeps exactly the L causal outputs), plus bias, then
    SiLU as v * logistic(v)."""
    x, w = c["x"].astype(np.float64), c["w"].astype(np.float64)
    batch, L, dim = x.shape
    W = w.shape[1]
    out = np.empty((batch, L, dim))
    fin = np.empty((batch, dim, W - 1))
    for b in range(batch):
        for d in range(dim):
            pre = (c["state"][b, d].astype(np.float64) if c["state"] is not None
                   else np.zeros(W - 1))
            xx = np.concatenate([pre, x[b, :, d]])
            v = np.correlate(xx, w[d], mode="valid")
            if c["bias"] is not None:
                v = v + float(c["bias"][d])
            out[b, :, d] = v * scipy.special.expit(v) if silu else v
            fin[b, d] = xx[len(xx) - (W - 1):]
    return out, fin


def run(c, silu=True, lib_path=None):
    return oracle.conv1d_fwd(c["x"], c["w"], c["bias"], silu, c["state"], lib_path=lib_path)


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("silu", [True, False])
@pytest.mark.parametrize("state", [True, False])
def test_equals_correlation_with_state_prefix(W, silu, state):
    rng = np.random.default_rng(W * 10 + silu * 2 + state)
    c = case(rng, 2, 19, 3, W, state=state)
    out, fin = run(c, silu)
    ref, ref_fin = reference(c, silu)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(fin, ref_fin)


def test_zero_state_equals_convolution_and_fir_filter():
    """No state = the page's zero padding: np.convolve with the reversed
    filter (first L outputs) and scipy's FIR filter give the same line."""
    rng = np.random.default_rng(3)
    c = case(rng, 1, 25, 2, 4, state=False, bias=False)
    out, _ = run(c, silu=False)
    for d in range(2):
        xd = c["x"][0, :, d].astype(np.float64)
        taps = c["w"][d, ::-1].astype(np.float64)
        np.testing.assert_allclose(out[0, :, d], np.convolve(xd, taps)[:25], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(out[0, :, d], scipy.signal.lfilter(taps, [1.0], xd),
                                   rtol=1e-12, atol=1e-13)


def test_impulse_response_is_the_reversed_filter():
    W, L, t0 = 4, 12, 5
    x = np.zeros((1, L, 1), np.float32)
    x[0, t0, 0] = 1.0
    w = np.array([[0.5, -0.25, 2.0, 1.5]], np.float32)
    out, _ = oracle.conv1d_fwd(x, w, None, False)
    expect = np.zeros(L)
    for j in range(W):
        expect[t0 + j] = w[0, W - 1 - j]  # output t0+j sees the impulse through tap W-1-j
    np.testing.assert_array_equal(out[0, :, 0], expect)


def test_silu_values():
    x = np.array([[[0.0], [1.0], [-1.0], [30.0], [-30.0]]], np.float32)
    w = np.ones((1, 1), np.float32)  # W = 1: out = silu(x)
    out, _ = oracle.conv1d_fwd(x, w, None, True)
    v = x[0, :, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, :, 0], v * scipy.special.expit(v), rtol=1e-15, atol=1e-300)
    assert out[0, 0, 0] == 0.0 and abs(out[0, 3, 0] - 30.0) < 1e-11


def test_split_resume_equals_one_call():
    rng = np.random.default_rng(11)
    c = case(rng, 2, 30, 3, 4)
    full, fin = run(c)
    for L1 in (0, 1, 2, 3, 17, 30):
        a = dict(c, x=c["x"][:, :L1])
        o1, s1 = run(a)
        b = dict(c, x=c["x"][:, L1:], state=s1.astype(np.float32))
        o2, s2 = run(b)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), full, rtol=1e-14, atol=1e-15)
        np.testing.assert_array_equal(s2, fin)


def test_chained_steps_equal_one_call():
    rng = np.random.default_rng(12)
    c = case(rng, 3, 9, 4, 4)
    full, fin = run(c)
    st = c["state"]
    for t in range(9):
        o, st64 = oracle.conv1d_update(st, c["x"][:, t], c["w"], c["bias"], True)
        np.testing.assert_allclose(o, full[:, t], rtol=1e-14, atol=1e-15)
        st = st64.astype(np.float32)
    np.testing.assert_array_equal(st, fin)


def test_short_input_final_state_keeps_older_state():
    rng = np.random.default_rng(13)
    c = case(rng, 1, 1, 2, 4)
    _, fin = run(c)
    np.testing.assert_array_equal(fin[0, :, :2], c["state"][0, :, 1:])
    np.testing.assert_array_equal(fin[0, :, 2], c["x"][0, 0, :])


# ----------------------------------------------------------------------------
# planted mistakes (temporary CPU builds of mutated copies)
MUTANTS = {
    "taps_reversed": ("(double)w[d * W + k]", "(double)w[d * W + (W - 1 - k)]"),
    "bias_dropped": ("double acc = bias ? (double)bias[d] : 0.0;", "double acc = 0.0;"),
    "current_token_missing": ("for (int64_t k = 0; k < W; ++k)", "for (int64_t k = 0; k < W - 1; ++k)"),
    "silu_sign": ("acc / (1.0 + exp(-acc))", "acc / (1.0 + exp(acc))"),
    "state_reversed": ("(W - 1) + s]", "(-1 - s)]"),
    "final_state_shifted": ("L - (W - 1) + j", "L - W + j"),
}


def _pins_pass(lib_path):
    try:
        rng = np.random.default_rng(21)
        for W in (3, 4):
            c = case(rng, 2, 13, 3, W)
            out, fin = run(c, True, lib_path=lib_path)
            ref, ref_fin = reference(c, True)
            if not (np.allclose(out, ref, rtol=1e-12, atol=1e-13) and np.array_equal(fin, ref_fin)):
                return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.conv_lib_path()), "conv_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = tmp_path / ("m_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    so = tmp_path / ("m_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(mutated),
                           "-lm"])
    assert _pins_pass(str(so)) is False, "planted mistake %r went unnoticed" % name


def test_unmutated_build_passes_the_same_pins():
    assert _pins_pass(None) is True
