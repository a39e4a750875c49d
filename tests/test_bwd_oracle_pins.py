"""Pins of the float64 gradient oracle (oracle/ssm_oracle_bwd.c).

The pages define the forward loop ("Linear Attention vs Softmax Attention",
section "Implementation"; softplus step size from "State Space Models in
Large Language Models", section "Dynamic Parameterization"); the gradients
are those of that loop.  They are checked two independent ways:
  * numerically: Richardson-extrapolated central differences of the
    forward oracle (a separate library) with steps that are exact in
    float32, for every element of every input;
  * by automatic differentiation: torch.autograd in float64 on the page's
    loop written with plain torch operations.
Copies of the oracle with one plausible slip planted must fail.
"""
import os
import subprocess

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

NAMES = ("x", "delta", "z", "B", "C", "A", "D", "delta_bias", "h0")
GRAD = dict(x="dx", delta="ddelta", z="dz", B="dB", C="dC", A="dA", D="dD",
            delta_bias="ddelta_bias", h0="dh0")


def grid(a):
    """Values on the 2^-12 grid: every finite-difference step below (2^-10,
    2^-11) then moves them exactly in float32."""
    return (np.round(np.asarray(a, np.float64) * 4096) / 4096).astype(np.float32)


def rand_case(rng, batch, L, dim, N, softplus=True, gate=True):
    f = lambda *s: grid(rng.standard_normal(s))
    c = dict(x=f(batch, L, dim), delta=grid(0.5 * rng.standard_normal((batch, L, dim))),
             A=grid(-np.exp(rng.uniform(-1, 1.5, (dim, N)))),
             B=f(batch, L, N), C=f(batch, L, N), D=f(dim), z=f(batch, L, dim) if gate else None,
             delta_bias=grid(rng.uniform(-3, 0, dim)), h0=f(batch, dim, N),
             softplus=softplus)
    if not softplus:
        c["delta"] = grid(np.abs(c["delta"]) + 0.05)
        c["delta_bias"] = grid(np.full(dim, 0.01))
    c["dout"] = f(batch, L, dim)
    c["dlast"] = f(batch, dim, N)
    return c


def loss_fwd(c):
    out, last = oracle.scan(c["x"], c["delta"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                            delta_bias=c["delta_bias"], delta_softplus=c["softplus"], h0=c["h0"])
    return float(np.sum(c["dout"].astype(np.float64) * out) +
                 np.sum(c["dlast"].astype(np.float64) * last))


def grads(c, lib_path=None):
    return oracle.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["dout"], D=c["D"],
                           z=c["z"], delta_bias=c["delta_bias"], delta_softplus=c["softplus"],
                           h0=c["h0"], dlast=c["dlast"], lib_path=lib_path)


def finite_difference(c, name, idx, eps=2.0 ** -10):
    """Central differences at steps eps and eps/2 combined by Richardson
    extrapolation (error O(eps^4)); every perturbed value is exact in
    float32."""
    base = c[name]

    def at(h):
        v = base.copy()
        v[idx] = np.float32(base[idx] + h)
        assert float(v[idx]) - float(base[idx]) == h, "step not exact in float32"
        return loss_fwd(dict(c, **{name: v}))

    d1 = (at(eps) - at(-eps)) / (2 * eps)
    d2 = (at(eps / 2) - at(-eps / 2)) / eps
    return (4 * d2 - d1) / 3


@pytest.mark.parametrize("softplus,gate", [(True, True), (False, True), (True, False)])
def test_every_gradient_element_matches_finite_differences(softplus, gate):
    rng = np.random.default_rng(7 + softplus * 2 + gate)
    c = rand_case(rng, 2, 6, 2, 3, softplus=softplus, gate=gate)
    g = grads(c)
    for name in NAMES:
        if c[name] is None:
            continue
        for idx in np.ndindex(c[name].shape):
            fd = finite_difference(c, name, idx)
            an = g[GRAD[name]][idx]
            assert abs(fd - an) <= 1e-8 + 1e-7 * abs(an), (name, idx, fd, an)


def torch_loop(c):
    """The page's forward loop in float64 torch ops, inputs as leaves."""
    t = {k: torch.tensor(np.asarray(c[k], np.float64), requires_grad=True)
         for k in NAMES if c[k] is not None}
    u = t["delta"] + t["delta_bias"]
    dt = F.softplus(u) if c["softplus"] else u
    h = t["h0"]
    outs = []
    for s in range(u.shape[1]):
        dA = torch.exp(dt[:, s, :, None] * t["A"])
        h = dA * h + dt[:, s, :, None] * t["B"][:, s, None, :] * t["x"][:, s, :, None]
        y = (h * t["C"][:, s, None, :]).sum(-1) + t["D"] * t["x"][:, s]
        if "z" in t:
            y = y * F.silu(t["z"][:, s])
        outs.append(y)
    out = torch.stack(outs, 1)
    loss = (torch.tensor(c["dout"], dtype=torch.float64) * out).sum() + \
        (torch.tensor(c["dlast"], dtype=torch.float64) * h).sum()
    loss.backward()
    return {GRAD[k]: v.grad.numpy() for k, v in t.items()}


def _matches_autograd(c, lib_path=None):
    g = grads(c, lib_path)
    ref = torch_loop(c)
    return all(np.allclose(g[k], v, rtol=1e-10, atol=1e-12) for k, v in ref.items())


@pytest.mark.parametrize("softplus,gate,shape", [
    (True, True, (2, 9, 3, 4)), (False, True, (1, 12, 2, 5)), (True, False, (3, 7, 2, 2)),
])
def test_matches_autograd_of_the_loop(softplus, gate, shape):
    rng = np.random.default_rng(sum(shape))
    c = rand_case(rng, *shape, softplus=softplus, gate=gate)
    g = grads(c)
    for k, v in torch_loop(c).items():
        np.testing.assert_allclose(g[k], v, rtol=1e-10, atol=1e-12, err_msg=k)


def test_no_tokens_passes_dlast_to_the_initial_state():
    rng = np.random.default_rng(3)
    c = rand_case(rng, 2, 0, 3, 4)
    g = grads(c)
    np.testing.assert_array_equal(g["dh0"], c["dlast"].astype(np.float64))
    assert not g["dA"].any() and not g["dD"].any() and not g["ddelta_bias"].any()


def test_thread_count_changes_only_the_last_bits():
    rng = np.random.default_rng(4)
    c = rand_case(rng, 2, 20, 7, 4)
    g1 = oracle.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["dout"], D=c["D"], z=c["z"],
                         delta_bias=c["delta_bias"], h0=c["h0"], dlast=c["dlast"], nthreads=1)
    g5 = oracle.scan_bwd(c["x"], c["delta"], c["A"], c["B"], c["C"], c["dout"], D=c["D"], z=c["z"],
                         delta_bias=c["delta_bias"], h0=c["h0"], dlast=c["dlast"], nthreads=5)
    for k in g1:
        if g1[k] is None:
            continue
        if k in ("dB", "dC"):
            np.testing.assert_allclose(g1[k], g5[k], rtol=1e-13, atol=1e-14)
        else:
            np.testing.assert_array_equal(g1[k], g5[k])


MUTANTS = {
    "softplus_derivative_missing": ("ddt * sigmoid(u)", "ddt"),
    "gate_derivative_sign": ("(1.0 + zv * (1.0 - s))", "(1.0 - zv * (1.0 - s))"),
    "dA_missing_step": ("a[n] * dt * dAn * hp[n];", "a[n] * dAn * hp[n];"),
    "adjoint_not_decayed": ("a[n] *= dAn;", ";"),
    "dC_uses_previous_state": ("dy * ht[n]", "dy * hp[n]"),
    "dx_missing_skip": ("double dxv = dskip * dy, ddt = 0.0;", "double dxv = 0.0, ddt = 0.0;"),
    "dB_missing_input": ("a[n] * dt * xv;", "a[n] * dt;"),
    "ddt_missing_input_term": (" + Bn * xv);", ");"),
    "readout_added_after_use": ("      a[n] += (double)j->C[bc + n] * dy;\n", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.bwd_lib_path()), "ssm_oracle_bwd.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = tmp_path / ("m_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    so = tmp_path / ("m_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(mutated),
                           "-lm", "-lpthread"])
    rng = np.random.default_rng(11)
    c = rand_case(rng, 2, 8, 3, 4)
    assert not _matches_autograd(c, str(so)), "planted mistake %r went unnoticed" % name


def test_unmutated_build_passes_the_same_check():
    rng = np.random.default_rng(11)
    assert _matches_autograd(rand_case(rng, 2, 8, 3, 4))
