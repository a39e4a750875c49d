"""Pins of the float64 SSD (Mamba-2) oracle (oracle/ssd_oracle.c).

The pages state the duality in words: the selective SSM with a scalar decay
per head is a 1-semiseparable matrix, the same as causal-masked linear
attention, and it is computed blockwise: matrix products inside chunks,
boundary states passed between chunks ("Linear Attention vs Softmax
Attention", section "Mamba (Selective State Space Models)"; "RWKV-v6 vs.
Mamba-3 Selective State Spaces", sections "3.1. State Space Duality (SSD)"
and "4. Hardware Acceleration"; "State Space Models in Large Language
Models", section "Mamba-2 and Structured State Space Duality (SSD)").  The
oracle is the recurrence; it is pinned against
  * the matrix side: the masked quadratic form y = (L o C B^T) (dt x), with
    L[t,s] the product of the decays between s and t, built densely;
  * the blockwise side: chunks of several sizes, masked matrix products
    inside each chunk and states passed between chunks;
  * the per-channel oracle of the Mamba-1 scan with the decay broadcast over
    the head's channels and states;
and copies with planted mistakes must fail.
"""
import os
import subprocess

import numpy as np
import pytest
import scipy.special

import oracle


def case(rng, batch, L, H, P, N, G, gate=True, h0=True, softplus=True):
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(x=f(batch, L, H, P), dt=(0.5 * f(batch, L, H)).astype(np.float32),
                A=(-np.exp(rng.uniform(-1, 1, H))).astype(np.float32),
                B=f(batch, L, G, N), C=f(batch, L, G, N), D=f(H),
                z=f(batch, L, H, P) if gate else None,
                dt_bias=rng.uniform(-3, 0, H).astype(np.float32),
                h0=f(batch, H, P, N) if h0 else None, softplus=softplus)


def run(c, lib_path=None):
    return oracle.ssd_scan(c["x"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                           dt_bias=c["dt_bias"], dt_softplus=c["softplus"], h0=c["h0"],
                           lib_path=lib_path)


def steps(c):
    u = c["dt"].astype(np.float64) + c["dt_bias"].astype(np.float64)
    return np.logaddexp(0.0, u) if c["softplus"] else u


def finish(c, y, b, h, x, sl=slice(None)):
    """skip and gate on a (tokens, P) block"""
    y = y + float(c["D"][h]) * x
    if c["z"] is not None:
        zv = c["z"][b, sl, h].astype(np.float64)
        y = y * zv * scipy.special.expit(zv)
    return y


def quadratic(c):
    """y = (L o C B^T) (dt x) + decay * C h0, densely, per (b, h)."""
    x = c["x"].astype(np.float64)
    batch, L, H, P = x.shape
    G, N = c["B"].shape[2:]
    d = steps(c)
    out = np.empty((batch, L, H, P))
    last = np.empty((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            Bm = c["B"][b, :, g].astype(np.float64)
            Cm = c["C"][b, :, g].astype(np.float64)
            lam = np.cumsum(d[b, :, h] * float(c["A"][h]))        # log decay through t
            Lmat = np.tril(np.exp(lam[:, None] - lam[None, :]))  # prod of decays s+1..t
            M = Lmat * (Cm @ Bm.T) * d[b, :, h][None, :]
            y = M @ x[b, :, h]
            h0 = np.zeros((P, N)) if c["h0"] is None else c["h0"][b, h].astype(np.float64)
            y += np.exp(lam)[:, None] * (Cm @ h0.T)
            out[b, :, h] = finish(c, y, b, h, x[b, :, h])
            w = np.exp(lam[-1] - lam) * d[b, :, h] if L else np.zeros(0)
            last[b, h] = np.exp(lam[-1] if L else 0.0) * h0 + (x[b, :, h] * w[:, None]).T @ Bm
    return out, last


def chunked(c, Q):
    """Blockwise: inside a chunk the masked product plus the entering state's
    readout; between chunks h <- e^(sum dt A) h + X_w^T B."""
    x = c["x"].astype(np.float64)
    batch, L, H, P = x.shape
    G, N = c["B"].shape[2:]
    d = steps(c)
    out = np.empty((batch, L, H, P))
    last = np.empty((batch, H, P, N))
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            st = np.zeros((P, N)) if c["h0"] is None else c["h0"][b, h].astype(np.float64)
            for t0 in range(0, L, Q):
                sl = slice(t0, min(t0 + Q, L))
                Bm = c["B"][b, sl, g].astype(np.float64)
                Cm = c["C"][b, sl, g].astype(np.float64)
                dd = d[b, sl, h]
                lam = np.cumsum(dd * float(c["A"][h]))
                S = np.tril(np.exp(lam[:, None] - lam[None, :])) * (Cm @ Bm.T) * dd[None, :]
                y = S @ x[b, sl, h] + np.exp(lam)[:, None] * (Cm @ st.T)
                out[b, sl, h] = finish(c, y, b, h, x[b, sl, h], sl)
                w = np.exp(lam[-1] - lam) * dd
                st = np.exp(lam[-1]) * st + (x[b, sl, h] * w[:, None]).T @ Bm
            last[b, h] = st
    return out, last


@pytest.mark.parametrize("shape", [(2, 13, 4, 3, 5, 2), (1, 40, 2, 4, 3, 1), (1, 1, 3, 2, 2, 3)])
@pytest.mark.parametrize("gate,h0,softplus", [(True, True, True), (False, False, True),
                                              (True, True, False)])
def test_equals_masked_quadratic_form(shape, gate, h0, softplus):
    rng = np.random.default_rng(sum(shape) + gate + 2 * h0 + 4 * softplus)
    c = case(rng, *shape, gate=gate, h0=h0, softplus=softplus)
    if not softplus:
        c["dt"] = np.abs(c["dt"]) + 0.05
        c["dt_bias"] = np.full_like(c["dt_bias"], 0.01)
    out, last = run(c)
    ref, ref_last = quadratic(c)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(last, ref_last, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("Q", [1, 4, 7, 16, 64])
def test_equals_chunked_form(Q):
    rng = np.random.default_rng(Q)
    c = case(rng, 2, 37, 3, 4, 6, 1)
    out, last = run(c)
    ref, ref_last = chunked(c, Q)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(last, ref_last, rtol=1e-11, atol=1e-12)


def test_equals_per_channel_scan_with_broadcast_decay():
    """The Mamba-1 oracle with channel d = (h, p), A[d, n] = A[h], the step
    broadcast over the head's channels and B, C taken from the head's
    group."""
    rng = np.random.default_rng(9)
    batch, L, H, P, N, G = 2, 21, 4, 3, 5, 2
    c = case(rng, batch, L, H, P, N, G)
    out, last = run(c)
    grp = np.arange(H) // (H // G)
    for h in range(H):
        o, l = oracle.scan(c["x"][:, :, h], np.repeat(c["dt"][:, :, h:h + 1], P, axis=2),
                           np.full((P, N), c["A"][h], np.float32), c["B"][:, :, grp[h]],
                           c["C"][:, :, grp[h]], D=np.full(P, c["D"][h], np.float32),
                           z=c["z"][:, :, h], delta_bias=np.full(P, c["dt_bias"][h], np.float32),
                           h0=c["h0"][:, h])
        np.testing.assert_allclose(out[:, :, h], o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(last[:, h], l, rtol=1e-13, atol=1e-14)


MUTANTS = {
    "decay_sign": ("exp(d * (double)A[hd])", "exp(-d * (double)A[hd])"),
    "input_without_step": ("d * (double)xt[p] * (double)Bt[n]", "(double)xt[p] * (double)Bt[n]"),
    "readout_before_update": (
        "            h[p * N + n] = a * h[p * N + n] + d * (double)xt[p] * (double)Bt[n];\n"
        "            y += (double)Ct[n] * h[p * N + n];",
        "            y += (double)Ct[n] * h[p * N + n];\n"
        "            h[p * N + n] = a * h[p * N + n] + d * (double)xt[p] * (double)Bt[n];"),
    "skip_dropped": ("if (D) y += (double)D[hd] * (double)xt[p];", ";"),
    "group_interleaved": ("const int64_t g = hd / (H / G);", "const int64_t g = hd % G;"),
    "initial_state_ignored": ("h[i] = h0 ? (double)h0[(b * H + hd) * P * N + i] : 0.0;",
                              "h[i] = 0.0;"),
    "bias_ignored": ("+ (dt_bias ? (double)dt_bias[hd] : 0.0)", "+ 0.0"),
}


def _pins_pass(lib_path):
    try:
        rng = np.random.default_rng(31)
        c = case(rng, 2, 11, 4, 3, 4, 2)
        out, last = run(c, lib_path)
        ref, ref_last = quadratic(c)
        return bool(np.allclose(out, ref, rtol=1e-10, atol=1e-12) and
                    np.allclose(last, ref_last, rtol=1e-10, atol=1e-12))
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.ssd_lib_path()), "ssd_oracle.c")).read()
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
