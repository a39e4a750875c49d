"""Seeded synthetic inputs for the selective scan -- shapes and value
distributions only.

This module draws random numbers and lays them out; it holds none of the
scan's arithmetic, and it imports neither the HIP binding nor the oracle, so
both sides can take their inputs from here.

Input recipe (the Mamba-shaped workloads):
  * dt[d] log-uniform in [lo, hi] per channel, delta_bias[d] = log(expm1(dt))
    (the inverse of softplus), computed in float64 and stored as float32;
  * delta = 0.5 * N(0,1), stored in the activation dtype, so that
    softplus(delta + bias) scatters around dt;
  * x, z, B, C ~ N(0,1) in the activation dtype (bf16 by round-to-nearest-even
    from float32);
  * A[d,n] = -(n+1) (the S4D-real initialisation: A = -exp(log(1..N)) per
    channel) or, with ``A_kind="general"``, -exp(log(n+1) + 0.1*N(0,1)), a
    stand-in for a trained A without the integer structure;
  * D_skip = 1; decode state ~ N(0,1).
Draw order with the numpy engine (PCG64, ``seed``): dt, x, z, B, C,
delta-noise, h0.  The "torch_cuda" engine draws the same tensors in the same
order from a seeded device Philox generator (used where a host copy of the
whole input would not fit or take too long).
"""
import math

import numpy as np
import torch

# The five workloads: sizes, dtypes and which optional parts are on.
CONFIGS = {
    "tiny_fp32": dict(batch=1, L=256, dim=64, dstate=16, dtype="fp32", gate=True,
                      last_state=False, dt_range=(1e-3, 1e-1)),
    "mamba130m_bf16": dict(batch=4, L=2048, dim=1536, dstate=16, dtype="bf16", gate=True,
                           last_state=False, dt_range=(1e-3, 1e-1)),
    "mamba2p8b_bf16": dict(batch=8, L=4096, dim=5120, dstate=16, dtype="bf16", gate=True,
                           last_state=True, dt_range=(1e-3, 1e-1)),
    "longctx_bf16": dict(batch=1, L=131072, dim=2048, dstate=16, dtype="bf16", gate=False,
                         last_state=False, dt_range=(1e-4, 1e-1)),
    "decode_fp32": dict(batch=256, L=1, dim=5120, dstate=16, dtype="fp32", gate=True,
                        last_state=True, dt_range=(1e-3, 1e-1), steps=1024),
}

# The causal depthwise convolution before the scan (width 4, SiLU) on the
# 130M- and 2.8B-shaped layers' activations, and its per-token update at the
# decode shape.
CONV_CONFIGS = {
    "conv1d_mamba130m_bf16": dict(batch=4, L=2048, dim=1536, width=4, dtype="bf16"),
    "conv1d_mamba2p8b_bf16": dict(batch=8, L=4096, dim=5120, width=4, dtype="bf16"),
    "conv1d_decode_fp32": dict(batch=256, L=1, dim=5120, width=4, dtype="fp32"),
}

# The SSD (Mamba-2) form: a Mamba-2-2.7B-shaped layer (d_model 2560, expand 2:
# 80 heads of 64 channels, dstate 128, one B/C group) over 4 x 2048 tokens.
SSD_CONFIGS = {
    "ssd_mamba2_2p7b_bf16": dict(batch=4, L=2048, H=80, P=64, N=128, G=1, gate=True),
}

# Packed variable-length prefill: the 130M-shaped layer's 8192 tokens as a
# batch of prompts of mixed lengths (log-uniform in [64, 4096], drawn from
# ``seed``) concatenated without padding; fresh prompts (zero initial state),
# every prompt's final state kept for decoding.
VARLEN_CONFIGS = {
    "varlen_mamba130m_bf16": dict(total=8192, len_range=(64, 4096), dim=1536, dstate=16,
                                  dtype="bf16", gate=True, last_state=True,
                                  dt_range=(1e-3, 1e-1)),
}

TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def algorithmic_bytes(batch, L, dim, dstate, dtype, gate, last_state, initial_state=False):
    """Bytes a fused forward must move at least once: every input read once,
    every output written once (x, delta, [z], out; B, C; A, D, bias; states)."""
    es = 4 if dtype == "fp32" else 2
    per_tok = (4 if gate else 3) * es
    b = batch * L * dim * per_tok + 2 * batch * L * dstate * es + dim * dstate * 4 + 2 * dim * 4
    if last_state:
        b += batch * dim * dstate * 4
    if initial_state:
        b += batch * dim * dstate * 4
    return b


def decode_step_bytes(batch, dim, dstate, dtype="fp32", gate=True):
    """Bytes of one decode update: state read + written, x/delta/[z]/out,
    B, C per sequence, and the per-channel parameters."""
    es = 4 if dtype == "fp32" else 2
    return (2 * batch * dim * dstate * 4 + batch * dim * (4 if gate else 3) * es
            + 2 * batch * dstate * es + dim * dstate * 4 + 2 * dim * 4)


def _bias_from_dt(dt):
    # inverse softplus of the target step size: log(exp(dt) - 1)
    return np.log(np.expm1(dt))


def _A(dim, dstate, kind, seed):
    if kind == "s4d_real":
        a = -np.exp(np.log(np.arange(1, dstate + 1, dtype=np.float64)))
        return np.broadcast_to(a, (dim, dstate)).astype(np.float32).copy()
    if kind == "general":
        r = np.random.default_rng(seed + 7919)
        alog = np.log(np.arange(1, dstate + 1, dtype=np.float64))[None, :] + 0.1 * r.standard_normal((dim, dstate))
        return (-np.exp(alog)).astype(np.float32)
    raise ValueError(kind)


def _to_dtype(a32, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a32))
    return t.to(TORCH_DTYPE[dtype])


class Problem:
    """Inputs of one scan call: device tensors plus their parameters."""

    def __init__(self, **kw):
        self.__dict__.update(kw)

    def tensors(self):
        return dict(x=self.x, delta=self.delta, A=self.A, B=self.B, C=self.C, D=self.D,
                    z=self.z, delta_bias=self.delta_bias, initial_state=self.h0)

    def host_f32(self, b_idx=None, d_idx=None):
        """float32 host copies for the oracle, optionally restricted to a
        subset of batch rows and channels (channels are independent)."""
        def sel(t, kind):
            if t is None:
                return None
            if kind == "bld":
                if b_idx is not None:
                    t = t[b_idx]
                if d_idx is not None:
                    t = t[..., d_idx]
            elif kind == "bln":
                if b_idx is not None:
                    t = t[b_idx]
            elif kind == "dn":
                if d_idx is not None:
                    t = t[d_idx]
            elif kind == "d":
                if d_idx is not None:
                    t = t[d_idx]
            elif kind == "bdn":
                if b_idx is not None:
                    t = t[b_idx]
                if d_idx is not None:
                    t = t[:, d_idx]
            return t.to(torch.float32).cpu().numpy()
        return dict(x=sel(self.x, "bld"), delta=sel(self.delta, "bld"), z=sel(self.z, "bld"),
                    B=sel(self.B, "bln"), C=sel(self.C, "bln"), A=sel(self.A, "dn"),
                    D=sel(self.D, "d"), delta_bias=sel(self.delta_bias, "d"),
                    h0=sel(self.h0, "bdn"))


def make_problem(batch, L, dim, dstate, dtype="fp32", gate=True, dt_range=(1e-3, 1e-1),
                 seed=0, device="cpu", engine="numpy", initial_state=False,
                 A_kind="s4d_real", with_D=True, with_bias=True, delta_softplus=True, **_):
    """Draw one problem.  ``engine`` is "numpy" (host PCG64, then copied to
    ``device``) or "torch_cuda" (device Philox, for the large shapes)."""
    lo, hi = dt_range
    A = _A(dim, dstate, A_kind, seed)
    tdt = TORCH_DTYPE[dtype]
    if engine == "numpy":
        rng = np.random.default_rng(seed)
        dt = np.exp(rng.uniform(math.log(lo), math.log(hi), size=dim))
        x = _to_dtype(rng.standard_normal((batch, L, dim), dtype=np.float32), dtype)
        z = _to_dtype(rng.standard_normal((batch, L, dim), dtype=np.float32), dtype)
        B = _to_dtype(rng.standard_normal((batch, L, dstate), dtype=np.float32), dtype)
        C = _to_dtype(rng.standard_normal((batch, L, dstate), dtype=np.float32), dtype)
        delta = _to_dtype(0.5 * rng.standard_normal((batch, L, dim), dtype=np.float32), dtype)
        h0 = (torch.from_numpy(rng.standard_normal((batch, dim, dstate), dtype=np.float32))
              if initial_state else None)
        move = lambda t: None if t is None else t.to(device)
        x, z, B, C, delta, h0 = map(move, (x, z, B, C, delta, h0))
    elif engine == "torch_cuda":
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        dt = torch.exp(torch.empty(dim, dtype=torch.float64, device=device).uniform_(
            math.log(lo), math.log(hi), generator=g)).cpu().numpy()
        rn = lambda *s: torch.randn(*s, generator=g, device=device, dtype=torch.float32)
        x = rn(batch, L, dim).to(tdt)
        z = rn(batch, L, dim).to(tdt)
        B = rn(batch, L, dstate).to(tdt)
        C = rn(batch, L, dstate).to(tdt)
        delta = (0.5 * rn(batch, L, dim)).to(tdt)
        h0 = rn(batch, dim, dstate) if initial_state else None
    else:
        raise ValueError(engine)
    bias = _bias_from_dt(dt).astype(np.float32)
    return Problem(
        batch=batch, L=L, dim=dim, dstate=dstate, dtype=dtype, delta_softplus=delta_softplus,
        x=x, delta=delta, z=z if gate else None, B=B, C=C,
        A=torch.from_numpy(A).to(device),
        D=torch.ones(dim, dtype=torch.float32, device=device) if with_D else None,
        delta_bias=torch.from_numpy(bias).to(device) if with_bias else None,
        h0=h0)


def make_decode_tokens(steps, batch, dim, dstate, seed=0, device="cuda", engine="torch_cuda",
                       dt_range=(1e-3, 1e-1), A_kind="s4d_real"):
    """Decode workload: an initial state and ``steps`` one-token inputs per
    sequence, step-major so that each step's slice is contiguous.
    Returns dict with state0 (batch,dim,N) and x/delta/z (steps,batch,dim),
    B/C (steps,batch,N), A, D, delta_bias."""
    lo, hi = dt_range
    A = torch.from_numpy(_A(dim, dstate, A_kind, seed)).to(device)
    if engine == "torch_cuda":
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        dt = torch.exp(torch.empty(dim, dtype=torch.float64, device=device).uniform_(
            math.log(lo), math.log(hi), generator=g)).cpu().numpy()
        rn = lambda *s: torch.randn(*s, generator=g, device=device, dtype=torch.float32)
        x = rn(steps, batch, dim)
        z = rn(steps, batch, dim)
        B = rn(steps, batch, dstate)
        C = rn(steps, batch, dstate)
        delta = 0.5 * rn(steps, batch, dim)
        state0 = rn(batch, dim, dstate)
    elif engine == "numpy":
        rng = np.random.default_rng(seed)
        dt = np.exp(rng.uniform(math.log(lo), math.log(hi), size=dim))
        f = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(device)
        x = f(steps, batch, dim)
        z = f(steps, batch, dim)
        B = f(steps, batch, dstate)
        C = f(steps, batch, dstate)
        delta = 0.5 * f(steps, batch, dim)
        state0 = f(batch, dim, dstate)
    else:
        raise ValueError(engine)
    bias = torch.from_numpy(_bias_from_dt(dt).astype(np.float32)).to(device)
    return dict(state0=state0, x=x, delta=delta, z=z, B=B, C=C, A=A,
                D=torch.ones(dim, dtype=torch.float32, device=device), delta_bias=bias)


def varlen_lengths(total, len_range, seed=0):
    """Sequence lengths, log-uniform in ``len_range``, drawn until they
    cover ``total`` tokens; the last one is cut so they sum to ``total``."""
    lo, hi = len_range
    rng = np.random.default_rng(seed + 104729)
    lens = []
    while sum(lens) < total:
        lens.append(int(round(math.exp(rng.uniform(math.log(lo), math.log(hi))))))
    lens[-1] -= sum(lens) - total
    return lens


class VarlenProblem:
    """Inputs of one packed-sequence scan call: (total, dim) activations,
    (total, dstate) B/C, offsets ``cu_seqlens`` (nseq + 1, int32) and
    per-sequence initial states (nseq, dim, dstate) or None."""

    def __init__(self, **kw):
        self.__dict__.update(kw)

    def tensors(self):
        return dict(x=self.x, delta=self.delta, A=self.A, B=self.B, C=self.C, D=self.D,
                    z=self.z, delta_bias=self.delta_bias, initial_state=self.h0,
                    cu_seqlens=self.cu_seqlens)

    def host_f32(self, s, d_idx=None):
        """float32 host copies of sequence s alone as a (1, len, .) problem
        (optionally restricted to channels d_idx), for the oracle."""
        t0, t1 = self.offsets[s], self.offsets[s + 1]

        def sel(t, cols):
            if t is None:
                return None
            if cols and d_idx is not None:
                t = t[..., d_idx]
            return t.to(torch.float32).cpu().numpy()
        tok = lambda t: None if t is None else t[t0:t1][None]
        h0 = None if self.h0 is None else self.h0[s:s + 1]
        if h0 is not None and d_idx is not None:
            h0 = h0[:, d_idx]
        return dict(x=sel(tok(self.x), True), delta=sel(tok(self.delta), True),
                    z=sel(tok(self.z), True), B=sel(tok(self.B), False), C=sel(tok(self.C), False),
                    A=sel(self.A if d_idx is None else self.A[d_idx], False),
                    D=sel(None if self.D is None else (self.D if d_idx is None else self.D[d_idx]), False),
                    delta_bias=sel(None if self.delta_bias is None else
                                   (self.delta_bias if d_idx is None else self.delta_bias[d_idx]), False),
                    h0=sel(h0, False))


def make_varlen_problem(lengths, dim, dstate, dtype="fp32", gate=True, dt_range=(1e-3, 1e-1),
                        seed=0, device="cpu", engine="numpy", initial_state=False, **kw):
    """Packed sequences of the given lengths (zeros allowed): the tokens are
    drawn as one (1, total, .) problem by ``make_problem`` (same recipe),
    the initial states from a second seeded stream."""
    lengths = [int(n) for n in lengths]
    total = sum(lengths)
    p = make_problem(1, total, dim, dstate, dtype=dtype, gate=gate, dt_range=dt_range, seed=seed,
                     device=device, engine=engine, initial_state=False, **kw)
    nseq = len(lengths)
    h0 = None
    if initial_state:
        rng = np.random.default_rng(seed + 15485863)
        h0 = torch.from_numpy(rng.standard_normal((nseq, dim, dstate), dtype=np.float32)).to(device)
    offsets = [0]
    for n in lengths:
        offsets.append(offsets[-1] + n)
    cu = torch.tensor(offsets, dtype=torch.int32, device=device)
    sq = lambda t: None if t is None else t[0]
    return VarlenProblem(lengths=lengths, offsets=offsets, nseq=nseq, total=total, dim=dim,
                         dstate=dstate, dtype=dtype, delta_softplus=p.delta_softplus,
                         x=sq(p.x), delta=sq(p.delta), z=sq(p.z), B=sq(p.B), C=sq(p.C), A=p.A,
                         D=p.D, delta_bias=p.delta_bias, h0=h0, cu_seqlens=cu)


def make_conv_problem(batch, L, dim, width=4, dtype="fp32", seed=0, device="cpu", engine="numpy",
                      initial_state=False, with_bias=True, **_):
    """Inputs of the causal depthwise convolution: x ~ N(0,1) (batch, L, dim)
    in the activation dtype; weight (dim, width) and bias (dim) uniform in
    +-1/sqrt(width) (PyTorch's default bound for a depthwise Conv1d, fan-in =
    width), float32; conv state (batch, dim, width-1) ~ N(0,1) in the
    activation dtype.  Draw order: weight, bias, x, state."""
    bound = 1.0 / math.sqrt(width)
    tdt = TORCH_DTYPE[dtype]
    if engine == "numpy":
        rng = np.random.default_rng(seed + 271828)
        w = torch.from_numpy(rng.uniform(-bound, bound, (dim, width)).astype(np.float32))
        bias = torch.from_numpy(rng.uniform(-bound, bound, dim).astype(np.float32))
        x = _to_dtype(rng.standard_normal((batch, L, dim), dtype=np.float32), dtype)
        st = (_to_dtype(rng.standard_normal((batch, dim, width - 1), dtype=np.float32), dtype)
              if initial_state else None)
        move = lambda t: None if t is None else t.to(device)
        w, bias, x, st = map(move, (w, bias, x, st))
    elif engine == "torch_cuda":
        g = torch.Generator(device=device)
        g.manual_seed(seed + 271828)
        w = torch.empty(dim, width, device=device).uniform_(-bound, bound, generator=g)
        bias = torch.empty(dim, device=device).uniform_(-bound, bound, generator=g)
        x = torch.randn(batch, L, dim, generator=g, device=device).to(tdt)
        st = (torch.randn(batch, dim, width - 1, generator=g, device=device).to(tdt)
              if initial_state else None)
    else:
        raise ValueError(engine)
    return Problem(batch=batch, L=L, dim=dim, width=width, dtype=dtype, x=x, weight=w,
                   bias=bias if with_bias else None, state0=st)


def make_ssd_problem(batch, L, H, P, N, G=1, gate=True, dt_range=(1e-3, 1e-1), seed=0,
                     device="cpu", engine="numpy", initial_state=False, with_D=True,
                     with_bias=True, dt_softplus=True, **_):
    """Inputs of the SSD form: per head a step size log-uniform in dt_range
    (bias = inverse softplus), dt = 0.5 N(0,1), A[h] = -U(1, 16) (Mamba-2's
    range of decay rates), D = 1; x, z, B, C ~ N(0,1) in bf16; state ~
    N(0,1).  Draw order: step sizes, A, x, z, B, C, dt, state."""
    lo, hi = dt_range
    bf = torch.bfloat16
    if engine == "numpy":
        rng = np.random.default_rng(seed + 6700417)
        dts = np.exp(rng.uniform(math.log(lo), math.log(hi), size=H))
        A = -rng.uniform(1.0, 16.0, size=H).astype(np.float32)
        f = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32))
        x, z, B, C = f(batch, L, H, P), f(batch, L, H, P), f(batch, L, G, N), f(batch, L, G, N)
        dt = 0.5 * f(batch, L, H)
        h0 = f(batch, H, P, N) if initial_state else None
        mv = lambda t, dtp=bf: None if t is None else t.to(dtp).to(device)
        x, z, B, C, dt = (mv(t) for t in (x, z, B, C, dt))
        h0 = mv(h0, torch.float32)
        A = torch.from_numpy(A).to(device)
    elif engine == "torch_cuda":
        g = torch.Generator(device=device)
        g.manual_seed(seed + 6700417)
        dts = torch.exp(torch.empty(H, dtype=torch.float64, device=device).uniform_(
            math.log(lo), math.log(hi), generator=g)).cpu().numpy()
        A = -torch.empty(H, device=device).uniform_(1.0, 16.0, generator=g)
        rn = lambda *s: torch.randn(*s, generator=g, device=device)
        x, z, B, C = rn(batch, L, H, P).to(bf), rn(batch, L, H, P).to(bf), rn(batch, L, G, N).to(bf), \
            rn(batch, L, G, N).to(bf)
        dt = (0.5 * rn(batch, L, H)).to(bf)
        h0 = rn(batch, H, P, N) if initial_state else None
    else:
        raise ValueError(engine)
    bias = torch.from_numpy(_bias_from_dt(dts).astype(np.float32)).to(device)
    return Problem(batch=batch, L=L, H=H, P=P, N=N, G=G, dt_softplus=dt_softplus, x=x,
                   z=z if gate else None, B=B, C=C, dt=dt, A=A,
                   D=torch.ones(H, dtype=torch.float32, device=device) if with_D else None,
                   dt_bias=bias if with_bias else None, h0=h0)
