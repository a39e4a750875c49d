"""GPU parity of the forward scan with the float64 oracle.

Every case runs the HIP path through the C ABI (ssm_scan_fwd) and compares
each output element with the oracle on the same seeded inputs.  Full-size
workloads are compared on sampled channels (whole sequences), which the
oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_31_amd import ssm_scan_fwd, ssm_scan_fwd_chunked
from selective_state_space_31_amd.workloads import CONFIGS, make_problem
from tests._helpers import TOL, assert_close, oracle_for, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run_and_compare(p, b_idx=None, d_idx=None, last=True, what=""):
    print("case:", what, flush=True)
    out, last_state = ssm_scan_fwd(**p.tensors(), delta_softplus=p.delta_softplus,
                                   return_last_state=True)
    torch.cuda.synchronize()
    ref, ref_last = oracle_for(p, b_idx, d_idx)
    got = out
    gl = last_state
    if b_idx is not None:
        got, gl = got[b_idx], gl[b_idx]
    if d_idx is not None:
        got, gl = got[..., d_idx], gl[:, d_idx]
    rtol, atol = TOL[p.dtype]
    assert_close(to_np(got), ref, rtol, atol, what + " out")
    if last:
        assert_close(to_np(gl), ref_last, rtol, atol, what + " last_state")


def test_config_tiny_fp32():
    c = CONFIGS["tiny_fp32"]
    p = make_problem(**c, seed=0, device=DEV)
    run_and_compare(p, what="tiny_fp32")


def test_config_mamba130m_bf16_full():
    c = CONFIGS["mamba130m_bf16"]
    p = make_problem(**c, seed=0, device=DEV)
    run_and_compare(p, what="mamba130m_bf16")


def test_config_mamba2p8b_bf16_sampled():
    c = CONFIGS["mamba2p8b_bf16"]
    p = make_problem(**c, seed=0, device=DEV, engine="torch_cuda")
    rng = np.random.default_rng(1)
    d_idx = np.unique(np.concatenate([[0, 63, 64, c["dim"] - 1], rng.choice(c["dim"], 60, replace=False)]))
    b_idx = np.array([0, 3, c["batch"] - 1])
    run_and_compare(p, b_idx, torch.from_numpy(d_idx).to(DEV), what="mamba2p8b_bf16 sampled")


def test_config_longctx_bf16_sampled():
    c = CONFIGS["longctx_bf16"]
    p = make_problem(**c, seed=0, device=DEV, engine="torch_cuda")
    rng = np.random.default_rng(2)
    d_idx = np.unique(np.concatenate([[0, 1, c["dim"] - 1], rng.choice(c["dim"], 29, replace=False)]))
    run_and_compare(p, None, torch.from_numpy(d_idx).to(DEV), what="longctx_bf16 sampled")


def test_config_longctx_bf16_general_A_sampled():
    """The 131k-token layer with a non-structured (trained-like) A: every
    decay its own exponential over memories of up to 10^4 steps, in the
    plan's 512-token chunks; sampled channels against the oracle."""
    c = CONFIGS["longctx_bf16"]
    p = make_problem(**c, seed=5, device=DEV, engine="torch_cuda", A_kind="general")
    rng = np.random.default_rng(3)
    d_idx = np.unique(np.concatenate([[0, 63, 64, c["dim"] - 1], rng.choice(c["dim"], 28, replace=False)]))
    run_and_compare(p, None, torch.from_numpy(d_idx).to(DEV), what="longctx_bf16 general A sampled")


SHAPES = [
    # (batch, L, dim, N)
    (1, 1, 64, 16), (2, 3, 64, 16), (1, 63, 64, 16), (1, 64, 64, 16), (1, 65, 64, 16),
    (3, 257, 100, 16), (2, 130, 1, 16), (1, 77, 37, 16), (2, 200, 130, 16),
    (2, 90, 70, 1), (2, 90, 70, 2), (2, 90, 70, 3), (2, 90, 70, 4), (2, 90, 70, 5),
    (2, 90, 70, 8), (1, 90, 70, 12), (1, 90, 70, 32), (1, 50, 70, 33), (1, 50, 70, 64),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_L%d_d%d_N%d" % s)
def test_shapes(shape, dtype):
    b, L, dim, N = shape
    p = make_problem(b, L, dim, N, dtype=dtype, gate=True, seed=hash(shape) % 1000, device=DEV,
                     initial_state=True)
    run_and_compare(p, what="shape %s %s" % (shape, dtype))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("N", [1, 4, 5, 8, 12, 16, 32, 64])
def test_general_A_state_widths(N, dtype):
    """A non-structured A (every decay its own exponential, read from the
    exponent table) at every state width the kernels are built for, exact
    and padded: the library's plan (32-token chunks in groups) and 200-token
    chunks with a ragged last one.  (With N = 1 every A has the S4D-real
    shape.)"""
    p = make_problem(1, 1000, 70, N, dtype=dtype, gate=True, seed=300 + N, device=DEV,
                     A_kind="general", initial_state=True)
    ref, ref_last = oracle_for(p)
    rtol, atol = TOL[dtype]
    for cl in (0, 200):
        print("case: general A, N", N, dtype, "chunk_len", cl, flush=True)
        out, last = ssm_scan_fwd_chunked(**p.tensors(), chunk_len=cl, return_last_state=True)
        torch.cuda.synchronize()
        assert_close(to_np(out), ref, rtol, atol, "general A N=%d chunk_len %d out" % (N, cl))
        assert_close(to_np(last), ref_last, rtol, atol, "general A N=%d chunk_len %d last" % (N, cl))


FLAGS = [
    dict(gate=False), dict(with_D=False), dict(with_bias=False), dict(delta_softplus=False),
    dict(initial_state=False), dict(A_kind="general"), dict(A_kind="general", gate=False),
    dict(gate=False, with_D=False, with_bias=False, initial_state=False),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("flags", FLAGS, ids=lambda f: "-".join("%s=%s" % kv for kv in f.items()))
def test_optional_inputs(flags, dtype):
    kw = dict(gate=True, initial_state=True)
    kw.update(flags)
    p = make_problem(2, 150, 96, 16, dtype=dtype, seed=11, device=DEV, **kw)
    if not p.delta_softplus:
        # keep Delta = delta + bias positive and moderate without softplus
        p.delta = (p.delta.float().abs() * 0.1).to(p.delta.dtype)
        p.delta_bias = torch.full_like(p.delta_bias, 0.01) if p.delta_bias is not None else None
    run_and_compare(p, what="flags %s %s" % (flags, dtype))


def test_no_last_state_requested():
    p = make_problem(1, 40, 64, 16, dtype="fp32", seed=5, device=DEV)
    out = ssm_scan_fwd(**p.tensors())
    torch.cuda.synchronize()
    ref, _ = oracle_for(p)
    assert_close(to_np(out), ref, *TOL["fp32"], what="out only")


def test_empty_sequence_copies_initial_state():
    p = make_problem(2, 0, 64, 16, dtype="fp32", seed=6, device=DEV, initial_state=True)
    out, last = ssm_scan_fwd(**p.tensors(), return_last_state=True)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 64)
    assert torch.equal(last, p.h0)


def test_resume_in_place_over_chunks():
    """last_state may be the initial_state buffer; with the sequence cut into
    many chunks, the output pass must not read initial_state after another
    chunk has overwritten it."""
    p = make_problem(2, 4096, 64, 16, dtype="fp32", seed=9, device=DEV, initial_state=True)
    ref, ref_last = oracle_for(p)
    buf = p.h0.clone()
    t = p.tensors()
    t["initial_state"] = buf
    out, last = ssm_scan_fwd(**t, last_state=buf)
    torch.cuda.synchronize()
    assert last.data_ptr() == buf.data_ptr()
    assert_close(to_np(out), ref, *TOL["fp32"], what="in place out")
    assert_close(to_np(last), ref_last, *TOL["fp32"], what="in place last_state")


# ---------------------------------------------------------------------------
# long memories, the limits of the step size, and independence of the split
# ---------------------------------------------------------------------------

def test_fp32_general_A_long_memory():
    """float32, a non-structured A (every decay its own exponential), 8192
    tokens with dt log-uniform in [1e-4, 1e-1]: memories of ~10^4 steps,
    where a biased exponential would drift past the float32 tolerance.  The
    sequence runs as many chunks (batch 1, two channel tiles)."""
    p = make_problem(1, 8192, 128, 16, dtype="fp32", gate=True, seed=21, device=DEV,
                     A_kind="general", dt_range=(1e-4, 1e-1), initial_state=True)
    run_and_compare(p, what="fp32 general A, L=8192, dt in [1e-4, 1e-1]")


def test_fp32_s4d_long_memory():
    p = make_problem(1, 16384, 64, 16, dtype="fp32", gate=False, seed=22, device=DEV,
                     dt_range=(1e-4, 1e-1), initial_state=True)
    run_and_compare(p, what="fp32 S4D-real A, L=16384, dt in [1e-4, 1e-1]")


LIMIT_L = 4096  # batch 1, one channel tile: the plan cuts this into 128 chunks


@pytest.mark.parametrize("A_kind", ["s4d_real", "general"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_limit_hold(dtype, A_kind):
    """delta -> -inf: softplus gives Delta = 0, so exp(Delta A) = 1 and the
    input term vanishes; the state is held exactly (the chenyuan1125.github.io
    page, section "Selectivity Does Not Drop Tokens; It Changes the Update":
    a small step preserves the state) and out_t = C_t . h0 + D x_t."""
    p = make_problem(1, LIMIT_L, 64, 16, dtype=dtype, gate=True, seed=31, device=DEV,
                     A_kind=A_kind, initial_state=True)
    p.delta = torch.full_like(p.delta, -1000.0)
    out, last = ssm_scan_fwd(**p.tensors(), return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(last, p.h0), "the state must be held bit for bit"
    ref, ref_last = oracle_for(p)
    np.testing.assert_array_equal(ref_last, to_np(p.h0))  # the oracle holds it too
    assert_close(to_np(out), ref, *TOL[dtype], what="hold out")


@pytest.mark.parametrize("A_kind", ["s4d_real", "general"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_limit_reset(dtype, A_kind):
    """Delta = 1000 (softplus off): exp(Delta A) underflows to 0 for every
    state, the past is forgotten at every token and h_t = Delta B_t x_t (same
    page: a large step resets the state to the current input)."""
    p = make_problem(1, LIMIT_L, 64, 16, dtype=dtype, gate=True, seed=32, device=DEV,
                     A_kind=A_kind, initial_state=True, delta_softplus=False, with_bias=False)
    p.delta = torch.full_like(p.delta, 1000.0)
    out, last = ssm_scan_fwd(**p.tensors(), delta_softplus=False, return_last_state=True)
    torch.cuda.synchronize()
    # closed form of the last state: (Delta x_L[d]) B_L[n], rounded in that
    # order (every earlier contribution is multiplied by an exact 0)
    xl = p.x[0, -1].float()
    bl = p.B[0, -1].float()
    expect = ((1000.0 * xl)[:, None] * bl[None, :])[None]
    assert torch.equal(last, expect), "the last state must be (1000 x_L) B_L exactly"
    ref, ref_last = oracle_for(p)
    # out_t = (Delta x_t (C_t . B_t) + D x_t) silu(z_t): the N products
    # Delta x C_n B_n are ~10^3-10^4 and often nearly cancel, so besides the
    # stated tolerance the float32 sum over n may be off by its own rounding,
    # at most 2 N 2^-24 sum_n |Delta x C_n B_n| (times the gate)
    h = p.host_f32()
    mag = 1000.0 * np.abs(h["x"]) * np.sum(np.abs(h["C"] * h["B"]), axis=-1, keepdims=True)
    gate = np.abs(h["z"] / (1.0 + np.exp(-h["z"].astype(np.float64))))
    rtol, atol = TOL[dtype]
    got = to_np(out)
    tol = atol + rtol * np.abs(ref) + 2 * 16 * 2.0 ** -24 * mag * gate
    bad = np.abs(got - ref) > tol
    assert not bad.any(), "reset out: %d elements outside" % int(bad.sum())
    assert_close(to_np(last), ref_last, rtol, atol, what="reset last_state")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_limit_cumsum(dtype):
    """N = 1, A = 0, Delta = 1 (softplus off), B = C = 1, no skip, no gate:
    h_t = h_(t-1) + x_t and out = cumsum(x), exact for small integers (every
    partial sum is an integer below 2^24); bf16 outputs are the cumsum rounded
    to nearest even, so the comparison is bit for bit."""
    L, dim = LIMIT_L, 64
    g = torch.Generator(device="cpu")
    g.manual_seed(33)
    xs = torch.randint(-4, 5, (1, L, dim), generator=g).to(torch.float32)
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    x = xs.to(tdt).to(DEV)
    ones_tok = torch.ones(1, L, 1, dtype=tdt, device=DEV)
    out, last = ssm_scan_fwd(x, torch.ones_like(x), torch.zeros(dim, 1, device=DEV), ones_tok,
                             ones_tok.clone(), delta_softplus=False, return_last_state=True)
    torch.cuda.synchronize()
    cs = torch.cumsum(xs.double(), dim=1)
    np.testing.assert_array_equal(out.cpu().float().numpy(), cs.to(tdt).float().numpy())
    np.testing.assert_array_equal(last.cpu()[..., 0].numpy(), cs[:, -1].float().numpy())
    # the oracle agrees exactly
    ref, ref_last = oracle.scan(xs.numpy(), np.ones((1, L, dim), np.float32),
                                np.zeros((dim, 1), np.float32), np.ones((1, L, 1), np.float32),
                                np.ones((1, L, 1), np.float32), delta_softplus=False)
    np.testing.assert_array_equal(ref, cs.numpy())


@pytest.mark.parametrize("A_kind", ["s4d_real", "general"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_chunk_plans_agree(dtype, A_kind):
    """One input under several time splits (the library's own, 8-token
    chunks, 24-token chunks, 128- and 200-token chunks, one chunk per
    sequence): every result matches the oracle, and the splits match each
    other within twice the tolerance (each is within one tolerance of the
    exact result).  A carry or LDS race would show up here as a
    split-dependent result.  Chunks of 128 tokens and more take the B/C rows
    from the LDS staging buffers (bf16, S4D-real A); 777 tokens leave ragged
    last chunks (9 and 177 tokens: a pair of token groups plus a tail)."""
    p = make_problem(2, 777, 96, 16, dtype=dtype, gate=True, seed=34, device=DEV, A_kind=A_kind,
                     initial_state=True)
    ref, ref_last = oracle_for(p)
    rtol, atol = TOL[dtype]
    res = {}
    for cl in (0, 8, 24, 128, 200, 777):
        print("case: chunk_len", cl, dtype, A_kind, flush=True)
        out, last = ssm_scan_fwd_chunked(**p.tensors(), chunk_len=cl, return_last_state=True)
        torch.cuda.synchronize()
        assert_close(to_np(out), ref, rtol, atol, "chunk_len %d out" % cl)
        assert_close(to_np(last), ref_last, rtol, atol, "chunk_len %d last_state" % cl)
        res[cl] = (to_np(out), to_np(last))
    for cl in (8, 24, 128, 200, 777):
        assert_close(res[cl][0], res[0][0], 2 * rtol, 2 * atol, "chunk_len %d vs default" % cl)
        assert_close(res[cl][1], res[0][1], 2 * rtol, 2 * atol, "chunk_len %d vs default last" % cl)
