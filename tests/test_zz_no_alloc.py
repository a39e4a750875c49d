"""ssm_scan_fwd_noalloc: the forward with the library's own device scratch
instead of a caller workspace.

Through the C ABI, two calls in a row -- a large input, then a smaller one
that reuses the scratch the first left behind -- each checked against
ssm_scan_fwd on the same inputs (same plan and kernels: equal bit for bit)
and against the float64 oracle where it is small enough to run whole."""
import ctypes

import numpy as np
import pytest
import torch

from selective_state_space_31_amd import ops
from selective_state_space_31_amd.workloads import CONFIGS, make_problem
from tests._helpers import TOL, assert_close, oracle_for, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def noalloc(p, out, last):
    """Direct C call: the binding below allocates nothing either."""
    lib = ops.load_library()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    b, L, dim = p.x.shape
    N = p.A.shape[1]
    rc = lib.ssm_scan_fwd_noalloc(P(p.x), P(p.delta), P(p.delta_bias), 1, P(p.A), P(p.B), P(p.C),
                                  P(p.D), P(p.z), P(out), P(last), P(p.h0), b, L, dim, N,
                                  ops._DTYPES[p.x.dtype],
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, ops.ssm_last_error()


def check_pair(p, what, with_oracle):
    print("case:", what, flush=True)
    b, L, dim = p.x.shape
    N = p.A.shape[1]
    out = torch.full_like(p.x, float("nan"))
    last = torch.full((b, dim, N), float("nan"), device=DEV)
    noalloc(p, out, last)
    ref_out, ref_last = ops.ssm_scan_fwd(**p.tensors(), return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), what + ": out differs from ssm_scan_fwd"
    assert torch.equal(last, ref_last), what + ": last_state differs from ssm_scan_fwd"
    if with_oracle:
        r, rl = oracle_for(p)
        assert_close(to_np(out), r, *TOL[p.dtype], what=what + " out")
        assert_close(to_np(last), rl, *TOL[p.dtype], what=what + " last_state")


def test_noalloc_two_calls_large_then_small():
    c = dict(CONFIGS["mamba130m_bf16"])
    big = make_problem(**c, seed=3, device=DEV, engine="torch_cuda", initial_state=True)
    assert ops.ssm_scan_fwd_workspace_bytes(4, 2048, 1536, 16, torch.bfloat16) > 0
    check_pair(big, "noalloc 4x2048x1536 bf16 (130M-shaped)", with_oracle=False)
    small = make_problem(1, 700, 96, 16, dtype="fp32", seed=4, device=DEV, initial_state=True,
                         A_kind="general")
    assert ops.ssm_scan_fwd_workspace_bytes(1, 700, 96, 16, torch.float32) > 0
    check_pair(small, "noalloc 1x700x96 fp32, after the large call", with_oracle=True)


def test_noalloc_without_scratch_and_sequence_split():
    # one chunk per sequence (no scratch needed) and an empty sequence
    p = make_problem(64, 40, 1536, 16, dtype="bf16", seed=5, device=DEV, initial_state=True)
    check_pair(p, "noalloc 64x40x1536 bf16", with_oracle=True)
    e = make_problem(2, 0, 64, 16, dtype="fp32", seed=6, device=DEV, initial_state=True)
    out = torch.empty_like(e.x)
    last = torch.empty(2, 64, 16, device=DEV)
    noalloc(e, out, last)
    torch.cuda.synchronize()
    assert torch.equal(last, e.h0)
