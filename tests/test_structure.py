"""Structural checks of the GPU forward: every output written, nothing
written past the ends, bitwise run-to-run determinism, causality, resume from
last_state, and host-side rejection of bad calls on real device buffers."""
import numpy as np
import pytest
import torch

from selective_state_space_31_amd import SsmError, ssm_scan_fwd, ssm_scan_fwd_chunked
from selective_state_space_31_amd.workloads import make_problem
from tests._helpers import TOL, assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_every_output_written_and_no_overrun(dtype):
    p = make_problem(3, 101, 70, 16, dtype=dtype, seed=41, device=DEV, initial_state=True)
    tdt = p.x.dtype
    guard = 4096
    buf = torch.full((3 * 101 * 70 + 2 * guard,), float("nan"), dtype=tdt, device=DEV)
    out = buf[guard:guard + 3 * 101 * 70].view(3, 101, 70)
    sbuf = torch.full((3 * 70 * 16 + 2 * guard,), 12345.0, dtype=torch.float32, device=DEV)
    last = sbuf[guard:guard + 3 * 70 * 16].view(3, 70, 16)
    ssm_scan_fwd(**p.tensors(), out=out, last_state=last)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert torch.isnan(buf[:guard].float()).all() and torch.isnan(buf[-guard:].float()).all()
    assert (sbuf[:guard] == 12345.0).all() and (sbuf[-guard:] == 12345.0).all()
    assert (last != 12345.0).any()


def test_bitwise_deterministic():
    p = make_problem(2, 513, 200, 16, dtype="bf16", seed=42, device=DEV, initial_state=True)
    o1, l1 = ssm_scan_fwd(**p.tensors(), return_last_state=True)
    o2, l2 = ssm_scan_fwd(**p.tensors(), return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bitwise_deterministic_staged_long_chunks():
    """A plan of 512-token chunks in groups (the long-context layer's), whose
    summary and output walks take B/C from the LDS staging buffers: three
    runs bit for bit equal."""
    p = make_problem(1, 32768, 2048, 16, dtype="bf16", gate=False, seed=44, device=DEV,
                     engine="torch_cuda")
    first = None
    for _ in range(3):
        o, l = ssm_scan_fwd_chunked(**p.tensors(), chunk_len=512, return_last_state=True)
        torch.cuda.synchronize()
        if first is None:
            first = (o, l)
        else:
            assert torch.equal(o, first[0]) and torch.equal(l, first[1])


def test_causal():
    p = make_problem(1, 300, 64, 16, dtype="fp32", seed=43, device=DEV)
    base = ssm_scan_fwd(**p.tensors())
    for s in (0, 1, 150, 299):
        x2 = p.x.clone()
        x2[:, s] += 1.0
        t = p.tensors()
        t["x"] = x2
        pert = ssm_scan_fwd(**t)
        torch.cuda.synchronize()
        assert torch.equal(pert[:, :s], base[:, :s]), s
        assert not torch.equal(pert[:, s], base[:, s])


@pytest.mark.parametrize("L1", [1, 64, 200])
def test_resume_from_last_state(L1):
    p = make_problem(2, 333, 96, 16, dtype="fp32", seed=44, device=DEV, initial_state=True)
    full, full_last = ssm_scan_fwd(**p.tensors(), return_last_state=True)
    t = p.tensors()
    cut = lambda a, sl: a[:, sl].contiguous()
    first = dict(t, x=cut(p.x, slice(0, L1)), delta=cut(p.delta, slice(0, L1)), z=cut(p.z, slice(0, L1)),
                 B=cut(p.B, slice(0, L1)), C=cut(p.C, slice(0, L1)))
    o1, l1 = ssm_scan_fwd(**first, return_last_state=True)
    second = dict(t, x=cut(p.x, slice(L1, None)), delta=cut(p.delta, slice(L1, None)),
                  z=cut(p.z, slice(L1, None)), B=cut(p.B, slice(L1, None)), C=cut(p.C, slice(L1, None)),
                  initial_state=l1)
    o2, l2 = ssm_scan_fwd(**second, return_last_state=True)
    torch.cuda.synchronize()
    assert_close(to_np(torch.cat([o1, o2], 1)), to_np(full), *TOL["fp32"], what="split out")
    assert_close(to_np(l2), to_np(full_last), *TOL["fp32"], what="split state")


def test_resume_in_place_state():
    p = make_problem(2, 50, 64, 16, dtype="fp32", seed=45, device=DEV, initial_state=True)
    ref_out, ref_last = ssm_scan_fwd(**p.tensors(), return_last_state=True)
    st = p.h0.clone()
    t = p.tensors()
    t["initial_state"] = st
    o = ssm_scan_fwd(**t, last_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o[0], ref_out) and torch.equal(st, ref_last)


def test_alias_rejected_on_device_buffers():
    p = make_problem(1, 10, 64, 16, dtype="fp32", seed=46, device=DEV)
    with pytest.raises(SsmError) as e:
        ssm_scan_fwd(**p.tensors(), out=p.x)
    assert e.value.code == -5
