"""ctypes wrapper around ``ssm_oracle.c`` -- TEST INFRASTRUCTURE ONLY.

The C file holds the whole computation (a sequential float64 loop written
from the pages; see its header).  This module only builds it with gcc,
marshals numpy arrays and picks a thread count.  It imports nothing from the
HIP package.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")
_lib = None


def oracle_lib_path():
    return _LIB


def build(force=False):
    """Compile the oracle with gcc (-O2, no fast-math: IEEE double throughout)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_alt_libs = {}


def _bind(path):
    lib = ctypes.CDLL(path)
    f = lib.ssm_oracle_scan
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    f.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_int]
    f.restype = ctypes.c_int
    return lib


def _load(lib_path=None):
    """The oracle library; ``lib_path`` loads another build of the same source
    (the pin tests use it to check that deliberately broken copies fail)."""
    global _lib
    if lib_path is not None:
        if lib_path not in _alt_libs:
            _alt_libs[lib_path] = _bind(lib_path)
        return _alt_libs[lib_path]
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def _f32(a, shape, name):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if tuple(a.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, a.shape, shape))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads():
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return max(1, min(n, 16))


def scan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
         h0=None, want_last_state=True, nthreads=None, lib_path=None):
    """Sequential float64 selective scan.

    x, delta, z: (batch, L, dim); B, C: (batch, L, N); A: (dim, N);
    D, delta_bias: (dim,); h0: (batch, dim, N).  Values are taken as float32
    (bf16 inputs must be passed already widened).  Returns (out, last_state)
    as float64 arrays of shapes (batch, L, dim) and (batch, dim, N).
    """
    x = np.asarray(x)
    batch, L, dim = x.shape
    N = np.asarray(A).shape[1]
    x = _f32(x, (batch, L, dim), "x")
    delta = _f32(delta, (batch, L, dim), "delta")
    A = _f32(A, (dim, N), "A")
    B = _f32(B, (batch, L, N), "B")
    C = _f32(C, (batch, L, N), "C")
    D = _f32(D, (dim,), "D")
    z = _f32(z, (batch, L, dim), "z")
    delta_bias = _f32(delta_bias, (dim,), "delta_bias")
    h0 = _f32(h0, (batch, dim, N), "h0")
    out = np.empty((batch, L, dim), dtype=np.float64)
    last = np.empty((batch, dim, N), dtype=np.float64) if want_last_state else None
    rc = _load(lib_path).ssm_oracle_scan(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                 _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                 _ptr(out), _ptr(last), batch, L, dim, N,
                                 int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("ssm_oracle_scan failed with code %d" % rc)
    return out, last


def state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 nthreads=None):
    """One decode step: the scan with L = 1 starting from ``state``.

    state: (batch, dim, N); x, delta, z: (batch, dim); B, C: (batch, N).
    Returns (out (batch, dim), new_state (batch, dim, N)) in float64.
    """
    x = np.asarray(x)
    batch, dim = x.shape
    N = np.asarray(A).shape[1]
    r = lambda a, s: None if a is None else np.asarray(a, dtype=np.float32).reshape(s)
    out, last = scan(r(x, (batch, 1, dim)), r(delta, (batch, 1, dim)), A,
                     r(B, (batch, 1, N)), r(C, (batch, 1, N)), D=D,
                     z=r(z, (batch, 1, dim)), delta_bias=delta_bias,
                     delta_softplus=delta_softplus, h0=state, nthreads=nthreads)
    return out[:, 0, :], last


def scan_varlen(x, delta, A, B, C, cu_seqlens, D=None, z=None, delta_bias=None,
                delta_softplus=True, h0=None, want_last_state=True, nthreads=None):
    """Packed variable-length sequences: the sequences are independent, each
    runs the scan above from its own initial state.

    x, delta, z: (total, dim); B, C: (total, N); cu_seqlens: nseq + 1 token
    offsets (sequence s is rows [cu[s], cu[s+1])); h0: (nseq, dim, N).
    Returns (out (total, dim), last_state (nseq, dim, N)) in float64.
    Follows "Linear Attention vs Softmax Attention: Can RWKV or Mamba Replace
    Transformers?", "Common Mistakes" and "Best Practices" item 4 (sequences
    concatenated without padding, with offsets) and "State Reset and
    Isolation" (each sequence starts from its own state).
    """
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    nseq = len(cu) - 1
    x = np.asarray(x, dtype=np.float32)
    total, dim = x.shape
    N = np.asarray(A).shape[1]
    if nseq < 1 or cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to total")
    tok = lambda a, s: None if a is None else np.asarray(a, dtype=np.float32)[cu[s]:cu[s + 1]][None]
    out = np.empty((total, dim), dtype=np.float64)
    last = np.empty((nseq, dim, N), dtype=np.float64) if want_last_state else None
    for s in range(nseq):
        o, l = scan(tok(x, s), tok(delta, s), A, tok(B, s), tok(C, s), D=D, z=tok(z, s),
                    delta_bias=delta_bias, delta_softplus=delta_softplus,
                    h0=None if h0 is None else np.asarray(h0, dtype=np.float32)[s:s + 1],
                    want_last_state=True, nthreads=nthreads)
        out[cu[s]:cu[s + 1]] = o[0]
        if last is not None:
            last[s] = l[0]
    return out, last
