"""ctypes wrapper around ``ssm_oracle_bwd.c`` -- TEST INFRASTRUCTURE ONLY.

Float64 gradients of the selective scan (see the C file's header for what is
computed and the passages it follows).  This module builds the C file with
gcc and marshals numpy arrays; it imports nothing from the HIP package.
"""
import ctypes
import os
import subprocess

import numpy as np

from .oracle import default_threads

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle_bwd.c")
_LIB = os.path.join(_HERE, "libssm_oracle_bwd.so")
_libs = {}


def bwd_lib_path():
    return _LIB


def build(force=False):
    """Compile the gradient oracle with gcc (-O2, IEEE double)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load(lib_path=None):
    path = lib_path or build()
    if path not in _libs:
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.ssm_oracle_scan_bwd.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P,
                                            P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I]
        lib.ssm_oracle_scan_bwd.restype = I
        _libs[path] = lib
    return _libs[path]


def _f32(a, shape, name):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if tuple(a.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, a.shape, shape))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan_bwd(x, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, dlast=None, nthreads=None, lib_path=None):
    """Gradients of sum(dout*out) + sum(dlast*last_state) for the scan with
    these inputs (shapes as in ``oracle.scan``).  Returns a dict of float64
    arrays: dx, ddelta, dz (None without z), dB, dC (batch, L, N), dA (dim,
    N), dD, ddelta_bias (dim,), dh0 (batch, dim, N)."""
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
    dout = _f32(dout, (batch, L, dim), "dout")
    dlast = _f32(dlast, (batch, dim, N), "dlast")
    g = dict(dx=np.empty((batch, L, dim)), ddelta=np.empty((batch, L, dim)),
             dz=np.empty((batch, L, dim)) if z is not None else None,
             dB=np.empty((batch, L, N)), dC=np.empty((batch, L, N)), dA=np.empty((dim, N)),
             dD=np.empty(dim), ddelta_bias=np.empty(dim), dh0=np.empty((batch, dim, N)))
    rc = _load(lib_path).ssm_oracle_scan_bwd(
        _p(x), _p(delta), _p(delta_bias), int(bool(delta_softplus)), _p(A), _p(B), _p(C), _p(D),
        _p(z), _p(h0), _p(dout), _p(dlast), _p(g["dx"]), _p(g["ddelta"]), _p(g["dA"]), _p(g["dB"]),
        _p(g["dC"]), _p(g["dD"]), _p(g["dz"]), _p(g["ddelta_bias"]), _p(g["dh0"]), batch, L, dim, N,
        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("ssm_oracle_scan_bwd failed with code %d" % rc)
    return g
