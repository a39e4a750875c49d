"""ctypes wrapper around ``ssd_oracle.c`` -- TEST INFRASTRUCTURE ONLY.

The SSD (Mamba-2) form of the selective scan in float64 (see the C file's
header for what is computed and the passages it follows).  This module
builds it with gcc and marshals numpy arrays; it imports nothing from the
HIP package.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_libs = {}


def ssd_lib_path():
    return _LIB


def build(force=False):
    """Compile the SSD oracle with gcc (-O2, IEEE double)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load(lib_path=None):
    path = lib_path or build()
    if path not in _libs:
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.ssd_oracle_fwd.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64,
                                       I64]
        lib.ssd_oracle_fwd.restype = I
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


def ssd_scan(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
             lib_path=None):
    """x, z (batch, L, heads, headdim); dt (batch, L, heads); A, D, dt_bias
    (heads,); B, C (batch, L, groups, dstate); h0 (batch, heads, headdim,
    dstate).  Returns (out, last_state) in float64."""
    x = np.asarray(x)
    batch, L, H, P = x.shape
    G, N = np.asarray(B).shape[2:]
    x = _f32(x, (batch, L, H, P), "x")
    dt = _f32(dt, (batch, L, H), "dt")
    A = _f32(A, (H,), "A")
    B = _f32(B, (batch, L, G, N), "B")
    C = _f32(C, (batch, L, G, N), "C")
    D = _f32(D, (H,), "D")
    z = _f32(z, (batch, L, H, P), "z")
    dt_bias = _f32(dt_bias, (H,), "dt_bias")
    h0 = _f32(h0, (batch, H, P, N), "h0")
    out = np.empty((batch, L, H, P))
    last = np.empty((batch, H, P, N))
    rc = _load(lib_path).ssd_oracle_fwd(_p(x), _p(dt), _p(dt_bias), int(bool(dt_softplus)), _p(A),
                                        _p(B), _p(C), _p(D), _p(z), _p(h0), _p(out), _p(last),
                                        batch, L, H, P, N, G)
    if rc != 0:
        raise RuntimeError("ssd_oracle_fwd failed with code %d" % rc)
    return out, last
