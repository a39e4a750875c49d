"""ctypes wrapper around ``conv_oracle.c`` -- TEST INFRASTRUCTURE ONLY.

The causal depthwise convolution (+ SiLU) before the scan, in float64 (see
the C file's header for what it computes and the passage it follows).  This
module builds it with gcc and marshals numpy arrays; it imports nothing from
the HIP package.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "libconv_oracle.so")
_libs = {}


def conv_lib_path():
    return _LIB


def build(force=False):
    """Compile the convolution oracle with gcc (-O2, IEEE double)."""
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
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.conv_oracle_fwd.argtypes = [P, P, P, ctypes.c_int, P, P, P, I64, I64, I64, I64]
        lib.conv_oracle_fwd.restype = ctypes.c_int
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


def conv1d_fwd(x, weight, bias=None, silu=True, initial_state=None, lib_path=None):
    """x (batch, L, dim), weight (dim, W), bias (dim,), initial_state
    (batch, dim, W-1).  Returns (out (batch, L, dim), final_state
    (batch, dim, W-1)) as float64."""
    x = np.asarray(x)
    batch, L, dim = x.shape
    W = np.asarray(weight).shape[1]
    x = _f32(x, (batch, L, dim), "x")
    weight = _f32(weight, (dim, W), "weight")
    bias = _f32(bias, (dim,), "bias")
    initial_state = _f32(initial_state, (batch, dim, W - 1), "initial_state")
    out = np.empty((batch, L, dim))
    state1 = np.empty((batch, dim, W - 1))
    rc = _load(lib_path).conv_oracle_fwd(_p(x), _p(weight), _p(bias), int(bool(silu)),
                                         _p(initial_state), _p(out), _p(state1), batch, L, dim, W)
    if rc != 0:
        raise RuntimeError("conv_oracle_fwd failed with code %d" % rc)
    return out, state1


def conv1d_update(state, x, weight, bias=None, silu=True):
    """One decoding step: state (batch, dim, W-1), x (batch, dim).  Returns
    (out (batch, dim), new_state (batch, dim, W-1)) as float64."""
    x = np.asarray(x, dtype=np.float32)
    out, st = conv1d_fwd(x[:, None, :], weight, bias, silu, initial_state=state)
    return out[:, 0, :], st
