"""Thin Python binding of the C ABI in include/ssm_scan.h.

Argument marshalling only: every step of the scan runs in the HIP kernels of
libssm_scan.so.  PyTorch supplies device memory and the current HIP stream.
The functions keep the C names.  If the library is missing the import of the
first call fails loudly; there is no fallback implementation.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_scan.so")

SSM_DTYPE_F32 = 0
SSM_DTYPE_BF16 = 1
_DTYPES = {torch.float32: SSM_DTYPE_F32, torch.bfloat16: SSM_DTYPE_BF16}

STATUS = {0: "SSM_OK", -1: "SSM_ERR_NULL", -2: "SSM_ERR_SHAPE", -3: "SSM_ERR_UNSUPPORTED",
          -4: "SSM_ERR_ALIGN", -5: "SSM_ERR_ALIAS", -6: "SSM_ERR_WORKSPACE", -7: "SSM_ERR_HIP"}

EXPORTS = ("ssm_scan_fwd", "ssm_scan_fwd_workspace_bytes", "ssm_scan_fwd_chunked",
           "ssm_scan_fwd_chunked_workspace_bytes", "ssm_scan_fwd_noalloc", "ssm_scan_fwd_varlen",
           "ssm_scan_fwd_varlen_workspace_bytes", "ssm_state_update", "ssm_causal_conv1d_fwd",
           "ssm_causal_conv1d_update", "ssm_scan_bwd", "ssm_scan_bwd_workspace_bytes",
           "ssm_ssd_fwd", "ssm_ssd_fwd_workspace_bytes", "ssm_last_error", "ssm_abi_version")


class SsmError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


_lib = None


def load_library(path=LIB_PATH):
    """Load libssm_scan.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libssm_scan.so not found at %s: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')" % path)
    lib = ctypes.CDLL(path)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.ssm_scan_fwd.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]
    lib.ssm_scan_fwd.restype = I
    lib.ssm_scan_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.ssm_scan_fwd_workspace_bytes.restype = SZ
    lib.ssm_scan_fwd_chunked.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I,
                                         I64, P, SZ, P]
    lib.ssm_scan_fwd_chunked.restype = I
    lib.ssm_scan_fwd_chunked_workspace_bytes.argtypes = [I64, I64, I64, I64, I, I64]
    lib.ssm_scan_fwd_chunked_workspace_bytes.restype = SZ
    lib.ssm_scan_fwd_noalloc.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I, P]
    lib.ssm_scan_fwd_noalloc.restype = I
    lib.ssm_scan_fwd_varlen.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64,
                                        I, P, SZ, P]
    lib.ssm_scan_fwd_varlen.restype = I
    lib.ssm_scan_fwd_varlen_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.ssm_scan_fwd_varlen_workspace_bytes.restype = SZ
    lib.ssm_state_update.argtypes = [P, P, P, P, I, P, P, P, P, P, P, I64, I64, I64, I, P]
    lib.ssm_state_update.restype = I
    lib.ssm_causal_conv1d_fwd.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I, I, P]
    lib.ssm_causal_conv1d_fwd.restype = I
    lib.ssm_causal_conv1d_update.argtypes = [P, P, P, P, P, I64, I64, I64, I, I, P]
    lib.ssm_causal_conv1d_update.restype = I
    lib.ssm_scan_bwd.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                 I64, I64, I64, I64, I, P, SZ, P]
    lib.ssm_scan_bwd.restype = I
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I]
    lib.ssm_scan_bwd_workspace_bytes.restype = SZ
    lib.ssm_ssd_fwd.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I,
                                P, SZ, P]
    lib.ssm_ssd_fwd.restype = I
    lib.ssm_ssd_fwd_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I64]
    lib.ssm_ssd_fwd_workspace_bytes.restype = SZ
    lib.ssm_last_error.argtypes = []
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_abi_version.argtypes = []
    lib.ssm_abi_version.restype = I
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _raise(code):
    msg = load_library().ssm_last_error().decode(errors="replace")
    raise SsmError(code, msg)


def ssm_abi_version():
    return load_library().ssm_abi_version()


def ssm_last_error():
    return load_library().ssm_last_error().decode(errors="replace")


def ssm_scan_fwd_workspace_bytes(batch, seqlen, dim, dstate, dtype=torch.bfloat16):
    return int(load_library().ssm_scan_fwd_workspace_bytes(batch, seqlen, dim, dstate, _DTYPES[dtype]))


def ssm_scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 initial_state=None, return_last_state=False, out=None, last_state=None,
                 workspace=None, stream=None):
    """Selective scan forward over (batch, seqlen, dim) activations.

    Returns ``out`` (same dtype as x), or ``(out, last_state)`` when
    ``return_last_state`` is set (or a ``last_state`` buffer is passed).
    """
    return _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, initial_state,
                     return_last_state, out, last_state, workspace, stream, 0)


def ssm_scan_fwd_chunked_workspace_bytes(batch, seqlen, dim, dstate, chunk_len,
                                         dtype=torch.bfloat16):
    return int(load_library().ssm_scan_fwd_chunked_workspace_bytes(batch, seqlen, dim, dstate,
                                                                   _DTYPES[dtype], chunk_len))


def ssm_scan_fwd_chunked(x, delta, A, B, C, chunk_len, D=None, z=None, delta_bias=None,
                         delta_softplus=True, initial_state=None, return_last_state=False,
                         out=None, last_state=None, workspace=None, stream=None):
    """``ssm_scan_fwd`` with the sequence cut into chunks of ``chunk_len``
    tokens (0 = the library's choice; >= seqlen = one chunk)."""
    return _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, initial_state,
                     return_last_state, out, last_state, workspace, stream, int(chunk_len))


def ssm_scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                         initial_state=None, out=None, last_state=None, stream=None):
    """``ssm_scan_fwd`` with the library's own device scratch instead of a
    workspace (the C call allocates nothing; ``out`` and ``last_state`` are
    allocated here only when not passed).  Calls overlapping in time on one
    device race on that scratch."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    batch, L, dim = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    _check(x, "x", (batch, L, dim), dt, dev)
    _check(delta, "delta", (batch, L, dim), dt, dev)
    _check(z, "z", (batch, L, dim), dt, dev, optional=True)
    _check(B, "B", (batch, L, N), dt, dev)
    _check(C, "C", (batch, L, N), dt, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev, optional=True)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    _check(initial_state, "initial_state", (batch, dim, N), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty((batch, L, dim), dtype=dt, device=dev)
    _check(out, "out", (batch, L, dim), dt, dev)
    _check(last_state, "last_state", (batch, dim, N), torch.float32, dev, optional=True)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_fwd_noalloc(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                  _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(out),
                                  _ptr(last_state), _ptr(initial_state), batch, L, dim, N,
                                  _DTYPES[dt], ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if last_state is not None:
        return out, last_state
    return out


def _scan_fwd(x, delta, A, B, C, D, z, delta_bias, delta_softplus, initial_state,
              return_last_state, out, last_state, workspace, stream, chunk_len):
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    batch, L, dim = x.shape
    if A.dim() != 2:
        raise ValueError("A must be (dim, dstate)")
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    _check(x, "x", (batch, L, dim), dt, dev)
    _check(delta, "delta", (batch, L, dim), dt, dev)
    _check(z, "z", (batch, L, dim), dt, dev, optional=True)
    _check(B, "B", (batch, L, N), dt, dev)
    _check(C, "C", (batch, L, N), dt, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev, optional=True)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    _check(initial_state, "initial_state", (batch, dim, N), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty((batch, L, dim), dtype=dt, device=dev)
    _check(out, "out", (batch, L, dim), dt, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (batch, dim, N), torch.float32, dev, optional=True)
    need = int(lib.ssm_scan_fwd_chunked_workspace_bytes(batch, L, dim, N, _DTYPES[dt], chunk_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_fwd_chunked(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                  _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(out),
                                  _ptr(last_state), _ptr(initial_state), batch, L, dim, N,
                                  _DTYPES[dt], chunk_len, _ptr(workspace), ws_bytes,
                                  ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if last_state is not None:
        return out, last_state
    return out


def ssm_scan_fwd_varlen_workspace_bytes(nseq, total_len, dim, dstate, dtype=torch.bfloat16):
    return int(load_library().ssm_scan_fwd_varlen_workspace_bytes(nseq, total_len, dim, dstate,
                                                                  _DTYPES[dtype]))


def ssm_scan_fwd_varlen(x, delta, A, B, C, cu_seqlens, D=None, z=None, delta_bias=None,
                        delta_softplus=True, initial_state=None, return_last_state=False, out=None,
                        last_state=None, workspace=None, stream=None):
    """Selective scan forward over packed sequences: x (total_len, dim),
    B/C (total_len, dstate), cu_seqlens (nseq + 1) int32 offsets on the
    device; states are (nseq, dim, dstate).

    Returns ``out``, or ``(out, last_state)`` as ``ssm_scan_fwd`` does.
    """
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be (total_len, dim)")
    T, dim = x.shape
    if A.dim() != 2:
        raise ValueError("A must be (dim, dstate)")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be (nseq + 1,) with nseq >= 1")
    nseq = cu_seqlens.numel() - 1
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    _check(x, "x", (T, dim), dt, dev)
    _check(delta, "delta", (T, dim), dt, dev)
    _check(z, "z", (T, dim), dt, dev, optional=True)
    _check(B, "B", (T, N), dt, dev)
    _check(C, "C", (T, N), dt, dev)
    _check(cu_seqlens, "cu_seqlens", (nseq + 1,), torch.int32, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev, optional=True)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    _check(initial_state, "initial_state", (nseq, dim, N), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty((T, dim), dtype=dt, device=dev)
    _check(out, "out", (T, dim), dt, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((nseq, dim, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (nseq, dim, N), torch.float32, dev, optional=True)
    need = int(lib.ssm_scan_fwd_varlen_workspace_bytes(nseq, T, dim, N, _DTYPES[dt]))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_fwd_varlen(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                 _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(out),
                                 _ptr(last_state), _ptr(initial_state), _ptr(cu_seqlens), nseq, T,
                                 dim, N, _DTYPES[dt], _ptr(workspace), ws_bytes,
                                 ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if last_state is not None:
        return out, last_state
    return out


def ssm_state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=True, out=None, stream=None):
    """One decode step: ``state`` (batch, dim, dstate) float32 is updated in
    place; returns ``out`` (batch, dim) in x's dtype."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be (batch, dim)")
    batch, dim = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    _check(state, "state", (batch, dim, N), torch.float32, dev)
    _check(x, "x", (batch, dim), dt, dev)
    _check(delta, "delta", (batch, dim), dt, dev)
    _check(z, "z", (batch, dim), dt, dev, optional=True)
    _check(B, "B", (batch, N), dt, dev)
    _check(C, "C", (batch, N), dt, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev, optional=True)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty((batch, dim), dtype=dt, device=dev)
    _check(out, "out", (batch, dim), dt, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_state_update(_ptr(state), _ptr(x), _ptr(delta), _ptr(delta_bias),
                              int(bool(delta_softplus)), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(out), batch, dim, N, _DTYPES[dt], ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return out


def ssm_causal_conv1d_fwd(x, weight, bias=None, initial_conv_state=None, silu=True,
                          return_final_state=False, out=None, final_conv_state=None, stream=None):
    """Causal depthwise convolution (+ SiLU) over (batch, seqlen, dim)
    activations; weight (dim, width) float32, conv states (batch, dim,
    width-1) in x's dtype.  Returns ``out``, or ``(out, final_conv_state)``."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    batch, L, dim = x.shape
    if weight.dim() != 2:
        raise ValueError("weight must be (dim, width)")
    W = weight.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    _check(x, "x", (batch, L, dim), dt, dev)
    _check(weight, "weight", (dim, W), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev, optional=True)
    _check(initial_conv_state, "initial_conv_state", (batch, dim, W - 1), dt, dev, optional=True)
    if out is None:
        out = torch.empty((batch, L, dim), dtype=dt, device=dev)
    _check(out, "out", (batch, L, dim), dt, dev)
    if final_conv_state is None and return_final_state:
        final_conv_state = torch.empty((batch, dim, W - 1), dtype=dt, device=dev)
    _check(final_conv_state, "final_conv_state", (batch, dim, W - 1), dt, dev, optional=True)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(initial_conv_state),
                                   _ptr(out), _ptr(final_conv_state), batch, L, dim, W,
                                   int(bool(silu)), _DTYPES[dt], ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if final_conv_state is not None:
        return out, final_conv_state
    return out


def ssm_causal_conv1d_update(conv_state, x, weight, bias=None, silu=True, out=None, stream=None):
    """One decoding step: ``conv_state`` (batch, dim, width-1) in x's dtype is
    shifted in place; returns ``out`` (batch, dim)."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be (batch, dim)")
    batch, dim = x.shape
    W = weight.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    _check(conv_state, "conv_state", (batch, dim, W - 1), dt, dev)
    _check(x, "x", (batch, dim), dt, dev)
    _check(weight, "weight", (dim, W), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty((batch, dim), dtype=dt, device=dev)
    _check(out, "out", (batch, dim), dt, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_causal_conv1d_update(_ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias),
                                      _ptr(out), batch, dim, W, int(bool(silu)), _DTYPES[dt],
                                      ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return out


def ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, dtype=torch.bfloat16):
    return int(load_library().ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate,
                                                           _DTYPES[dtype]))


def ssm_scan_bwd(x, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=True,
                 initial_state=None, dlast_state=None, grads=None, workspace=None, stream=None):
    """Gradients of ``ssm_scan_fwd`` for the loss sum(dout*out) +
    sum(dlast_state*last_state).  Returns a dict: dx, ddelta, dz (None
    without z) in x's dtype; dA, dB, dC, dD (None without D), ddelta_bias,
    dinitial_state in float32.  ``grads`` may supply preallocated outputs
    under the same keys."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, dim)")
    batch, L, dim = x.shape
    N = A.shape[1]
    dev, dt = x.device, x.dtype
    if dt not in _DTYPES:
        raise TypeError("activations must be float32 or bfloat16, got %s" % dt)
    f32 = torch.float32
    _check(x, "x", (batch, L, dim), dt, dev)
    _check(delta, "delta", (batch, L, dim), dt, dev)
    _check(z, "z", (batch, L, dim), dt, dev, optional=True)
    _check(dout, "dout", (batch, L, dim), dt, dev)
    _check(B, "B", (batch, L, N), dt, dev)
    _check(C, "C", (batch, L, N), dt, dev)
    _check(A, "A", (dim, N), f32, dev)
    _check(D, "D", (dim,), f32, dev, optional=True)
    _check(delta_bias, "delta_bias", (dim,), f32, dev, optional=True)
    _check(initial_state, "initial_state", (batch, dim, N), f32, dev, optional=True)
    _check(dlast_state, "dlast_state", (batch, dim, N), f32, dev, optional=True)
    g = dict(grads or {})
    shapes = dict(dx=((batch, L, dim), dt), ddelta=((batch, L, dim), dt),
                  dz=((batch, L, dim), dt) if z is not None else None, dA=((dim, N), f32),
                  dB=((batch, L, N), f32), dC=((batch, L, N), f32),
                  dD=((dim,), f32) if D is not None else None, ddelta_bias=((dim,), f32),
                  dinitial_state=((batch, dim, N), f32))
    for k, sd in shapes.items():
        if sd is None:
            g[k] = None
            continue
        if g.get(k) is None:
            g[k] = torch.empty(sd[0], dtype=sd[1], device=dev)
        _check(g[k], k, sd[0], sd[1], dev)
    need = int(lib.ssm_scan_bwd_workspace_bytes(batch, L, dim, N, _DTYPES[dt]))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_bwd(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                          _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(initial_state),
                          _ptr(dout), _ptr(dlast_state), _ptr(g["dx"]), _ptr(g["ddelta"]),
                          _ptr(g["dz"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                          _ptr(g["dD"]), _ptr(g["ddelta_bias"]), _ptr(g["dinitial_state"]),
                          batch, L, dim, N, _DTYPES[dt], _ptr(workspace), ws_bytes,
                          ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    return g


def ssm_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups=1):
    return int(load_library().ssm_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, dstate,
                                                          ngroups))


def ssm_ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
                initial_state=None, return_last_state=False, out=None, last_state=None,
                workspace=None, stream=None):
    """SSD (Mamba-2) forward: x, z (batch, seqlen, nheads, headdim) bf16;
    dt (batch, seqlen, nheads) bf16; A, D, dt_bias (nheads,) float32; B, C
    (batch, seqlen, ngroups, dstate) bf16; states (batch, nheads, headdim,
    dstate) float32.  Returns ``out`` or ``(out, last_state)``."""
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim), B (batch, seqlen, ngroups, dstate)")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev, dt_ = x.device, x.dtype
    if dt_ != torch.bfloat16:
        raise TypeError("ssm_ssd_fwd takes bfloat16 activations, got %s" % dt_)
    f32 = torch.float32
    _check(x, "x", (batch, L, H, P), dt_, dev)
    _check(dt, "dt", (batch, L, H), dt_, dev)
    _check(z, "z", (batch, L, H, P), dt_, dev, optional=True)
    _check(B, "B", (batch, L, G, N), dt_, dev)
    _check(C, "C", (batch, L, G, N), dt_, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev, optional=True)
    _check(dt_bias, "dt_bias", (H,), f32, dev, optional=True)
    _check(initial_state, "initial_state", (batch, H, P, N), f32, dev, optional=True)
    if out is None:
        out = torch.empty((batch, L, H, P), dtype=dt_, device=dev)
    _check(out, "out", (batch, L, H, P), dt_, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, H, P, N), dtype=f32, device=dev)
    _check(last_state, "last_state", (batch, H, P, N), f32, dev, optional=True)
    need = int(lib.ssm_ssd_fwd_workspace_bytes(batch, L, H, P, N, G))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_ssd_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(A), _ptr(B),
                         _ptr(C), _ptr(D), _ptr(z), _ptr(out), _ptr(last_state),
                         _ptr(initial_state), batch, L, H, P, N, G, _DTYPES[dt_], _ptr(workspace),
                         ws_bytes, ctypes.c_void_p(stream))
    if rc != 0:
        _raise(rc)
    if last_state is not None:
        return out, last_state
    return out
