"""MI355X-native selective scan (Mamba-class SSM recurrence).

``ssm_scan_fwd`` / ``ssm_scan_fwd_varlen`` / ``ssm_state_update``, the gradient
``ssm_scan_bwd``, the SSD (Mamba-2) ``ssm_ssd_fwd`` and the
``ssm_causal_conv1d_*`` pair are thin bindings of the C ABI in
include/ssm_scan.h; the work runs in hand-written gfx950 HIP kernels
(libssm_scan.so, built in-tree).  ``workloads`` draws seeded synthetic inputs.
"""
_OPS = ("ssm_scan_fwd", "ssm_scan_fwd_chunked", "ssm_scan_fwd_chunked_workspace_bytes",
        "ssm_scan_fwd_noalloc",
        "ssm_scan_fwd_varlen", "ssm_state_update", "ssm_scan_fwd_workspace_bytes",
        "ssm_scan_fwd_varlen_workspace_bytes", "ssm_causal_conv1d_fwd", "ssm_causal_conv1d_update",
        "ssm_scan_bwd", "ssm_scan_bwd_workspace_bytes", "ssm_ssd_fwd", "ssm_ssd_fwd_workspace_bytes",
        "ssm_last_error", "ssm_abi_version",
        "load_library", "SsmError", "LIB_PATH", "EXPORTS")

__all__ = list(_OPS)


def __getattr__(name):
    # the binding (and the shared library) load on first use, so that the
    # input generators can be imported without the HIP library
    if name in _OPS:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
