"""Float64 CPU oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path never does.
"""
from .oracle import build, scan, scan_varlen, state_update, oracle_lib_path  # noqa: F401
from .conv import conv1d_fwd, conv1d_update, conv_lib_path  # noqa: F401
from .conv import build as build_conv  # noqa: F401
from .bwd import scan_bwd, bwd_lib_path  # noqa: F401
from .bwd import build as build_bwd  # noqa: F401
from .ssd import ssd_scan, ssd_lib_path  # noqa: F401
from .ssd import build as build_ssd  # noqa: F401
