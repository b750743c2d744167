"""MI355X-native scan primitives: element-scan, matrix-scan, linear-scan and table-scan on gfx950.

The computation lives in ``libsx_scan.so`` (hand-written HIP kernels behind
the C ABI in ``include/sx_scan.h``); this package is its Python binding.
PyTorch provides device memory and streams.
"""

from ._binding import (BODIES, SxError, cumsum, element_scan, element_scan_backward, linear_scan, load_library,
                       matrix_scan, matrix_scan_backward, matrix_scan_status, set_lookback_spin_limit, table_scan)

__all__ = ["BODIES", "SxError", "element_scan", "element_scan_backward", "matrix_scan", "matrix_scan_backward",
           "linear_scan", "cumsum", "table_scan", "load_library", "matrix_scan_status", "set_lookback_spin_limit"]
__version__ = "0.1.0"
