"""The allocation-free matrix-scan entry point (sx_matrix_scan_noalloc) against
sx_matrix_scan, through the C ABI.

sx_matrix_scan_noalloc keeps its look-back state in a fixed device array
instead of a caller's workspace; its results must be those of sx_matrix_scan
on the same inputs, to the matrix-scan bar (1e-4 relative to the state for f32
operands, 2e-2 for bf16). Two calls in a row, the second on a smaller input,
so that the second runs on the array as the first left it.
"""

import pytest
import torch

from scan_primitives_amd import _binding as B
from scan_primitives_amd import workloads as W
from tests.helpers import MS_TOL_BF16, MS_TOL_F32, assert_matrix_close, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc(lib, a, b, axis, reverse, out):
    i64 = B.i64_array
    code = B._DTYPES[a.dtype]
    return lib.sx_matrix_scan_noalloc(code, a.dim(), i64(a.shape), i64(a.stride()), a.data_ptr(), b.dim(),
                                      i64(b.shape), i64(b.stride()), b.data_ptr(), axis, 1 if reverse else 0, 0,
                                      B._DTYPES[out.dtype], out.data_ptr(), B._stream_handle(a.device))


def test_noalloc_matches_matrix_scan_on_two_calls():
    import scan_primitives_amd as sx
    lib = B.load_library()
    cases = [W.make_matrix(32, 8192, 16, 1, torch.float32, seed=4),                  # the f32 m = 1 workload
             W.make_matrix(3, 700, 16, 16, torch.bfloat16, reverse=True, seed=431)]  # then a smaller one
    for w in cases:
        print(f"\n[case] allocation-free: {w.name}", flush=True)
        t = w.on(DEV)
        a, b = t["a"], t["b"]
        ref = sx.matrix_scan(a, b, axis=w.axis, reverse=w.reverse)
        out = torch.empty_like(ref)
        st = _noalloc(lib, a, b, w.axis, w.reverse, out)
        assert st == 0, lib.sx_last_error()
        torch.cuda.synchronize()
        tol = MS_TOL_F32 if a.dtype == torch.float32 else MS_TOL_BF16
        assert_matrix_close(out, ref.float().cpu().double().numpy(), tol)  # against the existing entry point
        assert_matrix_close(out, run_oracle(w), tol)                          # and against the oracle


def test_noalloc_rejects_state_beyond_its_array():
    lib = B.load_library()
    a = torch.zeros(64, 8192, 16, 16, device=DEV)  # 26 MiB of look-back state, beyond the 16 MiB array
    b = torch.zeros(64, 8192, 16, 1, device=DEV)
    out = torch.empty_like(b)
    assert _noalloc(lib, a, b, 1, False, out) == B.SX_E_WORKSPACE
    assert b"allocation-free" in lib.sx_last_error()
