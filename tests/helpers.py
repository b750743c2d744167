"""Shared helpers for the tests: run one workload on the GPU path or the oracle,
and the tolerance checks the parity tests apply."""

import numpy as np
import torch

import oracle
import scan_primitives_amd as sx

# Element-scan f32: |gpu - ref| <= ATOL + RTOL * |ref| elementwise, against the float64 oracle.
ES_ATOL = 1e-5
ES_RTOL = 1e-5
# Matrix-scan: ||gpu[t] - ref[t]||_F <= tol * ||ref[t]||_F for every state (n x m block).
MS_TOL_F32 = 1e-4
MS_TOL_BF16 = 2e-2


def run_gpu(w, dev):
    t = w.on(dev)
    if w.op == "element_scan":
        return sx.element_scan(w.body, t["initial"], [t["x"], t["s"]], axis=w.axis, state_axis=w.state_axis,
                               reverse=w.reverse)
    if w.op == "table_scan":
        return sx.table_scan(t["table"], t["symbols"], axis=w.axis, start=w.meta.get("start", 0))
    if w.op == "linear_scan":
        a = t["a"] if "a" in t else w.meta["a_number"]
        return sx.linear_scan(a, t["b"], axis=w.axis, reverse=w.reverse, out_dtype=w.out_dtype)
    return sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse, out_dtype=w.out_dtype)


def run_oracle(w, dtype=np.float64):
    t = w.tensors
    f = lambda v: v.float().numpy()  # noqa: E731  (bf16 and f32 widen exactly)
    if w.op == "element_scan":
        return oracle.element_scan(w.body, f(t["initial"]), [f(t["x"]), f(t["s"])], axis=w.axis,
                                   state_axis=w.state_axis, reverse=w.reverse, dtype=dtype)
    if w.op == "linear_scan":
        # a number takes the tensors' dtype, as the binding does
        a = f(t["a"]) if "a" in t else f(torch.tensor(w.meta["a_number"], dtype=t["b"].dtype))
        return oracle.linear_scan(a, f(t["b"]), axis=w.axis, reverse=w.reverse, dtype=dtype)
    return oracle.matrix_scan(f(t["a"]), f(t["b"]), axis=w.axis, reverse=w.reverse, dtype=dtype)


def assert_element_close(got: torch.Tensor, ref: np.ndarray, atol=ES_ATOL, rtol=ES_RTOL):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{int(bad.sum())} of {err.size} elements outside {atol}+{rtol}|ref|; worst at "
                             f"{idx}: got {g[idx]!r}, ref {ref[idx]!r}, max abs err {err.max():.3e}")


def assert_linear_close(got: torch.Tensor, ref: np.ndarray, tol: float, axis: int):
    """linear-scan is matrix-scan over 1 x 1 matrices: the matrix-scan bar on 1 x 1 states."""
    assert_matrix_close(got[..., None, None], ref[..., None, None], tol, axis=axis % max(ref.ndim, 1))


def matrix_state_errors(got: torch.Tensor, ref: np.ndarray):
    """Per-state relative Frobenius error ||g - r|| / ||r|| over the trailing [n, m] block."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    num = np.sqrt(np.sum((g - ref) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    return num, den


def assert_matrix_close(got: torch.Tensor, ref: np.ndarray, tol: float, axis: int = 1):
    """||g[t] - r[t]||_F <= tol * max(||r[t]||_F, RMS over the scan of ||r[t']||_F) for every state.

    The floor is the root-mean-square state norm of the same scan (same
    leading index, all t): a state whose terms cancel to near zero carries the
    absolute f32 error of those terms, so its own norm is no scale for it.
    """
    num, den = matrix_state_errors(got, ref)
    if den.size == 0:
        return
    scale = np.sqrt(np.mean(den ** 2, axis=axis, keepdims=True))
    ref_norm = np.maximum(den, scale)
    bad = num > tol * ref_norm
    if bad.any():
        idx = np.unravel_index(np.argmax(num / np.maximum(ref_norm, 1e-300)), num.shape)
        raise AssertionError(f"{int(bad.sum())} of {num.size} states outside relative {tol}; worst at {idx}: "
                             f"rel err {num[idx] / max(ref_norm[idx], 1e-300):.3e}")
