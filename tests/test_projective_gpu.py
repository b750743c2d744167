"""Parity of the HIP matrix-scan ``:projective`` path with the CPU oracle.

The oracle (``oracle.matrix_scan_projective``) multiplies a running matrix,
started at the identity, by each step's a and rescales it and h after every
step by that matrix's entry of largest absolute value. The GPU runs the same recurrence in f32.
The bar is the matrix-scan bar: ||gpu[t] - ref[t]||_F <= tol * max(||ref[t]||_F,
RMS of the state norms of the same scan), tol = 1e-4 for f32 operands and
2e-2 for bf16.

Cases: the pipelined shapes (n = 16, m = 1 and bf16 m = 16; one long enough
that the chunk products compose over several rounds of loads), other n and m,
broadcast a, both directions, products that grow (a plain scan in f32 would
overflow; the projective one stays in range), the full-size f32 matrix
workload on sampled rows, and the refusal of a gradient.
"""

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx
from tests.helpers import MS_TOL_BF16, MS_TOL_F32, assert_matrix_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _draw(a_shape, b_shape, dtype, seed, scale=0.9, noise=0.05):
    g = torch.Generator().manual_seed(seed)
    n = a_shape[-1]
    a = (scale * torch.eye(n) + noise * torch.randn(a_shape, generator=g)).to(dtype)
    b = torch.randn(b_shape, generator=g).to(dtype)
    return a, b


def _check(a, b, axis, reverse):
    print(f"\n[case] projective a {tuple(a.shape)} b {tuple(b.shape)} {a.dtype} axis {axis} reverse {reverse}",
          flush=True)
    got = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=axis, reverse=reverse, projective=True)
    torch.cuda.synchronize()
    ref = oracle.matrix_scan_projective(a.float().numpy(), b.float().numpy(), axis=axis, reverse=reverse)
    assert np.all(np.isfinite(got.float().cpu().numpy()))
    tol = MS_TOL_F32 if a.dtype == torch.float32 else MS_TOL_BF16
    lead = len(ref.shape) - 2
    assert_matrix_close(got, ref, tol, axis=axis % lead)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("B,T,n,m,dtype", [(3, 500, 16, 1, torch.float32), (2, 300, 16, 16, torch.bfloat16),
                                           (2, 200, 5, 3, torch.float32), (2, 130, 16, 17, torch.float32),
                                           (1, 1, 16, 1, torch.float32), (2, 64, 1, 1, torch.float32),
                                           (2, 257, 16, 16, torch.float32),
                                           # 18 chunks of 128 steps, the last ragged: the chunk products
                                           # compose over more than one round of loads
                                           (2, 128 * 17 + 5, 16, 1, torch.float32)])
def test_projective_shapes(B, T, n, m, dtype, reverse):
    a, b = _draw((B, T, n, n), (B, T, n, m), dtype, seed=201 + n + m + T)
    _check(a, b, 1, reverse)


@pytest.mark.parametrize("a_shape,b_shape,axis", [((300, 16, 16), (3, 300, 16, 1), 1),
                                                  ((16, 16), (2, 250, 16, 2), 1),
                                                  ((70, 2, 4, 4), (70, 2, 4, 2), 0)])
def test_projective_broadcast_and_axes(a_shape, b_shape, axis):
    a, b = _draw(a_shape, b_shape, torch.float32, seed=211)
    _check(a, b, axis, False)


@pytest.mark.parametrize("reverse", [False, True])
def test_projective_growing_products_stay_in_range(reverse):
    # spectral radius about 1.5: over 1000 steps the plain product reaches 1.5^1000, far past f32's range;
    # the projective scan normalises it every step
    a, b = _draw((2, 1000, 16, 16), (2, 1000, 16, 1), torch.float32, seed=221, scale=1.5, noise=0.05)
    plain = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=1, reverse=reverse)
    assert not torch.all(torch.isfinite(plain)), "the plain scan was expected to overflow here"
    _check(a, b, 1, reverse)


def test_projective_matrix_workload_sampled_rows():
    from scan_primitives_amd import workloads as W
    w = W.make_matrix(32, 8192, 16, 1, torch.float32, seed=4)
    print(f"\n[case] projective {w.name}", flush=True)
    got = sx.matrix_scan(w.tensors["a"].to(DEV), w.tensors["b"].to(DEV), axis=1, projective=True)
    torch.cuda.synchronize()
    for r in (0, 13, 31):
        ref = oracle.matrix_scan_projective(w.tensors["a"][r].numpy(), w.tensors["b"][r].numpy(), axis=0)
        assert_matrix_close(got[r], ref, MS_TOL_F32, axis=0)


def test_projective_has_no_gradient():
    a, b = _draw((2, 50, 4, 4), (2, 50, 4, 1), torch.float32, seed=231)
    ad, bd = a.to(DEV).requires_grad_(), b.to(DEV).requires_grad_()
    h = sx.matrix_scan(ad, bd, axis=1, projective=True)
    with pytest.raises(sx.SxError) as e:
        h.sum().backward()
    assert e.value.name == "E-UNSUPPORTED"
