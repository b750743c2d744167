"""Parity of the HIP matrix-scan gradient with the CPU oracle's.

The GPU runs the forward scan, then ``matrix_scan_backward`` on its result
and a seeded upstream gradient g; the oracle computes the same gradients in
float64 from the same a, b and g (``oracle.matrix_scan_vjp``). The bar is
the matrix-scan bar on blocks: for grad_b (n x m states) and grad_a (n x n
blocks), ||gpu - ref||_F <= tol * max(||ref||_F, RMS of the block norms of
the same tensor), tol = 1e-4 for f32 and 2e-2 for bf16 (whose forward result
h, rounded to bf16, enters grad_a).

Shapes cover the pipelined kernel (n = 16 with m = 1, and bf16 with m = 16)
and the per-unit kernel (n < 16, m = 3, m = 17, f32 m = 16), several units
with a ragged last one, both directions, broadcast operands (gradients
summed over the broadcast dims), grad_a's runs of steps with ragged ends and
a scan over the first dim, grad_a formed inside the f32 m = 1 adjoint scan
(batch dims, a scan over the first dim, one step), a strided g, autograd through
``sx.matrix_scan``, and the two matrix workloads at full size on sampled
batch rows (a row is an exact sub-problem) plus a per-step residual check of
the adjoint recurrence over every row.
"""

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W
from tests.helpers import MS_TOL_BF16, MS_TOL_F32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _blocks_close(got, ref, tol, what):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    num = np.sqrt(np.sum((g - ref) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    if den.size == 0:
        return
    floor = np.sqrt(np.mean(den ** 2))
    scale = np.maximum(den, floor)
    bad = num > tol * scale
    if bad.any():
        idx = np.unravel_index(np.argmax(num / np.maximum(scale, 1e-300)), num.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {num.size} blocks outside relative {tol}; worst at {idx}: "
                             f"{num[idx] / max(scale[idx], 1e-300):.3e}")


def _draw(a_shape, b_shape, dtype, seed, a_scale=0.9, noise=0.05):
    g = torch.Generator().manual_seed(seed)
    n = a_shape[-1]
    a = (a_scale * torch.eye(n) + noise * torch.randn(a_shape, generator=g)).to(dtype)
    b = torch.randn(b_shape, generator=g).to(dtype)
    return a, b, g


def _check(a, b, axis, reverse, seed, grad_dtype=None, g_view=None):
    dt = a.dtype
    tol = MS_TOL_F32 if dt == torch.float32 and grad_dtype in (None, torch.float32) else MS_TOL_BF16
    print(f"\n[case] grad a {tuple(a.shape)} b {tuple(b.shape)} {dt} axis {axis} reverse {reverse}", flush=True)
    ad, bd = a.to(DEV), b.to(DEV)
    h = sx.matrix_scan(ad, bd, axis=axis, reverse=reverse)
    gen = torch.Generator().manual_seed(seed + 1000)
    gh = torch.randn(tuple(h.shape), generator=gen).to(dt)
    gd = gh.to(DEV) if g_view is None else g_view(gh.to(DEV))
    ga, gb = sx.matrix_scan_backward(ad, tuple(b.shape), h, gd, axis=axis, reverse=reverse, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    want_dt = dt if grad_dtype is None else grad_dtype
    assert ga.dtype == want_dt and gb.dtype == want_dt
    ra, rb = oracle.matrix_scan_vjp(a.float().numpy(), b.float().numpy(), gd.float().cpu().numpy(), axis=axis,
                                    reverse=reverse)
    _blocks_close(gb, rb, tol, "grad_b")
    _blocks_close(ga, ra, tol, "grad_a")


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("B,T", [(3, 700), (2, 96), (1, 97), (2, 1), (2, 2), (4, 17)])
def test_grad_pipelined_f32_m1(B, T, reverse):
    a, b, _ = _draw((B, T, 16, 16), (B, T, 16, 1), torch.float32, seed=31 + T)
    _check(a, b, 1, reverse, seed=31 + T)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("B,T,m", [(2, 400, 16), (1, 130, 32)])
def test_grad_pipelined_bf16_tiles(B, T, m, reverse):
    a, b, _ = _draw((B, T, 16, 16), (B, T, 16, m), torch.bfloat16, seed=41 + T)
    _check(a, b, 1, reverse, seed=41 + T)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("n,m,T,dtype", [(5, 3, 150, torch.float32), (16, 17, 140, torch.float32),
                                         (16, 16, 200, torch.float32), (3, 1, 300, torch.bfloat16),
                                         (1, 1, 260, torch.float32), (16, 1, 129, torch.bfloat16)])
def test_grad_unit_kernel_shapes(n, m, T, dtype, reverse):
    a, b, _ = _draw((2, T, n, n), (2, T, n, m), dtype, seed=51 + n + m)
    _check(a, b, 1, reverse, seed=51 + n + m)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("a_shape,axis,dt", [
    ((3, 37, 16, 16), 1, torch.float32),   # 111 steps: the last run of four ends past the last step
    ((1, 5, 16, 16), 1, torch.bfloat16),   # fewer steps than two runs
    ((37, 3, 16, 16), 0, torch.bfloat16),  # scan over the first dim: the step before is 3 steps apart
])
def test_grad_a_m16_runs(a_shape, axis, dt, reverse):
    # grad_a for m = 16 takes runs of consecutive steps per wave: ragged ends and a scan axis that is
    # not the innermost leading dim
    a, b, _ = _draw(a_shape, a_shape, dt, seed=91 + a_shape[0])
    _check(a, b, axis, reverse, seed=91 + a_shape[0])


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("a_shape,b_shape,axis", [
    ((2, 3, 130, 16, 16), (2, 3, 130, 16, 1), 2),  # two batch dims
    ((130, 3, 16, 16), (130, 3, 16, 1), 0),        # scan over the first dim: the time stride is 3 steps
    ((1, 1, 16, 16), (1, 1, 16, 1), 1),            # one step: its grad_a is zero
])
def test_grad_f32_m1_grad_a_in_the_scan(a_shape, b_shape, axis, reverse):
    # f32 gradients with n = 16, m = 1: the adjoint scan forms grad_a in its replay, at 16 times the
    # result's offsets; these layouts move the time and batch strides away from the plain [B, T] case
    a, b, _ = _draw(a_shape, b_shape, torch.float32, seed=95 + axis)
    _check(a, b, axis, reverse, seed=95 + axis)


def test_grad_bf16_operands_f32_gradients():
    a, b, _ = _draw((2, 300, 16, 16), (2, 300, 16, 1), torch.bfloat16, seed=61)
    _check(a, b, 1, False, seed=61, grad_dtype=torch.float32)


@pytest.mark.parametrize("n,m,dt", [(16, 1, torch.float32), (16, 16, torch.float32), (5, 3, torch.float32),
                                    (5, 3, torch.bfloat16), (16, 32, torch.bfloat16)])
def test_grad_bf16_gradients(n, m, dt):
    # bf16 gradients with b at the result's shape: the adjoint is rounded into grad_b and grad_a is
    # formed from it (one-, MFMA- and element-wise grad_a paths, f32 and bf16 h)
    a, b, _ = _draw((2, 300, n, n), (2, 300, n, m), dt, seed=62 + n + m)
    _check(a, b, 1, True, seed=62, grad_dtype=torch.bfloat16)


@pytest.mark.parametrize("a_shape,b_shape,axis", [
    ((300, 16, 16), (3, 300, 16, 1), 1),      # a shared by the batch
    ((3, 1, 16, 16), (3, 300, 16, 1), 1),     # a constant in time
    ((16, 16), (2, 250, 16, 1), 1),           # a one matrix for everything
    ((3, 200, 16, 16), (200, 16, 1), 1),      # b shared by the batch
    ((2, 100, 5, 5), (1, 100, 5, 3), -1),     # b shared, axis from the end
    ((2, 3, 70, 4, 4), (2, 3, 70, 4, 2), 2),  # two batch dims
    ((70, 2, 4, 4), (70, 2, 4, 2), 0),        # scan over the first leading dim
])
@pytest.mark.parametrize("reverse", [False, True])
def test_grad_broadcast_and_axes(a_shape, b_shape, axis, reverse):
    a, b, _ = _draw(a_shape, b_shape, torch.float32, seed=71 + len(a_shape))
    _check(a, b, axis, reverse, seed=71 + len(a_shape))


def test_grad_bf16_broadcast_a_bf16_gradients():
    a, b, _ = _draw((300, 16, 16), (2, 300, 16, 16), torch.bfloat16, seed=81)
    _check(a, b, 1, False, seed=81)


def test_grad_strided_g():
    a, b, _ = _draw((2, 200, 16, 16), (2, 200, 16, 1), torch.float32, seed=91)
    # g as a view: every other step of a longer tensor (leading stride 2 steps)
    _check(a, b, 1, False, seed=91,
           g_view=lambda g: torch.stack([g, torch.zeros_like(g)], dim=2).reshape(2, 400, 16, 1)[:, ::2])


def test_grad_expanded_g_from_sum():
    # loss = h.sum(): g is an expanded tensor of ones (stride 0 everywhere); the binding copies its matrix dims
    a, b, _ = _draw((2, 150, 16, 16), (2, 150, 16, 1), torch.float32, seed=92)
    ad, bd = a.to(DEV).requires_grad_(), b.to(DEV).requires_grad_()
    sx.matrix_scan(ad, bd, axis=1).sum().backward()
    ra, rb = oracle.matrix_scan_vjp(a.numpy(), b.numpy(), np.ones((2, 150, 16, 1)), axis=1)
    _blocks_close(bd.grad, rb, MS_TOL_F32, "grad_b")
    _blocks_close(ad.grad, ra, MS_TOL_F32, "grad_a")


@pytest.mark.parametrize("reverse", [False, True])
def test_autograd_through_matrix_scan(reverse):
    a, b, _ = _draw((2, 130, 6, 6), (2, 130, 6, 2), torch.float32, seed=93)
    w = torch.randn((2, 130, 6, 2), generator=torch.Generator().manual_seed(94))
    ad, bd = a.to(DEV).requires_grad_(), b.to(DEV).requires_grad_()
    h = sx.matrix_scan(ad, bd, axis=1, reverse=reverse)
    (h * w.to(DEV)).sum().backward()
    ra, rb = oracle.matrix_scan_vjp(a.numpy(), b.numpy(), w.numpy(), axis=1, reverse=reverse)
    _blocks_close(bd.grad, rb, MS_TOL_F32, "grad_b")
    _blocks_close(ad.grad, ra, MS_TOL_F32, "grad_a")


# autograd with a result dtype other than the operands': bf16 operands with an f32
# result (the bf16 bar: the operands are bf16 and grad_a, grad_b round to bf16), and
# f32 operands with a bf16 result (the bf16 bar: the rounded result enters grad_a).
# The gradients take the operands' dtype.
@pytest.mark.parametrize("dtype,out_dtype", [(torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("m", [1, 16])
def test_autograd_with_another_result_dtype(dtype, out_dtype, m):
    a, b, _ = _draw((2, 300, 16, 16), (2, 300, 16, m), dtype, seed=95 + m)
    w = torch.randn((2, 300, 16, m), generator=torch.Generator().manual_seed(96))
    ad, bd = a.to(DEV).requires_grad_(), b.to(DEV).requires_grad_()
    h = sx.matrix_scan(ad, bd, axis=1, reverse=True, out_dtype=out_dtype)
    assert h.dtype == out_dtype
    (h.float() * w.to(DEV)).sum().backward()
    assert ad.grad.dtype == dtype and bd.grad.dtype == dtype
    ra, rb = oracle.matrix_scan_vjp(a.float().numpy(), b.float().numpy(), w.numpy(), axis=1, reverse=True)
    _blocks_close(bd.grad, rb, MS_TOL_BF16, "grad_b")
    _blocks_close(ad.grad, ra, MS_TOL_BF16, "grad_a")


def test_grad_empty_and_errors():
    a = torch.zeros((2, 0, 4, 4), device=DEV)
    b = torch.zeros((2, 0, 4, 3), device=DEV)
    ga, gb = sx.matrix_scan_backward(a, b.shape, b, b)
    assert ga.shape == a.shape and gb.shape == b.shape
    # a constant in time over an empty axis: its gradient is zero
    a1 = torch.ones((2, 1, 4, 4), device=DEV)
    ga, gb = sx.matrix_scan_backward(a1, (2, 0, 4, 3), b, b)
    assert ga.shape == a1.shape and torch.count_nonzero(ga) == 0
    x = torch.zeros((2, 5, 4, 4), device=DEV)
    h = torch.zeros((2, 5, 4, 1), device=DEV)
    with pytest.raises(sx.SxError) as e:
        sx.matrix_scan_backward(x, (2, 5, 4, 1), h, h.to(torch.bfloat16))
    assert e.value.name == "E-DIM-002"
    with pytest.raises(sx.SxError) as e:
        sx.matrix_scan_backward(x, (2, 5, 4, 1), h, torch.zeros((2, 5, 4, 2), device=DEV))
    assert e.value.name == "E-DIM-001"


@pytest.mark.parametrize("idx", [3, 4])
def test_grad_standard_workload_sampled_rows_and_adjoint_residual(idx):
    """The matrix workloads at full size: the gradient on three sampled batch
    rows against the oracle, and the adjoint recurrence lam[t] = g[t] +
    a[s]^T lam[s] checked step by step over every row (this is what a wrong
    entering state anywhere in the look-back would break)."""
    w = W.standard_workloads([idx])[0]
    print(f"\n[case] gradient of {w.name}", flush=True)
    t = w.on(DEV)
    a, b = t["a"], t["b"]
    h = sx.matrix_scan(a, b, axis=w.axis, reverse=w.reverse)
    gen = torch.Generator().manual_seed(95)
    g = torch.randn(tuple(h.shape), generator=gen).to(h.dtype).to(DEV)
    grad_dtype = torch.float32  # keep the adjoint itself for the residual check
    ga, gb = sx.matrix_scan_backward(a, tuple(b.shape), h, g, axis=w.axis, reverse=w.reverse, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    rows = [0, 7, a.shape[0] - 1]
    tol = MS_TOL_F32 if a.dtype == torch.float32 else MS_TOL_BF16
    for r in rows:
        ra, rb = oracle.matrix_scan_vjp(w.tensors["a"][r].float().numpy(), w.tensors["b"][r].float().numpy(),
                                        g[r].float().cpu().numpy(), axis=0, reverse=w.reverse)
        _blocks_close(gb[r], rb, tol, f"grad_b row {r}")
        _blocks_close(ga[r], ra, tol, f"grad_a row {r}")
    # residual of the adjoint over every row (float64 on the device)
    lam = gb.double()
    a64 = a.double()
    g64 = g.double()
    if not w.reverse:   # the step after t is t + 1
        pred = g64[:, :-1] + torch.matmul(a64[:, 1:].transpose(-1, -2).contiguous(), lam[:, 1:])
        res, ref = lam[:, :-1] - pred, lam[:, :-1]
        last_ok = torch.equal(lam[:, -1], g64[:, -1])
    else:               # the step after t is t - 1
        pred = g64[:, 1:] + torch.matmul(a64[:, :-1].transpose(-1, -2).contiguous(), lam[:, :-1])
        res, ref = lam[:, 1:] - pred, lam[:, 1:]
        last_ok = torch.equal(lam[:, 0], g64[:, 0])
    assert last_ok, "the adjoint at the last step is g there"
    num = res.pow(2).sum(dim=(-2, -1)).sqrt()
    den = ref.pow(2).sum(dim=(-2, -1)).sqrt()
    floor = den.pow(2).mean(dim=1, keepdim=True).sqrt()
    rel = (num / torch.maximum(den, floor)).max().item()
    assert rel <= 1e-4, f"adjoint residual {rel:.3e}"
