"""Parity of the HIP linear-scan (and cumsum) with the CPU oracle.

linear-scan is matrix-scan over one-by-one matrices, so its bar is the
matrix-scan bar on 1 x 1 states: |gpu[t] - ref[t]| <= tol * max(|ref[t]|,
RMS of |ref| over the same lane's scan), tol = 1e-4 when the result is
stored in f32 (f32 or bf16 operands: both are computed in f32 from exactly
widened inputs) and 2e-2 when it is stored in bf16.

Cases cover the lane kernel (few lanes, short axes) and the slab kernel
(8192 lanes or more, 512 trips or more), ragged lane counts and slab tails,
broadcast operands (a number, a stride-0 axis), strided views, both
directions, bf16 in and out, and empty results. The measured shape,
[64,4096,256] along axis 1, is compared on sampled lanes at full size.
"""

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W
from tests.helpers import MS_TOL_BF16, MS_TOL_F32, assert_linear_close, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(w):
    print(f"\n[case] {w.name}", flush=True)
    got = run_gpu(w, DEV)
    torch.cuda.synchronize()
    ref = run_oracle(w)
    out_dtype = w.out_dtype or w.tensors["b"].dtype
    tol = MS_TOL_F32 if out_dtype == torch.float32 else MS_TOL_BF16
    assert got.dtype == out_dtype
    assert_linear_close(got, ref, tol, axis=w.axis)


@pytest.mark.parametrize("shape,axis,reverse", [
    ((3, 37, 19), 1, False),
    ((3, 37, 19), 1, True),
    ((41, 5, 3), 0, False),
    ((2, 3, 130), -1, True),
    ((1, 1, 1), 1, False),
    ((5, 1, 7), 1, True),
    ((200,), 0, False),
    ((200,), 0, True),
])
@pytest.mark.parametrize("a_kind", ["decay", "signed"])
def test_linear_small(shape, axis, reverse, a_kind):
    _check(W.make_linear(shape, axis=axis, reverse=reverse, a_kind=a_kind, seed=11))


@pytest.mark.parametrize("shape,axis,reverse", [
    ((2, 777, 4163), 1, False),   # 8326 lanes (ragged last workgroup), 777 trips (ragged last slab)
    ((2, 777, 4163), 1, True),
    ((8200, 600), 1, False),      # axis last: every lane strided by one element along time
    ((600, 8200), 0, True),
])
def test_linear_slab_path(shape, axis, reverse):
    _check(W.make_linear(shape, axis=axis, reverse=reverse, a_kind="signed", seed=12))


@pytest.mark.parametrize("shape,axis,reverse", [
    ((3, 300, 17), 1, False),
    ((2, 777, 4163), 1, True),
])
def test_cumsum(shape, axis, reverse):
    w = W.make_linear(shape, axis=axis, reverse=reverse, a_kind="ones", seed=13)
    _check(w)
    # cumsum is the plain running sum
    b = w.tensors["b"].to(DEV)
    got = sx.cumsum(b, axis=axis, reverse=reverse)
    ref = np.flip(np.cumsum(np.flip(b.double().cpu().numpy(), axis), axis), axis) if reverse \
        else np.cumsum(b.double().cpu().numpy(), axis)
    assert_linear_close(got, ref, MS_TOL_F32, axis=axis)


@pytest.mark.parametrize("shape,a_shape,axis", [
    ((2, 777, 4163), (777, 1), 1),   # a broadcast over batch and lanes (stride 0)
    ((3, 40, 19), (3, 40, 1), 1),    # a shared by the lanes of one batch entry
    ((3, 40, 19), (19,), 1),         # a constant along the axis
    ((2, 777, 4163), (4163,), 1),    # the same in the slab kernel: read once per lane
    ((4, 50), (1, 50), -1),
])
def test_linear_broadcast_a(shape, a_shape, axis):
    _check(W.make_linear(shape, axis=axis, a_shape=a_shape, a_kind="decay", seed=14))


@pytest.mark.parametrize("shape", [(3, 37, 19), (2, 777, 4163)])
def test_linear_number_a(shape):
    _check(W.make_linear(shape, axis=1, a_kind="number", seed=15))


def test_linear_number_b_and_tensor_a():
    g = torch.Generator().manual_seed(16)
    a = (0.9 + 0.1 * torch.rand((5, 300, 7), generator=g))
    got = sx.linear_scan(a.to(DEV), 0.5, axis=1)
    ref = oracle.linear_scan(a.numpy(), np.float32(0.5), axis=1)
    assert got.shape == (5, 300, 7)
    assert_linear_close(got, ref, MS_TOL_F32, axis=1)


@pytest.mark.parametrize("shape,reverse", [((3, 37, 19), False), ((2, 777, 4163), True)])
@pytest.mark.parametrize("out_dtype", [None, torch.float32])
@pytest.mark.parametrize("a_kind", ["decay", "ones"])  # ones: cumsum, a constant in time
def test_linear_bf16(shape, reverse, out_dtype, a_kind):
    _check(W.make_linear(shape, axis=1, reverse=reverse, dtype=torch.bfloat16, a_kind=a_kind, seed=17,
                         out_dtype=out_dtype))


def test_linear_bf16_store_is_the_rounded_f32_result():
    w = W.make_linear((2, 777, 4163), axis=1, dtype=torch.bfloat16, a_kind="decay", seed=18)
    t = w.on(DEV)
    f32 = sx.linear_scan(t["a"], t["b"], axis=1, out_dtype=torch.float32)
    b16 = sx.linear_scan(t["a"], t["b"], axis=1)
    assert torch.equal(b16, f32.to(torch.bfloat16))  # torch rounds f32 to bf16 to nearest even


def test_linear_strided_views():
    g = torch.Generator().manual_seed(19)
    big_b = torch.randn((4, 130, 2, 33), generator=g)
    big_a = 0.9 + 0.1 * torch.rand((33, 4, 130), generator=g)
    b = big_b.to(DEV)[:, :, 1, :]              # [4, 130, 33], strides (8580, 66, 1)
    a = big_a.to(DEV).permute(1, 2, 0)         # [4, 130, 33], strides (130, 1, 520)
    got = sx.linear_scan(a, b, axis=1, reverse=True)
    ref = oracle.linear_scan(a.cpu().numpy(), b.cpu().numpy(), axis=1, reverse=True)
    assert_linear_close(got, ref, MS_TOL_F32, axis=1)


def test_linear_empty_and_errors():
    z = torch.zeros((3, 0, 5), device=DEV)
    assert sx.linear_scan(z, z, axis=1).shape == (3, 0, 5)
    assert sx.cumsum(torch.zeros((0, 4), device=DEV), axis=1).shape == (0, 4)
    x = torch.zeros((3, 4), device=DEV)
    with pytest.raises(sx.SxError) as e:
        sx.linear_scan(x, torch.zeros((2, 4), device=DEV))
    assert e.value.name == "E-DIM-001"
    with pytest.raises(sx.SxError) as e:
        sx.linear_scan(x, x, axis=2)
    assert e.value.name == "E-DIM-001"
    with pytest.raises(sx.SxError) as e:
        sx.linear_scan(x, x.to(torch.bfloat16))
    assert e.value.name == "E-DIM-002"
    with pytest.raises(sx.SxError) as e:
        sx.linear_scan(x[:, :2], x, axis=0)
    assert e.value.name == "E-DIM-001"


@pytest.mark.parametrize("a_kind", ["decay", "ones"])
def test_linear_measured_shape_sampled_lanes(a_kind):
    """The measured workload at full size, [64,4096,256] along axis 1, in the
    launch the bench times; the oracle runs on 512 sampled lanes (lanes are
    independent, so a slice of the inputs is an exact sub-problem)."""
    w = W.make_linear(a_kind=a_kind)
    print(f"\n[case] {w.name} (sampled lanes)", flush=True)
    got = run_gpu(w, DEV)
    torch.cuda.synchronize()
    rng = np.random.default_rng(20)
    bi = rng.integers(0, 64, 512)
    ci = rng.integers(0, 256, 512)
    b = w.tensors["b"][bi, :, ci].double().numpy()          # [512, 4096]
    if "a" in w.tensors:
        a = w.tensors["a"][bi, :, ci].double().numpy()
    else:
        a = np.float64(w.meta["a_number"])
    ref = oracle.linear_scan(a, b, axis=1)
    g = got[torch.as_tensor(bi), :, torch.as_tensor(ci)]
    assert_linear_close(g, ref, MS_TOL_F32, axis=1)
