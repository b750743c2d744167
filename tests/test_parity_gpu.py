"""Parity of the HIP library with the CPU oracle, element by element.

Every case draws seeded inputs from ``scan_primitives_amd.workloads``, runs
the C ABI (through the Python binding) on the GPU and the float64 oracle on
the CPU, and compares:

* element-scan (f32): |gpu - ref| <= 1e-5 + 1e-5 |ref| for every element;
* matrix-scan: ||gpu[t] - ref[t]||_F <= tol * max(||ref[t]||_F, the RMS state
  norm of the same scan) for every state, tol = 1e-4 for f32 operands and
  2e-2 for bf16 operands.

Sizes span several tiles with a ragged tail; the five standard workloads run
at full size.
"""

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W
from tests.helpers import (MS_TOL_BF16, MS_TOL_F32, assert_element_close, assert_matrix_close, run_gpu,
                           run_oracle)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _announce(w):
    print(f"\n[case] {w.name}", flush=True)


# ------------------------------------------------------------------ element-scan


@pytest.mark.parametrize("shape,axis,reverse", [
    ((3, 37, 19), 1, False),
    ((3, 37, 19), 1, True),
    ((41, 5, 3), 0, False),
    ((2, 3, 130), -1, True),
    ((1, 1, 1), 1, False),
    ((5, 1, 7), 1, True),
    ((64,), 0, False),
])
def test_tanh_small(shape, axis, reverse):
    w = W.make_tanh(shape, axis=axis, reverse=reverse, seed=100 + len(shape))
    _announce(w)
    assert_element_close(run_gpu(w, DEV), run_oracle(w))


@pytest.mark.parametrize("shape,axis,reverse", [
    ((3, 200, 19), 1, True),
    ((3, 200, 19), 1, False),
    ((257, 3, 5), 0, True),
    ((2, 9, 1000), -1, False),
    ((3, 40, 19), 1, True),     # axes of at most 64 trips: every position loaded before the first trip
    ((64, 7), 0, False),
    ((2, 5, 63), -1, True),
])
def test_max_plus_small(shape, axis, reverse):
    w = W.make_max_plus(shape, axis=axis, reverse=reverse, seed=110)
    _announce(w)
    got = run_gpu(w, DEV)
    assert_element_close(got, run_oracle(w))


@pytest.mark.parametrize("shape,axis,reverse", [
    ((33, 600, 250), 1, False),    # 8250 lanes: the last 64-lane group is partial
    ((520, 40, 17), 1, True),      # too short an axis for slabs: the lane kernel
    ((9000, 513), 0, True),        # long axis, few lanes: the lane kernel
    ((600, 8200), 0, False),       # axis 0 with 8200 contiguous lanes: the slab kernel
])
def test_max_plus_slab_path(shape, axis, reverse):
    w = W.make_max_plus(shape, axis=axis, reverse=reverse, seed=111)
    _announce(w)
    got = run_gpu(w, DEV)
    assert_element_close(got, run_oracle(w))


@pytest.mark.parametrize("shape,axis,reverse", [
    ((33, 700, 256), 1, True),     # 8448 lanes, 700 trips: the slab kernel, 2 full slabs and a ragged one
    ((3, 1000, 512), 1, False),    # below 8192 lanes the lane kernel runs: two rows of lanes per batch
    ((1, 200, 256), 1, False),     # one row of lanes
    ((2, 128, 768), 1, True),      # a short axis
    ((4, 5000, 256), 1, True),     # a long axis
    ((300, 1024), 0, False),       # axis 0: the lanes are the contiguous last dim
])
def test_max_plus_rows_path(shape, axis, reverse):
    """Lanes along a contiguous last dim, with ragged axis lengths."""
    w = W.make_max_plus(shape, axis=axis, reverse=reverse, seed=112)
    _announce(w)
    got = run_gpu(w, DEV)
    assert_element_close(got, run_oracle(w))


def test_max_plus_rows_strided_views():
    """Padded rows, a strided initial, and a view shifted by one element."""
    g = torch.Generator().manual_seed(113)
    xb = torch.randn(5, 300, 320, generator=g)
    cb = 0.1 * torch.rand(5, 300, 320, generator=g)
    ib = torch.randn(256, 5, generator=g)
    x, c, init = xb[:, :, :256], cb[:, :, :256], ib.t()  # init [5, 256] with strides (1, 5)
    ref = oracle.element_scan("max_plus", init.numpy(), [x.numpy(), c.numpy()], axis=1, reverse=True)
    got = sx.element_scan("max_plus", init.to(DEV), [xb.to(DEV)[:, :, :256], cb.to(DEV)[:, :, :256]], axis=1,
                          reverse=True)
    assert_element_close(got, ref)
    x1, c1 = xb[:, :, 1:257], cb[:, :, 1:257]
    ref = oracle.element_scan("max_plus", init.numpy(), [x1.numpy(), c1.numpy()], axis=1, reverse=False)
    got = sx.element_scan("max_plus", init.to(DEV), [xb.to(DEV)[:, :, 1:257], cb.to(DEV)[:, :, 1:257]], axis=1)
    assert_element_close(got, ref)


@pytest.mark.parametrize("B,T,H,n,gate,reverse", [
    (2, 45, 5, 16, 1, False),
    (2, 45, 5, 16, 16, True),
    (3, 33, 2, 5, 1, True),
    (1, 70, 3, 1, 1, False),
    (2, 17, 9, 16, 1, False),
])
def test_norm_cap_small(B, T, H, n, gate, reverse):
    w = W.make_norm_cap(B, T, H, n, gate_width=gate, reverse=reverse, seed=120, zero_initial=False)
    _announce(w)
    got = run_gpu(w, DEV)
    ref = run_oracle(w)
    assert_element_close(got, ref)
    assert float(torch.linalg.vector_norm(got, dim=-1).max()) <= 1 + 1e-5


@pytest.mark.parametrize("B,T,H,n,gate,reverse", [
    (2, 300, 5, 16, 1, False),     # chunked along the axis (few lanes): ragged last chunk
    (3, 257, 2, 5, 5, True),       # per-component gate (bound uses the largest |a|), reverse
    (1, 1000, 3, 16, 16, False),
])
def test_norm_cap_chunked(B, T, H, n, gate, reverse):
    w = W.make_norm_cap(B, T, H, n, gate_width=gate, reverse=reverse, seed=125, zero_initial=False)
    _announce(w)
    assert_element_close(run_gpu(w, DEV), run_oracle(w))


@pytest.mark.parametrize("reverse", [False, True])
def test_norm_cap_chunked_without_contraction(reverse):
    # decay = 1 and tiny x: no trip contracts, no warm-up can be certified, and
    # every chunk has to run from the start of the axis; the result stays exact.
    g = torch.Generator().manual_seed(126)
    x = 1e-2 * torch.randn(2, 200, 3, 16, generator=g)
    decay = torch.ones(2, 200, 3, 1)
    init = 0.1 * torch.randn(2, 3, 16, generator=g)
    ref = oracle.element_scan("norm_cap", init.numpy(), [x.numpy(), decay.numpy()], axis=1, state_axis=-1,
                              reverse=reverse)
    got = sx.element_scan("norm_cap", init.to(DEV), [x.to(DEV), decay.to(DEV)], axis=1, state_axis=-1,
                          reverse=reverse)
    assert_element_close(got, ref)


@pytest.mark.parametrize("x_scale,reverse", [(0.8, False), (0.85, True)])
def test_norm_cap_partly_certified_warm_ups(x_scale, reverse):
    # x scaled so that about 40% (0.8) or 87% (0.85) of the 8-trip chunks certify their warm-up within
    # the 20 trips the register path keeps: certified and uncertified quads share waves, and the
    # uncertified ones walk further back. initial lies far outside the unit ball (|initial| about 100),
    # so chunks within reach of the axis start must run exactly from it.
    w = W.make_norm_cap(8, 512, 16, 16, gate_width=1, reverse=reverse, seed=127, zero_initial=False,
                        x_scale=x_scale)
    w.tensors["initial"] = 25.0 * w.tensors["initial"]
    _announce(w)
    got = run_gpu(w, DEV)
    assert_element_close(got, run_oracle(w))
    assert float(torch.linalg.vector_norm(got, dim=-1).max()) <= 1 + 1e-5


@pytest.mark.parametrize("case", ["x_width_one", "both_width_one", "aligned_view", "unaligned_view",
                                  "strided_initial", "axis0", "many_vectors", "reverse_long"])
def test_norm_cap_layouts(case):
    """The 16-wide norm-cap layouts: four components per thread from 16-byte aligned memory (width-one x
    or gate, views whose offsets are multiples of four, any initial), one component per thread otherwise
    (unaligned views), split along the axis or not (many state vectors)."""
    g = torch.Generator().manual_seed(140)
    B, T, H, axis, rev = 2, 300, 5, 1, False
    xw, sw = 16, 1
    if case == "x_width_one":
        xw, sw = 1, 16
    elif case == "both_width_one":
        xw, sw = 1, 1
    elif case == "many_vectors":
        B, T, H = 2, 40, 8200
    elif case == "reverse_long":
        B, T, H, rev = 1, 2000, 3, True
    shape = (B, T, H)
    pad = 4 if case == "aligned_view" else (1 if case == "unaligned_view" else 0)
    xb = 2.0 * torch.randn(shape + (xw + pad,), generator=g)
    x = xb[..., pad:] if case == "unaligned_view" else xb[..., :xw]
    s = 0.8 + 0.2 * torch.rand(shape + (sw,), generator=g)
    init = 0.3 * torch.randn((B, H, 16), generator=g)
    if case == "strided_initial":
        init = 0.3 * torch.randn((16, H, B), generator=g).permute(2, 1, 0)  # non-contiguous, component stride H*B
    if case == "axis0":
        x, s = x.transpose(0, 1), s.transpose(0, 1)  # [T, B, H, .] scanned along axis 0 (strided lanes)
        axis = 0
    ref = oracle.element_scan("norm_cap", init.numpy(), [x.numpy(), s.numpy()], axis=axis, state_axis=-1,
                              reverse=rev)
    print(f"\n[case] norm-cap layout {case} x {tuple(x.shape)} s {tuple(s.shape)}", flush=True)
    xd = xb.to(DEV)
    xd = xd[..., pad:] if case == "unaligned_view" else xd[..., :xw]
    sd = s.to(DEV) if case != "axis0" else s.transpose(0, 1).contiguous().to(DEV).transpose(0, 1)
    if case == "axis0":
        xd = xd.transpose(0, 1)
    idev = init.to(DEV) if case != "strided_initial" else init.permute(2, 1, 0).contiguous().to(DEV).permute(2, 1, 0)
    got = sx.element_scan("norm_cap", idev, [xd, sd], axis=axis, state_axis=-1, reverse=rev)
    torch.cuda.synchronize()
    assert_element_close(got, ref)


def test_element_scan_strided_and_broadcast_operands():
    # x as a transposed view, decay broadcast along the width (stride 0), initial non-contiguous
    g = torch.Generator().manual_seed(130)
    xt = torch.randn(19, 3, 50, generator=g)            # [width, batch, time]
    x = xt.permute(1, 2, 0)                              # [3, 50, 19], strides (50, 1, 150)
    decay = torch.rand(3, 50, 1, generator=g).expand(3, 50, 19)
    init = torch.randn(19, 3, generator=g).t()           # [3, 19] transposed
    ref = oracle.element_scan("tanh_affine", init.numpy(), [x.numpy(), decay.numpy()], axis=1)
    got = sx.element_scan("tanh_affine", init.to(DEV), [x.to(DEV), decay.to(DEV)], axis=1)
    assert_element_close(got, ref)


def _view_past_32_bits(shape, lead_stride, fill):
    """A view of `shape` into a device buffer of more than 2^31 floats: its first
    dim steps `lead_stride` (>= 2^31) elements, so lane offsets pass 32 bits.
    Only the viewed elements are written."""
    inner = int(np.prod(shape[1:]))
    base = torch.empty(lead_stride * (shape[0] - 1) + inner + 64, device=DEV)
    strides = (lead_stride,) + tuple(torch.empty(shape[1:]).stride())
    v = base.as_strided(shape, strides)
    v.copy_(fill.to(DEV))
    return base, v


def test_lane_offsets_past_32_bits():
    """x whose lane offsets pass 2^31 elements: the lane kernel takes its
    64-bit index path (checked on the host), and the results match."""
    g = torch.Generator().manual_seed(134)
    x = torch.randn(2, 64, 32, generator=g)
    decay = torch.rand(2, 64, 32, generator=g)
    init = torch.randn(2, 32, generator=g)
    base, xv = _view_past_32_bits((2, 64, 32), 2 ** 31, x)
    ref = oracle.element_scan("tanh_affine", init.numpy(), [x.numpy(), decay.numpy()], axis=1)
    got = sx.element_scan("tanh_affine", init.to(DEV), [xv, decay.to(DEV)], axis=1)
    assert_element_close(got, ref)
    del base, xv
    torch.cuda.empty_cache()


def test_norm_cap_initial_offsets_past_32_bits():
    """A norm-cap initial whose offsets pass 2^31 elements: the four-components
    -per-thread kernels index in 32 bits, so they must not take it (regression:
    their check covered x, the gate and out but not initial)."""
    w = W.make_norm_cap(B=2, T=40, H=3, n=16, zero_initial=False, seed=135)
    t = w.tensors
    base, iv = _view_past_32_bits((2, 3, 16), 2 ** 31, t["initial"])
    ref = run_oracle(w)
    got = sx.element_scan("norm_cap", iv, [t["x"].to(DEV), t["s"].to(DEV)], axis=1, state_axis=-1)
    assert_element_close(got, ref)
    del base, iv
    torch.cuda.empty_cache()


def test_vector_state_elementwise_bodies():
    g = torch.Generator().manual_seed(131)
    x = torch.randn(4, 60, 3, 7, generator=g)
    c = 0.1 * torch.rand(4, 60, 3, 1, generator=g)
    init = torch.randn(4, 3, 7, generator=g)
    for body in ("max_plus", "tanh_affine"):
        ref = oracle.element_scan(body, init.numpy(), [x.numpy(), c.numpy()], axis=1, state_axis=-1, reverse=True)
        got = sx.element_scan(body, init.to(DEV), [x.to(DEV), c.to(DEV)], axis=1, state_axis=-1, reverse=True)
        assert_element_close(got, ref)


def test_max_plus_matches_float32_serial_evaluation():
    # Subtract and maximum are correctly rounded, so a float32 evaluation in any
    # order that keeps each lane's trips serial agrees with the float32 oracle to
    # within the reassociation of the cost sums; report how close it is.
    w = W.make_max_plus((4, 300, 64), seed=132)
    got = run_gpu(w, DEV).cpu().numpy()
    ref32 = run_oracle(w, dtype=np.float32)
    err = np.abs(got.astype(np.float64) - ref32.astype(np.float64))
    print(f"max-plus vs float32 oracle: {int((err == 0).sum())} of {err.size} bit-identical, max err {err.max():.3e}")
    assert err.max() <= 1e-5 * (1 + np.abs(ref32).max())


def test_max_plus_short_axis_is_a_serial_float32_evaluation():
    # On an axis of at most 64 trips one thread runs each lane's trips in order, so the result is
    # the float32 oracle's (subtract and maximum are correctly rounded) bit for bit.
    for shape, reverse in (((4, 64, 64), True), ((5, 33, 17), False)):
        w = W.make_max_plus(shape, reverse=reverse, seed=133)
        got = run_gpu(w, DEV).cpu().numpy()
        assert np.array_equal(got, run_oracle(w, dtype=np.float32))


def test_element_scan_errors_on_device_tensors():
    x = torch.zeros(2, 0, 3, device=DEV)
    with pytest.raises(sx.SxError) as e:
        sx.element_scan("max_plus", torch.zeros(2, 3, device=DEV), [x, x], axis=1)
    assert e.value.name == "E-DIM-001"
    x = torch.zeros(2, 4, 3, device=DEV)
    with pytest.raises(sx.SxError) as e:
        sx.element_scan("max_plus", torch.zeros(2, 3, device=DEV), [x, x.double()], axis=1)
    assert e.value.name == "E-DIM-002"


# ------------------------------------------------------------------ matrix-scan


@pytest.mark.parametrize("B,T,n,m,reverse", [
    (3, 65, 16, 1, False),
    (3, 65, 16, 1, True),
    (2, 64, 16, 16, False),
    (2, 63, 16, 17, True),
    (4, 129, 3, 3, False),
    (2, 300, 1, 1, True),
    (1, 1, 16, 16, False),
    (5, 2, 7, 16, True),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_matrix_small(B, T, n, m, reverse, dtype):
    w = W.make_matrix(B, T, n, m, dtype, reverse=reverse, seed=140 + n + m)
    _announce(w)
    got = run_gpu(w, DEV)
    assert got.dtype == dtype
    assert_matrix_close(got, run_oracle(w), MS_TOL_F32 if dtype == torch.float32 else MS_TOL_BF16)


# Shapes that take the pipelined kernel (n = 16; m = 1, or m a multiple of 16 with
# bf16 inputs): several 16-column tiles, a last unit whose later waves lie wholly
# past the end (700 = 5 * 128 + 60), both output types, and enough units that each
# resident workgroup computes several of them in turn.
@pytest.mark.parametrize("B,T,m,dtype,out,reverse", [
    (3, 700, 32, torch.bfloat16, None, False),
    (3, 700, 32, torch.bfloat16, None, True),
    (2, 700, 16, torch.bfloat16, torch.float32, True),
    (2, 333, 48, torch.bfloat16, torch.float32, False),
    (5, 1000, 1, torch.float32, None, True),
    (5, 1000, 1, torch.bfloat16, None, False),
    (5, 1000, 1, torch.bfloat16, torch.float32, True),
    (3, 77, 1, torch.float32, torch.bfloat16, False),
    (4, 2021, 1, torch.float32, None, False),
    (4, 40000, 16, torch.bfloat16, None, False),
    (2, 90000, 1, torch.float32, None, True),
])
def test_matrix_pipelined_shapes(B, T, m, dtype, out, reverse):
    w = W.make_matrix(B, T, 16, m, dtype, reverse=reverse, seed=160 + m + T % 97, out_dtype=out)
    _announce(w)
    got = run_gpu(w, DEV)
    assert got.dtype == (out or dtype)
    f32_bar = (out or dtype) == torch.float32
    assert_matrix_close(got, run_oracle(w), MS_TOL_F32 if f32_bar else MS_TOL_BF16)


@pytest.mark.parametrize("dtype,m", [(torch.float32, 1), (torch.bfloat16, 16)])
def test_matrix_pipelined_broadcast_a(dtype, m):
    g = torch.Generator().manual_seed(170 + m)
    eye = torch.eye(16)
    b = torch.randn(3, 500, 16, m, generator=g).to(dtype)
    a = (0.9 * eye + 0.01 * torch.randn(1, 500, 16, 16, generator=g)).to(dtype)  # one a for every batch
    ref = oracle.matrix_scan(a.float().numpy(), b.float().numpy(), axis=1)
    got = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=1)
    tol = MS_TOL_F32 if dtype == torch.float32 else MS_TOL_BF16
    assert_matrix_close(got, ref, tol)
    a2 = (0.9 * eye + 0.01 * torch.randn(3, 1, 16, 16, generator=g)).to(dtype)  # constant in time
    ref = oracle.matrix_scan(a2.float().numpy(), b.float().numpy(), axis=1, reverse=True)
    got = sx.matrix_scan(a2.to(DEV), b.to(DEV), axis=1, reverse=True)
    assert_matrix_close(got, ref, tol)


# The pipelined kernel hands staged inputs and look-back state between waves and
# workgroups; a handoff made too early shows up only now and then (it did: a
# stage signalled before its last copy landed). Repeated calls on one workspace,
# zero-filled once, are checked one by one; before each call everything after
# the workspace header (flags and published maps and states, whatever earlier
# calls left) is overwritten with random bytes, none of which may count as
# published by the next call.
@pytest.mark.parametrize("idx", [3, 4])
def test_matrix_repeated_calls_dirty_workspace(idx):
    from scan_primitives_amd import _binding as Bd
    (w,) = W.standard_workloads([idx])
    _announce(w)
    t = w.on(DEV)
    a, b = t["a"], t["b"]
    ref = run_oracle(w)
    lib = Bd.load_library()
    i64 = Bd.i64_array
    ws_bytes = lib.sx_matrix_scan_workspace_bytes(a.dim(), i64(a.shape), b.dim(), i64(b.shape), w.axis)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(b)
    code = Bd._DTYPES[a.dtype]
    tol = MS_TOL_F32 if a.dtype == torch.float32 else MS_TOL_BF16
    for rep in range(6):
        ws[256:].random_(0, 256)
        st = lib.sx_matrix_scan(code, a.dim(), i64(a.shape), i64(a.stride()), a.data_ptr(), b.dim(), i64(b.shape),
                                i64(b.stride()), b.data_ptr(), w.axis, 1 if w.reverse else 0, 0, code, out.data_ptr(),
                                ws.data_ptr(), ws_bytes, Bd._stream_handle(a.device))
        assert st == 0, lib.sx_last_error()
        st = lib.sx_matrix_scan_workspace_status(ws.data_ptr(), ws_bytes, Bd._stream_handle(a.device))
        assert st == 0, lib.sx_last_error()
        assert_matrix_close(out, ref, tol)


@pytest.mark.parametrize("idx", [3, 4])
def test_matrix_step_residual_repeated_calls(idx):
    """Every stored state must follow from its predecessor by one step of the
    recurrence: r[t] = h[t] - (a[t] @ h[t-1] + b[t]) (h[t+1] for :reverse).
    The residual locates an error where it enters (a state handed across a
    unit boundary shows up at that step alone), whereas a comparison with the
    oracle sees it only if the products downstream do not damp it below the
    tolerance. Twenty calls on a dirty workspace; the bar is the storage
    rounding of h (bf16 keeps 8 bits), relative to the RMS state norm."""
    from scan_primitives_amd import _binding as Bd
    (w,) = W.standard_workloads([idx])
    _announce(w)
    assert w.axis == 1
    t = w.on(DEV)
    a, b = t["a"], t["b"]
    af, bf = a.float(), b.float()
    lib = Bd.load_library()
    i64 = Bd.i64_array
    ws_bytes = lib.sx_matrix_scan_workspace_bytes(a.dim(), i64(a.shape), b.dim(), i64(b.shape), w.axis)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(b)
    code = Bd._DTYPES[a.dtype]
    bar = 1e-4 if out.dtype == torch.float32 else 1.5e-2
    for rep in range(20):
        ws[256:].random_(0, 256)
        st = lib.sx_matrix_scan(code, a.dim(), i64(a.shape), i64(a.stride()), a.data_ptr(), b.dim(), i64(b.shape),
                                i64(b.stride()), b.data_ptr(), w.axis, 1 if w.reverse else 0, 0, code, out.data_ptr(),
                                ws.data_ptr(), ws_bytes, Bd._stream_handle(a.device))
        assert st == 0, lib.sx_last_error()
        h = out.float()
        zero = torch.zeros_like(h[:, :1])
        prev = torch.cat([h[:, 1:], zero], dim=1) if w.reverse else torch.cat([zero, h[:, :-1]], dim=1)
        res = (h - (torch.matmul(af, prev) + bf)).flatten(2).norm(dim=-1)
        scale = h.flatten(2).norm(dim=-1).pow(2).mean(dim=1, keepdim=True).sqrt()
        rel = res / scale
        worst = int(torch.argmax(rel).item())
        assert rel.max().item() <= bar, (f"call {rep}: residual {rel.max().item():.3g} at (batch, t) = "
                                         f"{divmod(worst, rel.shape[1])}")
    st = lib.sx_matrix_scan_workspace_status(ws.data_ptr(), ws_bytes, Bd._stream_handle(a.device))
    assert st == 0, lib.sx_last_error()


# "Tensor operations", Errors: a failure is a reported code. A look-back that
# gives up waiting for an earlier chunk (its bounded wait reaches the limit)
# must be reported, not return wrong states silently. A spin limit of one poll,
# set from the host, makes every look-back that finds an earlier chunk not yet
# published give up at once; every kernel still runs to its end. The next
# check after the default limit is back must find nothing.
def test_matrix_lookback_give_up_is_reported():
    w = W.make_matrix(32, 8192, 16, 1, torch.float32, seed=4)
    _announce(w)
    t = w.on(DEV)
    sx.matrix_scan(t["a"], t["b"], axis=1)
    sx.matrix_scan_status()  # nothing to report before
    sx.set_lookback_spin_limit(1)
    try:
        for _ in range(4):
            sx.matrix_scan(t["a"], t["b"], axis=1)
        with pytest.raises(sx.SxError) as e:
            sx.matrix_scan_status()
        assert e.value.name == "E-DEVICE" and "gave up" in str(e.value)
    finally:
        sx.set_lookback_spin_limit(0)
    sx.matrix_scan_status()  # cleared by the check that reported it
    got = sx.matrix_scan(t["a"], t["b"], axis=1)
    sx.matrix_scan_status()
    assert_matrix_close(got, run_oracle(w), MS_TOL_F32)


def _worst_state_error(got, ref, axis=1):
    from tests.helpers import matrix_state_errors
    num, den = matrix_state_errors(got, ref)
    scale = np.maximum(den, np.sqrt(np.mean(den ** 2, axis=axis, keepdims=True)))
    return float(np.max(num / scale))


# "Tensor operations", Operations table, matrix-scan row: under bf16 the scan is
# computed in f32. With bf16 operands widened exactly, an f32 result must then be
# as close to the float64 oracle as the f32-operand path's result on the same
# (widened) values: every product a[t] @ h must be exact, as it is on the f32
# path. A state carried in fewer bits (a bf16 split of h into two parts keeps
# about 17) is about a hundred times further off at these lengths and fails.
# The shapes take the pipelined kernel (n = 16, m = 1 and m = 16) and the
# per-unit kernel (m = 17; n = 12).
@pytest.mark.parametrize("B,T,n,m,reverse", [
    (5, 1000, 16, 1, False),
    (2, 2000, 16, 16, True),
    (3, 1200, 16, 17, False),
    (4, 1000, 12, 1, True),
])
def test_matrix_bf16_in_f32_out_matches_f32_path(B, T, n, m, reverse):
    w = W.make_matrix(B, T, n, m, torch.bfloat16, reverse=reverse, seed=150 + m + n, out_dtype=torch.float32)
    _announce(w)
    a, b = w.tensors["a"], w.tensors["b"]
    ref = run_oracle(w)
    got = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=1, reverse=reverse, out_dtype=torch.float32)
    assert got.dtype == torch.float32
    f32 = sx.matrix_scan(a.float().to(DEV), b.float().to(DEV), axis=1, reverse=reverse)
    e_bf16, e_f32 = _worst_state_error(got, ref), _worst_state_error(f32, ref)
    print(f"worst per-state error: bf16 operands {e_bf16:.3e}, f32 operands {e_f32:.3e}", flush=True)
    assert_matrix_close(got, ref, MS_TOL_F32)
    assert e_bf16 <= 2.0 * e_f32 + 1e-7, (e_bf16, e_f32)


@pytest.mark.parametrize("dtype,m,reverse", [(torch.float32, 1, False), (torch.bfloat16, 16, True)])
def test_matrix_batch_offsets_past_32_bits(dtype, m, reverse):
    """a as a view whose batch stride is 2^31 elements (offsets past 32 bits)
    on the pipelined kernels' shapes: every offset is formed in 64 bits."""
    g = torch.Generator().manual_seed(153 + m)
    T = 500
    a = (0.9 * torch.eye(16) + 0.01 * torch.randn(2, T, 16, 16, generator=g)).to(dtype)
    b = torch.randn(2, T, 16, m, generator=g).to(dtype)
    base = torch.empty(2 ** 31 + T * 256 + 64, dtype=dtype, device=DEV)
    av = base.as_strided((2, T, 16, 16), (2 ** 31, 256, 16, 1))
    av.copy_(a.to(DEV))
    ref = oracle.matrix_scan(a.float().numpy(), b.float().numpy(), axis=1, reverse=reverse)
    got = sx.matrix_scan(av, b.to(DEV), axis=1, reverse=reverse)
    assert_matrix_close(got, ref, MS_TOL_F32 if dtype == torch.float32 else MS_TOL_BF16)
    del base, av
    torch.cuda.empty_cache()


def test_matrix_broadcast_leading_dims_and_negative_axis():
    g = torch.Generator().manual_seed(151)
    a = 0.9 * torch.eye(5) + 0.05 * torch.randn(1, 40, 5, 5, generator=g)  # shared across the batch
    b = torch.randn(3, 40, 5, 2, generator=g)
    ref = oracle.matrix_scan(a.numpy(), b.numpy(), axis=-1)
    got = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=-1)
    assert got.shape == b.shape
    assert_matrix_close(got, ref, MS_TOL_F32, axis=1)
    # time-invariant a: a has no time axis and broadcasts over it (stride 0)
    a2 = 0.5 * torch.randn(3, 1, 5, 5, generator=g)
    ref = oracle.matrix_scan(a2.numpy(), b.numpy(), axis=1)
    got = sx.matrix_scan(a2.to(DEV), b.to(DEV), axis=1)
    assert_matrix_close(got, ref, MS_TOL_F32)


def test_matrix_scan_closed_forms_on_device():
    g = torch.Generator().manual_seed(152)
    b = torch.randn(2, 77, 4, 3, generator=g)
    got = sx.matrix_scan(torch.zeros(2, 77, 4, 4, device=DEV), b.to(DEV), axis=1)
    assert torch.equal(got.cpu(), b)                          # a = 0 gives b
    eye = torch.eye(4).expand(2, 77, 4, 4)
    got = sx.matrix_scan(eye.to(DEV), b.to(DEV), axis=1)
    np.testing.assert_allclose(got.cpu().numpy(), np.cumsum(b.numpy().astype(np.float64), axis=1),
                               rtol=1e-5, atol=1e-4)           # a = I gives a prefix sum


def test_matrix_scan_empty_and_errors():
    out = sx.matrix_scan(torch.zeros(2, 0, 3, 3, device=DEV), torch.zeros(2, 0, 3, 1, device=DEV), axis=1)
    assert out.shape == (2, 0, 3, 1)
    with pytest.raises(sx.SxError) as e:
        sx.matrix_scan(torch.zeros(2, 4, 17, 17, device=DEV), torch.zeros(2, 4, 17, 1, device=DEV), axis=1)
    assert e.value.name == "E-DIM-001"


# ------------------------------------------------------------------ the standard workloads at full size


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_standard_workload_full_size(idx):
    (w,) = W.standard_workloads([idx])
    _announce(w)
    got = run_gpu(w, DEV)
    torch.cuda.synchronize()
    ref = run_oracle(w)
    if w.op == "element_scan":
        assert_element_close(got, ref)
    else:
        tol = MS_TOL_F32 if w.tensors["a"].dtype == torch.float32 else MS_TOL_BF16
        assert_matrix_close(got, ref, tol)
