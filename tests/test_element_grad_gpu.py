"""Parity of the HIP element-scan gradients with the CPU oracle's.

Each case draws seeded inputs and an upstream gradient g, computes the
forward states h with the oracle in float32 (the precision the scan runs in;
for max-plus this is the serial float32 evaluation, exact), and runs the GPU
gradient on those h; the oracle's gradient (``oracle.element_scan_vjp``,
float64 values, branch decisions in float32 from the same float32 forward)
is the reference. So both sides take every branch decision (max-plus's
winner, norm-cap's cap) from the same states.

The bar is that of a linear scan, which the adjoint is: |gpu - ref| <=
1e-4 * max(|ref|, RMS of |ref| over the scan axis of the same lane, 1e-6)
elementwise, for grad_initial (floored by its own RMS), grad_x and grad_s.

Separate cases run GPU forward and GPU backward end to end through autograd
(``sx.element_scan`` with inputs that require grad), where the lane kernels'
forward states equal the serial float32 evaluation for max-plus.
"""

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4


def _close(got, ref, axis, what):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if ref.size == 0:
        return
    if axis is None:
        floor = np.sqrt(np.mean(ref ** 2))
    else:
        floor = np.sqrt(np.mean(ref ** 2, axis=axis, keepdims=True))
    scale = np.maximum(np.maximum(np.abs(ref), floor), 1e-6)
    err = np.abs(g - ref)
    bad = err > TOL * scale
    if bad.any():
        idx = np.unravel_index(np.argmax(err / scale), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside; worst at {idx}: got {g[idx]!r} "
                             f"ref {ref[idx]!r} (rel {err[idx] / scale[idx]:.3e})")


def _draw(body, shape, state, seed, x_width=None, s_width=None):
    """x, s, initial in the shapes the body takes; state None (scalar) or the state width n."""
    gen = torch.Generator().manual_seed(seed)
    if state is None:
        x = torch.randn(shape, generator=gen)
        s = (0.1 * torch.rand(shape, generator=gen)) if body == "max_plus" else torch.rand(shape, generator=gen)
        ax_shape = shape
    else:
        lead = shape
        x = (2.0 if body == "norm_cap" else 1.0) * torch.randn(lead + (x_width,), generator=gen)
        s = (0.8 + 0.2 * torch.rand(lead + (s_width,), generator=gen)) if body != "max_plus" else \
            0.1 * torch.rand(lead + (s_width,), generator=gen)
        ax_shape = lead + (state,)
    return x, s, ax_shape, gen


def _run(body, x, s, init, g, axis, state_axis, reverse):
    print(f"\n[case] {body} x {tuple(x.shape)} s {tuple(s.shape)} axis {axis} reverse {reverse}", flush=True)
    h32 = oracle.element_scan(body, init.numpy(), [x.numpy(), s.numpy()], axis=axis, state_axis=state_axis,
                              reverse=reverse, dtype=np.float32)
    gi, (gx, gs) = sx.element_scan_backward(body, init.to(DEV), [x.to(DEV), s.to(DEV)],
                                            torch.from_numpy(np.ascontiguousarray(h32)).to(DEV), g.to(DEV),
                                            axis=axis, state_axis=state_axis, reverse=reverse)
    torch.cuda.synchronize()
    ri, (rx, rs) = oracle.element_scan_vjp(body, init.numpy(), [x.numpy(), s.numpy()], g.numpy(), axis=axis,
                                           state_axis=state_axis, reverse=reverse)
    ax = axis % x.dim()
    _close(gi, ri, None, "grad_initial")
    _close(gx, rx, ax, "grad_x")
    _close(gs, rs, ax, "grad_s")


def _init_and_g(shape, axis, gen, state=False):
    ax = axis % len(shape)
    init = torch.randn(shape[:ax] + shape[ax + 1:], generator=gen)
    if state:
        init = 0.3 * init
    return init, torch.randn(shape, generator=gen)


SMALL = [((3, 37, 19), 1, False), ((3, 37, 19), 1, True), ((41, 5, 3), 0, False), ((2, 3, 130), -1, True),
         ((1, 1, 1), 1, False), ((5, 1, 7), 1, True), ((4, 200), 1, False)]


@pytest.mark.parametrize("shape,axis,reverse", SMALL)
@pytest.mark.parametrize("body", ["tanh_affine", "max_plus"])
def test_scalar_bodies_lane_kernel(body, shape, axis, reverse):
    x, s, _, gen = _draw(body, shape, None, seed=101 + len(shape))
    init, g = _init_and_g(shape, axis, gen)
    _run(body, x, s, init, g, axis, None, reverse)


@pytest.mark.parametrize("shape,axis,reverse", [((2, 600, 4163), 1, False), ((2, 600, 4163), 1, True),
                                                ((8200, 530), 1, True), ((777, 8200), 0, False)])
@pytest.mark.parametrize("body", ["tanh_affine", "max_plus"])
def test_scalar_bodies_slab_kernel(body, shape, axis, reverse):
    x, s, _, gen = _draw(body, shape, None, seed=111)
    init, g = _init_and_g(shape, axis, gen)
    _run(body, x, s, init, g, axis, None, reverse)


@pytest.mark.parametrize("n,xw,sw", [(16, 16, 1), (16, 16, 16), (5, 5, 1), (5, 1, 5), (1, 1, 1), (16, 1, 1)])
@pytest.mark.parametrize("body", ["norm_cap", "tanh_affine", "max_plus"])
@pytest.mark.parametrize("reverse", [False, True])
def test_vector_state(body, n, xw, sw, reverse):
    lead = (2, 45, 3)
    x, s, full, gen = _draw(body, lead, n, seed=121 + n + xw, x_width=xw, s_width=sw)
    init = 0.3 * torch.randn((2, 3, n), generator=gen)
    g = torch.randn(full, generator=gen)
    _run(body, x, s, init, g, 1, -1, reverse)


def test_norm_cap_workload_shape():
    # [8,1024,16,16] with a width-one gate, as the norm-cap workload (smaller x scale so both branches occur)
    gen = torch.Generator().manual_seed(131)
    x = torch.randn((8, 1024, 16, 16), generator=gen) * 0.3
    s = 0.8 + 0.2 * torch.rand((8, 1024, 16, 1), generator=gen)
    init = torch.zeros((8, 16, 16))
    g = torch.randn((8, 1024, 16, 16), generator=gen)
    _run("norm_cap", x, s, init, g, 1, -1, False)


def test_max_plus_workload_sampled_lanes():
    """The reverse max-plus workload at full size, [64,4096,256]: the GPU gradient
    of every lane from the oracle's float32 forward states; the oracle gradient
    on 512 sampled lanes (lanes are independent, so a slice is an exact sub-problem)."""
    from scan_primitives_amd import workloads as W
    w = W.make_max_plus()
    print(f"\n[case] gradient of {w.name}", flush=True)
    t = w.tensors
    gen = torch.Generator().manual_seed(141)
    g = torch.randn(tuple(t["x"].shape), generator=gen)
    h32 = oracle.element_scan("max_plus", t["initial"].numpy(), [t["x"].numpy(), t["s"].numpy()], axis=1,
                              reverse=True, dtype=np.float32)
    gi, (gx, gs) = sx.element_scan_backward("max_plus", t["initial"].to(DEV), [t["x"].to(DEV), t["s"].to(DEV)],
                                            torch.from_numpy(h32).to(DEV), g.to(DEV), axis=1, reverse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(142)
    bi, ci = rng.integers(0, 64, 512), rng.integers(0, 256, 512)
    sl = lambda a: a[bi, :, ci]  # noqa: E731   [512, 4096]
    ri, (rx, rs) = oracle.element_scan_vjp("max_plus", t["initial"].numpy()[bi, ci], [sl(t["x"].numpy()),
                                           sl(t["s"].numpy())], sl(g.numpy()), axis=1, reverse=True)
    bt, ct = torch.as_tensor(bi), torch.as_tensor(ci)
    _close(gi.cpu()[bt, ct], ri, None, "grad_initial")
    _close(gx.cpu()[bt, :, ct], rx, 1, "grad_x")
    _close(gs.cpu()[bt, :, ct], rs, 1, "grad_c")


@pytest.mark.parametrize("body,state", [("tanh_affine", None), ("max_plus", None), ("norm_cap", 16),
                                        ("tanh_affine", 4)])
@pytest.mark.parametrize("reverse", [False, True])
def test_autograd_through_element_scan(body, state, reverse):
    lead = (3, 150, 5) if state is None else (3, 150, 2)
    if state is None:
        x, s, full, gen = _draw(body, lead, None, seed=151)
        init = torch.randn((3, 5), generator=gen)
        st = None
    else:
        x, s, full, gen = _draw(body, lead, state, seed=151, x_width=state, s_width=1)
        init = 0.3 * torch.randn((3, 2, state), generator=gen)
        st = -1
    w = torch.randn(full, generator=gen)
    xd, sd, idd = (t.to(DEV).requires_grad_() for t in (x, s, init))
    h = sx.element_scan(body, idd, [xd, sd], axis=1, state_axis=st, reverse=reverse)
    (h * w.to(DEV)).sum().backward()
    ri, (rx, rs) = oracle.element_scan_vjp(body, init.numpy(), [x.numpy(), s.numpy()], w.numpy(), axis=1,
                                           state_axis=st, reverse=reverse)
    _close(idd.grad, ri, None, "grad_initial")
    _close(xd.grad, rx, 1, "grad_x")
    _close(sd.grad, rs, 1, "grad_s")


def test_element_grad_errors():
    x = torch.zeros((2, 5, 3), device=DEV)
    with pytest.raises(sx.SxError) as e:
        sx.element_scan_backward("max_plus", torch.zeros((2, 3), device=DEV), [x, x], x, x[:, :4], axis=1)
    assert e.value.name == "E-DIM-001"
    with pytest.raises(sx.SxError) as e:
        sx.element_scan_backward("max_plus", torch.zeros((2, 3), device=DEV), [x, x.double()], x, x, axis=1)
    assert e.value.name == "E-DIM-002"
