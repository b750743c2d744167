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
elementwise, for grad_initial (floored by its own RMS), grad_x and grad_s. The
gradient of a width-one sequence under a vector state is a sum over the state
of full-width terms; its scale is also floored by the sum of those terms'
scales (the same bar carried through the sum: where the terms cancel, f32
keeps an error of their size, not of the result's).

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


def _scale(ref, axis):
    """The per-element scale of the bar: max(|ref|, RMS of |ref| along the scan axis)."""
    if axis is None:
        floor = np.sqrt(np.mean(ref ** 2))
    else:
        floor = np.sqrt(np.mean(ref ** 2, axis=axis, keepdims=True))
    return np.maximum(np.abs(ref), floor)


TIE = 1e-5  # |y|^2 this close to 1 (relative): the two sides' f32 sums may take the cap either way


def _norm_cap_ties(init, x, s, axis, reverse):
    """Decision-dependent elements of a norm-cap gradient.

    Both sides decide the cap (|y|^2 > 1) in f32 from the same forward states,
    but sum |y|^2 in different orders, so a trip whose |y|^2 is within a few
    ulps of 1 may go either way; either result is a correct f32 evaluation.
    The trips after it in scan order do not depend on that decision (the
    gradient runs last to first); it and the trips before it, and
    grad_initial, do. Returns (mask over h's shape, mask over initial's
    shape), true where an element depends on such a near tie."""
    x32, s32, i32 = (np.asarray(t.numpy(), dtype=np.float32) for t in (x, s, init))
    h32 = oracle.element_scan("norm_cap", i32, [x32, s32], axis=axis, state_axis=-1, reverse=reverse,
                              dtype=np.float32)
    ax = axis % h32.ndim
    n = h32.shape[-1]
    ht = np.moveaxis(h32, ax, 0)
    xt = np.moveaxis(np.broadcast_to(x32, x32.shape[:-1] + (n,)), ax, 0)
    st = np.moveaxis(np.broadcast_to(s32, s32.shape[:-1] + (n,)), ax, 0)
    T = ht.shape[0]
    order = list(range(T - 1, -1, -1)) if reverse else list(range(T))
    dep = np.zeros(ht.shape[:-1], dtype=bool)  # [T, lanes...]
    hit = np.zeros(ht.shape[1:-1], dtype=bool)
    for i in range(T - 1, -1, -1):  # last to first: a tie marks itself and every earlier trip
        t = order[i]
        hp = ht[order[i - 1]] if i > 0 else i32
        y = st[t] * hp + xt[t]
        ss = np.sum(y.astype(np.float64) ** 2, axis=-1)
        hit |= np.abs(ss - 1.0) < TIE
        dep[t] = hit
    mask = np.moveaxis(np.broadcast_to(dep[..., None], ht.shape), 0, ax)
    return mask, hit[..., None] if init.dim() == hit.ndim + 1 else hit


def _close(got, ref, axis, what, summed_scale=None, skip=None, g_rms=0.0):
    """summed_scale: for a width-one sequence's gradient (a sum over the state of
    full-width terms), the sum of those terms' scales, so that the bar is the
    per-element bar carried through the sum (cancellation in the sum leaves the
    f32 result with an error of the size of its terms, not of the result).
    g_rms: the RMS of the incoming gradient; a gradient that vanishes by
    cancellation (a capped trip of a width-one norm-cap state maps y to y / |y|,
    whose derivative is zero) keeps an f32 residue of a few ulps of the terms
    that cancel, so the scale has a floor of 8 ulps of g_rms over the bar."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if ref.size == 0:
        return
    scale = np.maximum(_scale(ref, axis), max(1e-6, 8 * 2.0 ** -24 / TOL * g_rms))
    if summed_scale is not None:
        scale = np.maximum(scale, summed_scale)
    if skip is not None:  # near-tie dependent elements: either branch is correct; they must be finite
        skip = np.broadcast_to(skip, g.shape)
        assert np.all(np.isfinite(g[skip])), f"{what}: non-finite values where a near tie decides"
        g, ref, scale = g[~skip], ref[~skip], scale[~skip]
        if ref.size == 0:
            return
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
    sums = [None, None]
    if state_axis is not None and g.shape[-1] > 1 and 1 in (x.shape[-1], s.shape[-1]):
        # width-one sequences: the full-width terms their gradients sum, from the oracle on broadcast copies
        full = tuple(g.shape)
        _, terms = oracle.element_scan_vjp(body, init.numpy(), [x.expand(full).numpy().copy(),
                                           s.expand(full).numpy().copy()], g.numpy(), axis=axis,
                                           state_axis=state_axis, reverse=reverse)
        for i, t in enumerate((x, s)):
            if t.shape[-1] == 1:
                sums[i] = np.sum(_scale(terms[i], ax), axis=-1, keepdims=True)
    skip_h, skip_i = (None, None)
    if body == "norm_cap":
        skip_h, skip_i = _norm_cap_ties(init, x, s, axis, reverse)
    g_rms = float(np.sqrt(np.mean(g.numpy().astype(np.float64) ** 2))) if g.numel() else 0.0
    _close(gi, ri, None, "grad_initial", skip=skip_i, g_rms=g_rms)
    _close(gx, rx, ax, "grad_x", sums[0], skip=_width(skip_h, x), g_rms=g_rms)
    _close(gs, rs, ax, "grad_s", sums[1], skip=_width(skip_h, s), g_rms=g_rms)


def _width(mask, t):
    """A mask over h's shape narrowed to a width-one sequence's (any element of the state)."""
    if mask is None or t.shape[-1] == mask.shape[-1]:
        return mask
    return np.any(mask, axis=-1, keepdims=True)


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


@pytest.mark.parametrize("case", ["certified", "gate_one", "mixed", "zero_g_lane", "zero_gate", "small_x"])
@pytest.mark.parametrize("n,sw", [(16, 1), (5, 5)])
@pytest.mark.parametrize("reverse", [False, True])
def test_norm_cap_split_axis(case, n, sw, reverse):
    """Few state vectors and a long axis: the sweep is cut into chunks with certified warm-ups.
    gate_one makes the per-trip bound reach 1 (no certificate: the lane runs exactly from the
    sweep's start), mixed has such lanes beside certified ones, zero_g_lane a lane whose upstream
    gradient is zero, zero_gate gates of zero (the adjoint never crosses a trip), small_x bounds
    just under 1 (long warm-ups)."""
    gen = torch.Generator().manual_seed(161 + n)
    B, T, C = 2, 1500, 3
    x = 2.0 * torch.randn((B, T, C, n), generator=gen)
    s = 0.8 + 0.2 * torch.rand((B, T, C, sw), generator=gen)
    g = torch.randn((B, T, C, n), generator=gen)
    if case == "gate_one":
        s = torch.ones_like(s)
        x = 0.5 * x
    elif case == "mixed":
        s[:, :, 1] = 1.0
        x[:, :, 1] *= 0.25
    elif case == "zero_g_lane":
        g[1, :, 2] = 0.0
    elif case == "zero_gate":
        s = torch.zeros_like(s)
    elif case == "small_x":
        x = 0.35 * x
    init = 0.3 * torch.randn((B, C, n), generator=gen)
    _run("norm_cap", x, s, init, g, 1, -1, reverse)


@pytest.mark.parametrize("lead", [(2, 40, 4200), (3, 20, 2), (1, 33, 1)])
@pytest.mark.parametrize("xw,sw", [(16, 1), (1, 16), (1, 1), (16, 16)])
def test_norm_cap_width_one_sums(lead, xw, sw):
    """Width-one x or gate under a 16-wide state, summed over the state inside the norm-cap
    kernels: many state vectors (one row each), a short axis (one row each) and the
    shortest split axis."""
    x, s, full, gen = _draw("norm_cap", lead, 16, seed=171 + xw + sw, x_width=xw, s_width=sw)
    init = 0.3 * torch.randn((lead[0], lead[2], 16), generator=gen)
    g = torch.randn(full, generator=gen)
    _run("norm_cap", x, s, init, g, 1, -1, False)


@pytest.mark.parametrize("lead,reverse", [((1, 1, 1), False), ((2, 1, 1), True), ((2, 7, 1), False), ((3, 300, 2), True)])
def test_norm_cap_state_width_one(lead, reverse):
    """A norm-cap state of width one: a capped trip maps y to y / |y| = +-1, whose
    derivative is zero, so the gradient through it vanishes by cancellation (the
    oracle's float64 gives zeros, f32 a residue of a few ulps of the terms)."""
    x, s, full, gen = _draw("norm_cap", lead, 1, seed=181 + lead[1], x_width=1, s_width=1)
    init = 0.3 * torch.randn((lead[0], lead[2], 1), generator=gen)
    g = torch.randn(full, generator=gen)
    _run("norm_cap", x, s, init, g, 1, -1, reverse)


@pytest.mark.parametrize("T", [20, 600])
def test_norm_cap_unaligned_views(T):
    """x and the gate as views whose offsets are not multiples of four elements: the
    one-component-per-thread kernels take these (the four-per-thread ones need 16-byte
    alignment)."""
    gen = torch.Generator().manual_seed(181)
    xb = 2.0 * torch.randn((3, T, 5, 17), generator=gen)
    sb = 0.8 + 0.2 * torch.rand((3, T, 5, 17), generator=gen)
    x, s = xb[..., 1:], sb[..., :16]
    init = 0.3 * torch.randn((3, 5, 16), generator=gen)
    g = torch.randn((3, T, 5, 16), generator=gen)
    print(f"\n[case] norm_cap unaligned views T {T}", flush=True)
    xd, sd = xb.to(DEV)[..., 1:], sb.to(DEV)[..., :16]
    h32 = oracle.element_scan("norm_cap", init.numpy(), [x.numpy(), s.numpy()], axis=1, state_axis=-1,
                              dtype=np.float32)
    gi, (gx, gs) = sx.element_scan_backward("norm_cap", init.to(DEV), [xd, sd],
                                            torch.from_numpy(np.ascontiguousarray(h32)).to(DEV), g.to(DEV),
                                            axis=1, state_axis=-1)
    torch.cuda.synchronize()
    ri, (rx, rs) = oracle.element_scan_vjp("norm_cap", init.numpy(), [x.numpy(), s.numpy()], g.numpy(), axis=1,
                                           state_axis=-1)
    skip_h, skip_i = _norm_cap_ties(init, x, s, 1, False)
    _close(gi, ri, None, "grad_initial", skip=skip_i)
    _close(gx, rx, 1, "grad_x", skip=skip_h)
    _close(gs, rs, 1, "grad_s", skip=skip_h)


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
    skip_h, skip_i = _norm_cap_ties(init, x, s, 1, reverse) if body == "norm_cap" else (None, None)
    _close(idd.grad, ri, None, "grad_initial", skip=skip_i)
    _close(xd.grad, rx, 1, "grad_x", skip=_width(skip_h, x))
    _close(sd.grad, rs, 1, "grad_s", skip=_width(skip_h, s))


def test_element_grad_errors():
    x = torch.zeros((2, 5, 3), device=DEV)
    with pytest.raises(sx.SxError) as e:
        sx.element_scan_backward("max_plus", torch.zeros((2, 3), device=DEV), [x, x], x, x[:, :4], axis=1)
    assert e.value.name == "E-DIM-001"
    with pytest.raises(sx.SxError) as e:
        sx.element_scan_backward("max_plus", torch.zeros((2, 3), device=DEV), [x, x.double()], x, x, axis=1)
    assert e.value.name == "E-DIM-002"
