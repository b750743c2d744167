"""Seeded random shapes, GPU against the oracle.

The fixed parity cases pin each kernel path and edge case by hand; these draw
shapes, axes, directions and dtypes at random (a fixed seed per case, so every
case is reproducible by its id) to reach combinations the fixed cases do not:
matrix-scan forward and gradient over n, m, the scan axis among the leading
dims and both dtypes (which selects the pipelined, per-unit or fused-gradient
paths), element-scan bodies, linear-scan and table-scan over shapes both
below and above the slab kernel's thresholds, the element-scan gradients
(scalar and vector states, width-one sequences, long axes that norm-cap's
gradient splits) and :projective (products that shrink or grow). Bars as in
the fixed tests.
"""

import random

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W
from tests.helpers import (MS_TOL_BF16, MS_TOL_F32, assert_element_close, assert_linear_close, assert_matrix_close,
                           run_gpu, run_oracle)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _blocks_close(got, ref, tol, what):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    num = np.sqrt(np.sum((g - ref) ** 2, axis=(-2, -1)))
    den = np.sqrt(np.sum(ref ** 2, axis=(-2, -1)))
    if den.size == 0:
        return
    scale = np.maximum(den, np.sqrt(np.mean(den ** 2)))
    bad = num > tol * scale
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {num.size} blocks outside {tol}; worst "
                           f"{np.max(num / np.maximum(scale, 1e-300)):.3e}")


@pytest.mark.parametrize("case", range(40))
def test_matrix_scan_random(case):
    rng = random.Random(7000 + case)
    n = rng.choice([16, 16, 16, 1, 3, 5, 8, 13])
    m = rng.choice([1, 1, 16, 16, 2, 3, 17, 32])
    dt = rng.choice([torch.float32, torch.bfloat16])
    T = rng.choice([1, 2, 17, 95, 96, 97, 191, 300, 577, 1000])
    lead = list(rng.choice([(2,), (3,), (1,), (2, 3), (5,)]))
    reverse = rng.random() < 0.5
    pos = rng.randrange(len(lead) + 1)  # where the scan axis sits among the leading dims
    lead.insert(pos, T)
    axis = pos if rng.random() < 0.5 else pos - len(lead)
    g = torch.Generator().manual_seed(7000 + case)
    a = (0.9 * torch.eye(n) + 0.05 * torch.randn(tuple(lead) + (n, n), generator=g)).to(dt)
    b = torch.randn(tuple(lead) + (n, m), generator=g).to(dt)
    print(f"\n[case] a {tuple(a.shape)} b {tuple(b.shape)} {dt} axis {axis} reverse {reverse}", flush=True)
    tol = MS_TOL_F32 if dt == torch.float32 else MS_TOL_BF16
    h = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=axis, reverse=reverse)
    ref = oracle.matrix_scan(a.float().numpy(), b.float().numpy(), axis=axis, reverse=reverse)
    assert_matrix_close(h, ref, tol, axis=axis % len(lead))
    gh = torch.randn(tuple(h.shape), generator=g).to(dt)
    ga, gb = sx.matrix_scan_backward(a.to(DEV), tuple(b.shape), h, gh.to(DEV), axis=axis, reverse=reverse)
    torch.cuda.synchronize()
    ra, rb = oracle.matrix_scan_vjp(a.float().numpy(), b.float().numpy(), gh.float().numpy(), axis=axis,
                                    reverse=reverse)
    _blocks_close(gb, rb, tol, "grad_b")
    _blocks_close(ga, ra, tol, "grad_a")
    if dt == torch.bfloat16:  # bf16 in, f32 out: held to the f32 bar
        h32 = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=axis, reverse=reverse, out_dtype=torch.float32)
        assert_matrix_close(h32, ref, MS_TOL_F32, axis=axis % len(lead))


@pytest.mark.parametrize("case", range(40))
def test_element_linear_table_random(case):
    rng = random.Random(8000 + case)
    kind = rng.choice(["tanh", "max_plus", "max_plus_slab", "norm_cap", "linear", "linear_slab", "table"])
    reverse = rng.random() < 0.5
    seed = 8000 + case
    if kind in ("tanh", "max_plus", "max_plus_slab"):
        if kind == "max_plus_slab":  # at least 8192 lanes and 512 trips
            shape, axis = (rng.choice([2, 3]), rng.choice([512, 600, 777]), rng.choice([4096, 4100])), 1
        else:
            nd = rng.choice([2, 3, 4])
            shape = tuple(rng.choice([1, 2, 3, 17, 64, 65, 130]) for _ in range(nd))
            axis = rng.randrange(nd) - (nd if rng.random() < 0.5 else 0)
        w = (W.make_tanh if kind == "tanh" else W.make_max_plus)(shape, axis=axis, reverse=reverse, seed=seed)
        print(f"\n[case] {w.name}", flush=True)
        got = run_gpu(w, DEV)
        torch.cuda.synchronize()
        assert_element_close(got, run_oracle(w))
    elif kind == "norm_cap":
        B, T, H = rng.choice([1, 2, 3]), rng.choice([1, 5, 40, 300, 1024]), rng.choice([1, 3, 16])
        n = rng.choice([16, 16, 5, 1])
        w = W.make_norm_cap(B, T, H, n, gate_width=rng.choice([1, n]), reverse=reverse, seed=seed,
                            zero_initial=rng.random() < 0.5)
        print(f"\n[case] {w.name}", flush=True)
        got = run_gpu(w, DEV)
        torch.cuda.synchronize()
        assert_element_close(got, run_oracle(w))
    elif kind in ("linear", "linear_slab"):
        if kind == "linear_slab":
            shape, axis = (2, rng.choice([512, 700]), rng.choice([4096, 4163])), 1
        else:
            nd = rng.choice([1, 2, 3])
            shape = tuple(rng.choice([1, 2, 17, 64, 300]) for _ in range(nd))
            axis = rng.randrange(nd)
        dt = rng.choice([torch.float32, torch.bfloat16])
        w = W.make_linear(shape, axis=axis, reverse=reverse, dtype=dt,
                          a_kind=rng.choice(["decay", "signed", "ones", "number"]), seed=seed)
        print(f"\n[case] {w.name}", flush=True)
        got = run_gpu(w, DEV)
        torch.cuda.synchronize()
        assert_linear_close(got, run_oracle(w), MS_TOL_F32 if dt == torch.float32 else MS_TOL_BF16, axis)
    else:
        B, T = rng.choice([1, 3, 64, 300]), rng.choice([1, 7, 1023, 1024, 1025, 3000])
        w = W.make_table(rng.choice(["parity", "dfa16"]), B, T, axis=rng.choice([-1, 1]),
                         start=rng.choice([0, 1]), seed=seed)
        print(f"\n[case] {w.name} axis {w.axis} start {w.meta['start']}", flush=True)
        t = w.tensors
        got = sx.table_scan(t["table"].to(DEV), t["symbols"].to(DEV), axis=w.axis, start=w.meta["start"])
        ref = oracle.table_scan(t["table"].numpy(), t["symbols"].numpy(), axis=w.axis, start=w.meta["start"])
        assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("case", range(24))
def test_element_gradient_random(case):
    # the element-scan gradients (scalar and vector states, width-one sequences, norm-cap's split along
    # the axis), checked as the fixed gradient tests check them, near-tie handling included
    from tests.test_element_grad_gpu import _draw, _run

    rng = random.Random(9000 + case)
    body = rng.choice(["tanh_affine", "max_plus", "norm_cap"])
    reverse = rng.random() < 0.5
    if body != "norm_cap" and rng.random() < 0.5:  # scalar state
        nd = rng.choice([2, 3])
        shape = tuple(rng.choice([1, 2, 5, 37, 130, 600]) for _ in range(nd))
        axis = rng.randrange(nd) - (nd if rng.random() < 0.5 else 0)
        x, s, _, gen = _draw(body, shape, None, seed=9000 + case)
        ax = axis % nd
        init = torch.randn(shape[:ax] + shape[ax + 1:], generator=gen)
        g = torch.randn(shape, generator=gen)
        _run(body, x, s, init, g, axis, None, reverse)
    else:  # vector state along the last axis, the scan along axis 1
        n = rng.choice([16, 16, 5, 1])
        lead = (rng.choice([1, 2]), rng.choice([1, 7, 45, 300, 1500]), rng.choice([1, 3]))
        xw, sw = rng.choice([n, 1]), rng.choice([n, 1])
        x, s, full, gen = _draw(body, lead, n, seed=9000 + case, x_width=xw, s_width=sw)
        init = 0.3 * torch.randn((lead[0], lead[2], n), generator=gen)
        g = torch.randn(full, generator=gen)
        _run(body, x, s, init, g, 1, -1, reverse)


@pytest.mark.parametrize("case", range(16))
def test_projective_random(case):
    rng = random.Random(9500 + case)
    n = rng.choice([16, 16, 5, 1])
    m = rng.choice([1, 16, 3, 17])
    dt = torch.bfloat16 if (n == 16 and m == 16 and rng.random() < 0.5) else torch.float32
    T = rng.choice([1, 5, 127, 128, 129, 300, 1000])
    B = rng.choice([1, 2, 3])
    reverse = rng.random() < 0.5
    g = torch.Generator().manual_seed(9500 + case)
    a = (rng.choice([0.9, 1.5]) * torch.eye(n) + 0.05 * torch.randn((B, T, n, n), generator=g)).to(dt)
    b = torch.randn((B, T, n, m), generator=g).to(dt)
    print(f"\n[case] projective a {tuple(a.shape)} b {tuple(b.shape)} {dt} reverse {reverse}", flush=True)
    got = sx.matrix_scan(a.to(DEV), b.to(DEV), axis=1, reverse=reverse, projective=True)
    torch.cuda.synchronize()
    ref = oracle.matrix_scan_projective(a.float().numpy(), b.float().numpy(), axis=1, reverse=reverse)
    assert np.all(np.isfinite(got.float().cpu().numpy()))
    assert_matrix_close(got, ref, MS_TOL_F32 if dt == torch.float32 else MS_TOL_BF16, axis=1)
