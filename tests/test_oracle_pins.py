"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these re-types the oracle's recurrence. Each pin is a closed form, an
inverse problem (pick the states, solve for the inputs that produce them with
a different function, run the scan, get the states back), an invariant the
pages state, a special case that reduces to a library routine, or a worked
example from ``tests/golden/``. Together they fail on a dropped term, a wrong
sign, an off-by-one time index, a transposed operand, a wrong direction, or a
wrong axis.
"""

import json
import math
import pathlib

import numpy as np
import pytest

import oracle

GOLDEN = json.loads((pathlib.Path(__file__).parent / "golden" / "worked_examples.json").read_text())


def _rng(seed):
    return np.random.default_rng(seed)


def _move_time_first(arr, axis):
    return np.moveaxis(arr, axis, 0)


# --- worked examples ------------------------------------------------------------


def test_golden_tanh_affine():
    g = GOLDEN["tanh_affine_forward"]
    out = oracle.element_scan("tanh_affine", np.float64(g["initial"]), [g["x"], g["decay"]], axis=0)
    np.testing.assert_allclose(out, g["expected"], rtol=0, atol=g["tolerance"])


def test_golden_norm_cap():
    g = GOLDEN["norm_cap_forward"]
    out = oracle.element_scan("norm_cap", g["initial"], [g["x"], g["decay"]], axis=0, state_axis=-1)
    np.testing.assert_allclose(out, g["expected"], rtol=0, atol=g["tolerance"])


@pytest.mark.parametrize("key,reverse", [("max_plus_reverse", True), ("max_plus_forward", False)])
def test_golden_max_plus(key, reverse):
    g = GOLDEN[key]
    out = oracle.element_scan("max_plus", np.float64(g["initial"]), [g["x"], g["cost"]], axis=0,
                              reverse=reverse)
    np.testing.assert_array_equal(out, g["expected"])
    out32 = oracle.element_scan("max_plus", np.float32(g["initial"]), [g["x"], g["cost"]], axis=0,
                                reverse=reverse, dtype=np.float32)
    np.testing.assert_array_equal(out32, np.float32(g["expected"]))


@pytest.mark.parametrize("key,reverse", [("matrix_scan_forward", False), ("matrix_scan_reverse", True)])
def test_golden_matrix_scan(key, reverse):
    g = GOLDEN[key]
    out = oracle.matrix_scan(g["a"], g["b"], axis=0, reverse=reverse)
    np.testing.assert_array_equal(out, g["expected"])


# --- tanh-affine body -------------------------------------------------------------


@pytest.mark.parametrize("axis", [0, 1, -1])
def test_tanh_zero_decay_is_pointwise_tanh(axis):
    # decay = 0 removes the state from every trip: h[t] = tanh(x[t]).
    r = _rng(10)
    x = r.standard_normal((3, 5, 4))
    init_shape = tuple(d for i, d in enumerate(x.shape) if i != axis % 3)
    out = oracle.element_scan("tanh_affine", r.standard_normal(init_shape), [x, np.zeros_like(x)],
                              axis=axis)
    np.testing.assert_array_equal(out, np.tanh(x))


@pytest.mark.parametrize("axis,reverse", [(0, False), (1, False), (-1, True), (1, True)])
def test_tanh_inverse_problem(axis, reverse):
    # Pick states h in (-1, 1) and decays; x[t] = atanh(h[t]) - decay[t] * h_prev
    # makes the scan reproduce h. Wrong time indices or operand roles fail.
    r = _rng(11)
    shape = (3, 6, 4)
    ax = axis % 3
    h = r.uniform(-0.95, 0.95, shape)
    decay = r.uniform(-1.5, 1.5, shape)
    init = r.uniform(-2, 2, tuple(d for i, d in enumerate(shape) if i != ax))
    ht, dt = _move_time_first(h, ax), _move_time_first(decay, ax)
    xt = np.empty_like(ht)
    T = shape[ax]
    order = range(T - 1, -1, -1) if reverse else range(T)
    prev = init
    for t in order:
        xt[t] = np.arctanh(ht[t]) - dt[t] * prev
        prev = ht[t]
    x = np.moveaxis(xt, 0, ax)
    out = oracle.element_scan("tanh_affine", init, [x, decay], axis=axis, reverse=reverse)
    np.testing.assert_allclose(out, h, rtol=0, atol=1e-12)


def test_tanh_state_stays_in_open_interval():
    r = _rng(12)
    x = 3 * r.standard_normal((2, 50, 3))
    out = oracle.element_scan("tanh_affine", 5 * r.standard_normal((2, 3)),
                              [x, r.uniform(-2, 2, x.shape)], axis=1)
    assert np.all(np.abs(out) <= 1.0)


# --- norm-capped vector body -----------------------------------------------------------


@pytest.mark.parametrize("n,gate_width,reverse", [(16, 1, False), (16, 16, True), (5, 1, True), (1, 1, False)])
def test_norm_cap_inverse_problem(n, gate_width, reverse):
    # Pick states: some trips inside the unit ball (the cap does not fire, y = h),
    # some on the sphere with y = lam * h, lam > 1 (the cap fires and divides by
    # |y| = lam). Solve x = y - decay * h_prev and check the scan returns h.
    r = _rng(13 + n)
    B, T, H = 2, 9, 3
    h = r.standard_normal((B, T, H, n))
    h /= np.linalg.norm(h, axis=-1, keepdims=True)
    capped = r.random((B, T, H, 1)) < 0.5
    inside = r.uniform(0.1, 0.9, (B, T, H, 1))
    h = np.where(capped, h, h * inside)
    lam = np.where(capped, r.uniform(1.2, 3.0, (B, T, H, 1)), 1.0)
    decay = r.uniform(0.2, 1.0, (B, T, H, gate_width))
    init = 0.3 * r.standard_normal((B, H, n))
    x = np.empty_like(h)
    order = range(T - 1, -1, -1) if reverse else range(T)
    prev = init
    for t in order:
        x[:, t] = lam[:, t] * h[:, t] - decay[:, t] * prev
        prev = h[:, t]
    out = oracle.element_scan("norm_cap", init, [x, decay], axis=1, state_axis=-1, reverse=reverse)
    np.testing.assert_allclose(out, h, rtol=0, atol=1e-12)


def test_norm_cap_norm_at_most_one():
    r = _rng(14)
    x = 2 * r.standard_normal((3, 40, 2, 16))
    out = oracle.element_scan("norm_cap", 4 * r.standard_normal((3, 2, 16)),
                              [x, r.uniform(-1.2, 1.2, (3, 40, 2, 1))], axis=1, state_axis=-1)
    assert np.all(np.linalg.norm(out, axis=-1) <= 1 + 1e-12)


def test_norm_cap_linear_regime_closed_form():
    # With tiny inputs and |decay| < 1 the cap never fires, and the scan is the
    # gated linear recurrence with closed form
    # h[t] = prod_{r<=t} decay[r] * init + sum_{s<=t} prod_{s<r<=t} decay[r] * x[s].
    r = _rng(15)
    T, n = 7, 4
    x = 1e-3 * r.standard_normal((T, n))
    decay = r.uniform(0.1, 0.9, (T, 1))
    init = 1e-3 * r.standard_normal(n)
    expect = np.zeros((T, n))
    for t in range(T):
        acc = np.prod(decay[: t + 1, 0]) * init
        for s in range(t + 1):
            acc = acc + np.prod(decay[s + 1: t + 1, 0]) * x[s]
        expect[t] = acc
    out = oracle.element_scan("norm_cap", init, [x, decay], axis=0, state_axis=-1)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-18)


def test_norm_cap_saturated_is_unit_norm():
    r = _rng(16)
    x = 100 * r.standard_normal((2, 12, 16))
    out = oracle.element_scan("norm_cap", np.zeros((2, 16)), [x, r.uniform(0, 1, (2, 12, 1))],
                              axis=1, state_axis=-1)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), 1.0, rtol=0, atol=1e-12)


def test_norm_cap_needs_vector_state():
    with pytest.raises(ValueError):
        oracle.element_scan("norm_cap", np.zeros(3), [np.ones((4, 3)), np.ones((4, 3))], axis=0)


# --- max-plus body ---------------------------------------------------------------


def _max_plus_closed_form_reverse(x, c, init):
    # h[t] = max( max_{s>=t} (x[s] - sum_{r=t}^{s-1} c[r]),  init - sum_{r=t}^{T-1} c[r] )
    T = len(x)
    out = np.empty(T)
    for t in range(T):
        best = init - np.sum(c[t:])
        for s in range(t, T):
            best = max(best, x[s] - np.sum(c[t:s]))
        out[t] = best
    return out


def _max_plus_closed_form_forward(x, c, init):
    # h[t] = max( max_{s<=t} (x[s] - sum_{r=s+1}^{t} c[r]),  init - sum_{r=0}^{t} c[r] )
    T = len(x)
    out = np.empty(T)
    for t in range(T):
        best = init - np.sum(c[: t + 1])
        for s in range(t + 1):
            best = max(best, x[s] - np.sum(c[s + 1: t + 1]))
        out[t] = best
    return out


@pytest.mark.parametrize("reverse", [True, False])
def test_max_plus_closed_form(reverse):
    r = _rng(17)
    T, L = 11, 6
    x = r.standard_normal((T, L))
    c = r.uniform(0, 0.7, (T, L))
    init = r.standard_normal(L)
    out = oracle.element_scan("max_plus", init, [x, c], axis=0, reverse=reverse)
    ref = _max_plus_closed_form_reverse if reverse else _max_plus_closed_form_forward
    for lane in range(L):
        np.testing.assert_allclose(out[:, lane], ref(x[:, lane], c[:, lane], init[lane]),
                                   rtol=0, atol=1e-12)


def test_max_plus_zero_cost_is_reverse_cummax():
    # c = 0: h[t] = max(initial, max_{s>=t} x[s]), the running maximum from the end.
    r = _rng(18)
    x = r.standard_normal((4, 20, 5))
    init = r.standard_normal((4, 5))
    out = oracle.element_scan("max_plus", init, [x, np.zeros_like(x)], axis=1, reverse=True)
    ref = np.flip(np.maximum.accumulate(np.flip(x, 1), axis=1), 1)
    np.testing.assert_array_equal(out, np.maximum(ref, init[:, None, :]))


def test_max_plus_float32_mode_close_to_float64():
    r = _rng(19)
    x = r.standard_normal((300, 8)).astype(np.float32)
    c = (0.1 * r.random((300, 8))).astype(np.float32)
    init = r.standard_normal(8).astype(np.float32)
    o64 = oracle.element_scan("max_plus", init, [x, c], axis=0, reverse=True)
    o32 = oracle.element_scan("max_plus", init, [x, c], axis=0, reverse=True, dtype=np.float32)
    assert o32.dtype == np.float32
    np.testing.assert_allclose(o32, o64, rtol=1e-6, atol=1e-6)


# --- direction, axis and shape invariants for all bodies -----------------------------


@pytest.mark.parametrize("body,state_axis", [("tanh_affine", None), ("max_plus", None), ("norm_cap", -1),
                                             ("tanh_affine", -1), ("max_plus", -1)])
def test_reverse_is_flip_scan_flip(body, state_axis):
    # "Nonlinear element scans": reversing the sequences along the axis, scanning
    # forward and reversing the result gives what the :reverse scan gives.
    r = _rng(20)
    x = r.standard_normal((3, 13, 2, 4))
    s = r.uniform(0, 1, (3, 13, 2, 1 if state_axis is not None else 4))
    if state_axis is None:
        s = np.broadcast_to(s, x.shape).copy()
    init = r.standard_normal((3, 2, 4))
    rev = oracle.element_scan(body, init, [x, s], axis=1, state_axis=state_axis, reverse=True)
    fwd = oracle.element_scan(body, init, [np.flip(x, 1), np.flip(s, 1)], axis=1, state_axis=state_axis)
    np.testing.assert_array_equal(rev, np.flip(fwd, 1))


def test_vector_elementwise_body_equals_scalar_lanes():
    # A body without reductions applied to a vector state acts on each component
    # as its own scalar lane, with a width-one sequence broadcast over the vector.
    r = _rng(21)
    x = r.standard_normal((2, 9, 5))
    a = r.uniform(0, 1, (2, 9, 1))
    init = r.standard_normal((2, 5))
    vec = oracle.element_scan("tanh_affine", init, [x, a], axis=1, state_axis=-1)
    sca = oracle.element_scan("tanh_affine", init, [x, np.broadcast_to(a, x.shape)], axis=1)
    np.testing.assert_array_equal(vec, sca)


def test_element_scan_rejects_bad_arguments():
    x = np.ones((2, 3))
    with pytest.raises(ValueError):
        oracle.element_scan("tanh_affine", np.ones(2), [x, x], axis=0)  # initial must be [3]
    with pytest.raises(ValueError):
        oracle.element_scan("tanh_affine", np.ones(2), [x, x], axis=2)
    with pytest.raises(ValueError):
        oracle.element_scan("tanh_affine", np.ones(3), [x, np.ones((2, 4))], axis=0)
    with pytest.raises(ValueError):
        oracle.element_scan("max_plus", np.ones(3), [np.ones((0, 3)), np.ones((0, 3))], axis=0)


# --- matrix-scan ----------------------------------------------------------------------


def _product_sum_forward(a, b):
    # h[t] = sum_{s<=t} (a[t] a[t-1] ... a[s+1]) b[s]: the recurrence unrolled.
    T, n = a.shape[0], a.shape[1]
    out = np.zeros((T,) + b.shape[1:])
    for t in range(T):
        for s in range(t + 1):
            p = np.eye(n)
            for r_ in range(s + 1, t + 1):
                p = a[r_] @ p
            out[t] += p @ b[s]
    return out


def _product_sum_reverse(a, b):
    # h[t] = sum_{s>=t} (a[t] a[t+1] ... a[s-1]) b[s].
    T, n = a.shape[0], a.shape[1]
    out = np.zeros((T,) + b.shape[1:])
    for t in range(T):
        for s in range(t, T):
            p = np.eye(n)
            for r_ in range(s - 1, t - 1, -1):
                p = a[r_] @ p
            out[t] += p @ b[s]
    return out


@pytest.mark.parametrize("n,m,reverse", [(3, 1, False), (4, 2, True), (1, 1, False), (5, 3, True)])
def test_matrix_scan_product_sum(n, m, reverse):
    r = _rng(30 + n)
    T = 6
    a = r.standard_normal((T, n, n))
    b = r.standard_normal((T, n, m))
    out = oracle.matrix_scan(a, b, axis=0, reverse=reverse)
    ref = (_product_sum_reverse if reverse else _product_sum_forward)(a, b)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_matrix_scan_zero_a_is_b():
    r = _rng(31)
    b = r.standard_normal((3, 7, 4, 2))
    out = oracle.matrix_scan(np.zeros((3, 7, 4, 4)), b, axis=1)
    np.testing.assert_array_equal(out, b)


@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_scan_identity_a_is_cumsum(reverse):
    r = _rng(32)
    b = r.standard_normal((2, 9, 3, 2))
    eye = np.broadcast_to(np.eye(3), (2, 9, 3, 3))
    out = oracle.matrix_scan(eye, b, axis=1, reverse=reverse)
    ref = np.flip(np.cumsum(np.flip(b, 1), axis=1), 1) if reverse else np.cumsum(b, axis=1)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_matrix_scan_geometric_series():
    # Time-invariant a and b, given with a time axis of length one that
    # broadcasts: h[t] = (I - a)^{-1} (I - a^{t+1}) b.
    r = _rng(33)
    n, m, T = 4, 2, 12
    a = 0.3 * r.standard_normal((n, n))
    b = r.standard_normal((n, m))
    out = oracle.matrix_scan(a[None], np.broadcast_to(b, (T, n, m)), axis=0)
    eye = np.eye(n)
    for t in range(T):
        ref = np.linalg.solve(eye - a, (eye - np.linalg.matrix_power(a, t + 1)) @ b)
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-12)


def test_matrix_scan_first_a_unused_forward_last_unused_reverse():
    r = _rng(34)
    a = r.standard_normal((8, 3, 3))
    b = r.standard_normal((8, 3, 2))
    a2 = a.copy()
    a2[0] = 1e6
    np.testing.assert_array_equal(oracle.matrix_scan(a, b), oracle.matrix_scan(a2, b))
    a3 = a.copy()
    a3[-1] = 1e6
    np.testing.assert_array_equal(oracle.matrix_scan(a, b, reverse=True), oracle.matrix_scan(a3, b, reverse=True))
    np.testing.assert_array_equal(oracle.matrix_scan(a, b)[0], b[0])


def test_matrix_scan_columns_are_independent():
    # "Tensor operations", matrix-scan: the columns of b never mix; each runs through the same a's alone.
    r = _rng(35)
    a = r.standard_normal((10, 4, 4)) * 0.5
    b = r.standard_normal((10, 4, 3))
    whole = oracle.matrix_scan(a, b)
    for j in range(3):
        # equal up to float64 rounding: BLAS may order the sums differently per shape
        np.testing.assert_allclose(whole[..., j:j + 1], oracle.matrix_scan(a, b[..., j:j + 1]),
                                   rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_scan_inverse_problem(reverse):
    # Choose states h and matrices a; b[t] = h[t] - a[t] @ h_prev reproduces h.
    r = _rng(36)
    B, T, n, m = 3, 8, 5, 2
    a = r.standard_normal((B, T, n, n))
    h = r.standard_normal((B, T, n, m))
    b = np.empty_like(h)
    prev = np.zeros((B, n, m))
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        b[:, t] = h[:, t] - a[:, t] @ prev
        prev = h[:, t]
    out = oracle.matrix_scan(a, b, axis=1, reverse=reverse)
    np.testing.assert_allclose(out, h, rtol=1e-12, atol=1e-12)


def test_matrix_scan_broadcast_leading_dims():
    # a shared across the batch (leading dim 1) is the same as each batch's own scan.
    r = _rng(37)
    a = 0.5 * r.standard_normal((1, 6, 3, 3))
    b = r.standard_normal((4, 6, 3, 2))
    out = oracle.matrix_scan(a, b, axis=-1)
    assert out.shape == b.shape
    for i in range(4):
        np.testing.assert_allclose(out[i], oracle.matrix_scan(a[0], b[i], axis=0), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_scan_reverse_is_flip_scan_flip(reverse):
    r = _rng(38)
    a = r.standard_normal((2, 7, 3, 3))
    b = r.standard_normal((2, 7, 3, 1))
    got = oracle.matrix_scan(a, b, axis=1, reverse=not reverse)
    ref = np.flip(oracle.matrix_scan(np.flip(a, 1), np.flip(b, 1), axis=1, reverse=reverse), 1)
    np.testing.assert_array_equal(got, ref)


def test_matrix_scan_empty_axis_and_limits():
    assert oracle.matrix_scan(np.zeros((0, 2, 2)), np.zeros((0, 2, 1))).shape == (0, 2, 1)
    oracle.matrix_scan(np.zeros((2, 16, 16)), np.zeros((2, 16, 1)))
    with pytest.raises(ValueError):
        oracle.matrix_scan(np.zeros((2, 17, 17)), np.zeros((2, 17, 1)))
    with pytest.raises(ValueError):
        oracle.matrix_scan(np.zeros((2, 3, 3)), np.zeros((2, 4, 1)))


def test_matrix_scan_scalar_closed_form():
    # n = m = 1 is the prelude's linear-scan: h[t] = sum_s (prod_{s<r<=t} a[r]) b[s].
    r = _rng(39)
    T = 9
    a = r.uniform(-1.5, 1.5, T)
    b = r.standard_normal(T)
    out = oracle.matrix_scan(a.reshape(T, 1, 1), b.reshape(T, 1, 1))[:, 0, 0]
    ref = [sum(math.prod(a[s + 1: t + 1]) * b[s] for s in range(t + 1)) for t in range(T)]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# --- linear-scan and cumsum ----------------------------------------------------
# "Tensor operations", the "matrix-scan" section: linear-scan is the matrix
# recurrence over one-by-one matrices, operands broadcast to one shape; cumsum
# is built on it (a = 1).


@pytest.mark.parametrize("axis,reverse", [(0, False), (1, False), (1, True), (-1, True)])
def test_linear_scan_unit_a_is_cumsum(axis, reverse):
    x = _rng(60).standard_normal((4, 7, 5))
    ref = np.flip(np.cumsum(np.flip(x, axis), axis=axis), axis) if reverse else np.cumsum(x, axis=axis)
    np.testing.assert_allclose(oracle.cumsum(x, axis=axis, reverse=reverse), ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.linear_scan(1.0, x, axis=axis, reverse=reverse), ref, rtol=1e-13, atol=1e-13)


def test_linear_scan_zero_a_is_b():
    b = _rng(61).standard_normal((3, 9, 2))
    np.testing.assert_array_equal(oracle.linear_scan(np.zeros((3, 9, 2)), b, axis=1), b)
    np.testing.assert_array_equal(oracle.linear_scan(0.0, b, axis=1, reverse=True), b)


@pytest.mark.parametrize("reverse", [False, True])
def test_linear_scan_product_sum(reverse):
    # Closed form: h[t] = sum over s up to t of (a[s+1] ... a[t]) b[s]
    # (reverse: s from t up, with the product a[t] ... a[s-1]).
    r = _rng(62)
    T = 7
    a = r.uniform(-1.5, 1.5, (T, 3))
    b = r.standard_normal((T, 3))
    out = oracle.linear_scan(a, b, axis=0, reverse=reverse)
    ref = np.zeros((T, 3))
    for t in range(T):
        srcs = range(t, T) if reverse else range(t + 1)
        for s in srcs:
            between = range(t, s) if reverse else range(s + 1, t + 1)
            coeff = np.ones(3)
            for q in between:
                coeff = coeff * a[q]
            ref[t] += coeff * b[s]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_linear_scan_geometric_series():
    # constant a and b: h[t] = b (1 - a^(t+1)) / (1 - a)
    a, b, T = 0.7, 1.3, 20
    out = oracle.linear_scan(a, np.full(T, b), axis=0)
    t = np.arange(T)
    np.testing.assert_allclose(out, b * (1 - a ** (t + 1)) / (1 - a), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("reverse", [False, True])
def test_linear_scan_inverse_problem(reverse):
    # pick the states, solve each step for its b, scan, get the states back
    r = _rng(63)
    T = 11
    h = r.standard_normal((2, T, 3))
    a = r.uniform(-2, 2, (2, T, 3))
    prev = np.zeros_like(h)
    if reverse:
        prev[:, :-1] = h[:, 1:]
    else:
        prev[:, 1:] = h[:, :-1]
    b = h - a * prev
    np.testing.assert_allclose(oracle.linear_scan(a, b, axis=1, reverse=reverse), h, rtol=1e-12, atol=1e-12)


def test_linear_scan_broadcast_operands():
    r = _rng(64)
    a_row = r.uniform(0.5, 1.0, (1, 6, 1))       # one gate per step, shared by every lane
    b = r.standard_normal((4, 6, 3))
    ref = oracle.linear_scan(np.broadcast_to(a_row, b.shape).copy(), b, axis=1)
    np.testing.assert_array_equal(oracle.linear_scan(a_row, b, axis=1), ref)
    # a number and an array: the result takes the array's shape
    assert oracle.linear_scan(0.5, b, axis=-2).shape == b.shape


def test_linear_scan_first_a_unused_forward_last_unused_reverse():
    r = _rng(65)
    a = r.standard_normal((9, 2))
    b = r.standard_normal((9, 2))
    a2 = a.copy()
    a2[0] = 1e6
    np.testing.assert_array_equal(oracle.linear_scan(a, b), oracle.linear_scan(a2, b))
    a3 = a.copy()
    a3[-1] = 1e6
    np.testing.assert_array_equal(oracle.linear_scan(a, b, reverse=True), oracle.linear_scan(a3, b, reverse=True))


def test_linear_scan_empty_axis_and_numbers():
    out = oracle.linear_scan(np.ones((3, 0, 2)), np.ones((3, 0, 2)), axis=1)
    assert out.shape == (3, 0, 2)
    with pytest.raises(ValueError):
        oracle.linear_scan(1.0, 2.0)  # two numbers: no axis to scan
    with pytest.raises(ValueError):
        oracle.linear_scan(np.ones(4), np.ones(4), axis=1)


# ---------------------------------------------------------------- matrix-scan gradient
#
# "Tensor operations", the "matrix-scan" section: the gradient is a scan in
# the opposite direction over transposed a; the "gradient" section: a gradient
# has its operand's shape. The pins below fix the vector-Jacobian product by
# what it is, the derivative of L = sum(g * h), without reusing its loop.


def _loss(a, b, g, axis, reverse):
    return float(np.sum(g * oracle.matrix_scan(a, b, axis=axis, reverse=reverse)))


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("axis", [0, 1, -1])
def test_matrix_scan_vjp_exact_by_unit_perturbations(axis, reverse):
    # h is linear in b, and affine in each single entry of a (a step's matrix
    # enters every product at most once), so a unit change of one entry moves
    # L by exactly that entry's derivative: a brute-force Jacobian row each.
    rng = _rng(71)
    lead = (2, 4)
    a = 0.6 * rng.normal(size=lead + (3, 3))
    b = rng.normal(size=lead + (3, 2))
    g = rng.normal(size=lead + (3, 2))
    ga, gb = oracle.matrix_scan_vjp(a, b, g, axis=axis, reverse=reverse)
    assert ga.shape == a.shape and gb.shape == b.shape
    base = _loss(a, b, g, axis, reverse)
    for idx in np.ndindex(*b.shape):
        db = np.zeros_like(b)
        db[idx] = 1.0
        assert abs((_loss(a, b + db, g, axis, reverse) - base) - gb[idx]) < 1e-12 * (1 + abs(base))
    for idx in np.ndindex(*a.shape):
        da = np.zeros_like(a)
        da[idx] = 1.0
        assert abs((_loss(a + da, b, g, axis, reverse) - base) - ga[idx]) < 1e-11 * (1 + abs(base))


@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_scan_vjp_directional_derivative_with_broadcasting(reverse):
    # a constant in time, b shared by the batch: central differences of L
    # along random directions in the operands' own shapes
    rng = _rng(72)
    a = 0.3 * rng.normal(size=(3, 1, 4, 4)) + 0.5 * np.eye(4)   # broadcast over time 6 (axis 1)
    b = rng.normal(size=(6, 4, 2))                              # broadcast over batch 3
    g = rng.normal(size=(3, 6, 4, 2))
    ga, gb = oracle.matrix_scan_vjp(a, b, g, axis=1, reverse=reverse)
    assert ga.shape == a.shape and gb.shape == b.shape
    for _ in range(3):
        da, db = rng.normal(size=a.shape), rng.normal(size=b.shape)
        eps = 1e-5
        fd = (_loss(a + eps * da, b + eps * db, g, 1, reverse) - _loss(a - eps * da, b - eps * db, g, 1, reverse)) / (2 * eps)
        an = float(np.sum(ga * da) + np.sum(gb * db))
        assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (fd, an)


@pytest.mark.parametrize("reverse", [False, True])
def test_matrix_scan_vjp_grad_b_is_the_transposed_scan_run_backwards(reverse):
    # the page's statement, built explicitly: a'[t] = transpose of the a of the
    # step after t in the forward order, scanned in the other direction over g
    rng = _rng(73)
    T = 7
    a = 0.5 * rng.normal(size=(2, T, 5, 5))
    b = rng.normal(size=(2, T, 5, 3))
    g = rng.normal(size=(2, T, 5, 3))
    _, gb = oracle.matrix_scan_vjp(a, b, g, axis=1, reverse=reverse)
    at = np.swapaxes(a, -1, -2)
    shifted = np.zeros_like(at)
    if reverse:   # forward order is T-1 .. 0: the step after t is t-1
        shifted[:, 1:] = at[:, :-1]
    else:         # the step after t is t+1
        shifted[:, :-1] = at[:, 1:]
    want = oracle.matrix_scan(shifted, g, axis=1, reverse=not reverse)
    np.testing.assert_allclose(gb, want, rtol=1e-12, atol=1e-12)


def test_matrix_scan_vjp_first_step_a_has_zero_gradient():
    # a at the first step multiplies h = 0, in either direction
    rng = _rng(74)
    a = rng.normal(size=(3, 5, 4, 4))
    b = rng.normal(size=(3, 5, 4, 1))
    g = rng.normal(size=(3, 5, 4, 1))
    ga, _ = oracle.matrix_scan_vjp(a, b, g, axis=1)
    assert np.all(ga[:, 0] == 0) and np.any(ga[:, 1] != 0)
    ga, _ = oracle.matrix_scan_vjp(a, b, g, axis=1, reverse=True)
    assert np.all(ga[:, -1] == 0) and np.any(ga[:, -2] != 0)


def test_matrix_scan_vjp_scalar_closed_form():
    # n = m = 1, T = 3 forward: h0 = b0, h1 = a1 b0 + b1, h2 = a2 a1 b0 + a2 b1 + b2
    a = np.array([[[0.0]], [[2.0]], [[3.0]]])
    b = np.array([[[1.0]], [[5.0]], [[7.0]]])
    g = np.array([[[1.0]], [[10.0]], [[100.0]]])
    ga, gb = oracle.matrix_scan_vjp(a, b, g, axis=0)
    # dL/db0 = g0 + a1 g1 + a2 a1 g2 = 1 + 20 + 600; dL/db1 = g1 + a2 g2 = 310; dL/db2 = 100
    assert gb[:, 0, 0].tolist() == [621.0, 310.0, 100.0]
    # dL/da1 = (g1 + a2 g2) h0 = 310; dL/da2 = g2 h1 = 100 * 7
    assert ga[:, 0, 0].tolist() == [0.0, 310.0, 700.0]


# ---------------------------------------------------------------- element-scan gradients
#
# The vector-Jacobian product of sum(g * element_scan(...)) fixed by what it is,
# the derivative, without reusing the gradient loop: central differences of
# the pinned forward oracle, exact one-sided differences where the scan is
# piecewise linear (max-plus), and closed forms of special cases.

def _es_case(body, state, rng, shape=(3, 7, 4)):
    B, T, n = shape
    if state is None:
        x = rng.normal(size=shape)
        s = rng.uniform(0.0, 0.5, size=shape) if body == "max_plus" else rng.uniform(0.2, 1.0, size=shape)
        init = rng.normal(size=(B, n))
    else:
        x = 2.0 * rng.normal(size=(B, T, n))
        s = rng.uniform(0.5, 1.0, size=(B, T, state))
        init = 0.3 * rng.normal(size=(B, n))
    g = rng.normal(size=(B, T, n))
    return init, x, s, g


def _es_loss(body, init, x, s, g, state, reverse):
    st = None if state is None else -1
    return float(np.sum(g * oracle.element_scan(body, init, [x, s], axis=1, state_axis=st, reverse=reverse)))


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("body,state", [("tanh_affine", None), ("tanh_affine", 1), ("tanh_affine", 4),
                                        ("norm_cap", 1), ("norm_cap", 4), ("max_plus", None), ("max_plus", 1)])
def test_element_scan_vjp_central_differences(body, state, reverse):
    rng = _rng(81)
    init, x, s, g = _es_case(body, state, rng)
    st = None if state is None else -1
    gi, (gx, gs) = oracle.element_scan_vjp(body, init, [x, s], g, axis=1, state_axis=st, reverse=reverse)
    assert gi.shape == init.shape and gx.shape == x.shape and gs.shape == s.shape
    for _ in range(3):
        di, dx, ds = rng.normal(size=init.shape), rng.normal(size=x.shape), rng.normal(size=s.shape)
        eps = 1e-6
        fd = (_es_loss(body, init + eps * di, x + eps * dx, s + eps * ds, g, state, reverse)
              - _es_loss(body, init - eps * di, x - eps * dx, s - eps * ds, g, state, reverse)) / (2 * eps)
        an = float(np.sum(gi * di) + np.sum(gx * dx) + np.sum(gs * ds))
        assert abs(fd - an) <= 1e-6 * (1 + abs(an)), (fd, an)


@pytest.mark.parametrize("reverse", [False, True])
def test_max_plus_vjp_exact_by_unit_perturbations(reverse):
    # max-plus is piecewise linear: a perturbation small enough to change no
    # branch moves the loss by exactly the derivative times its size
    rng = _rng(82)
    init, x, c, g = _es_case("max_plus", None, rng, shape=(2, 6, 3))
    gi, (gx, gc) = oracle.element_scan_vjp("max_plus", init, [x, c], g, axis=1, reverse=reverse)
    base = _es_loss("max_plus", init, x, c, g, None, reverse)
    d = 2.0 ** -20
    for arr, grad, which in ((init, gi, 0), (x, gx, 1), (c, gc, 2)):
        for idx in np.ndindex(*arr.shape):
            pert = [init, x, c]
            moved = arr.copy()
            moved[idx] += d
            pert[which] = moved
            got = (_es_loss("max_plus", pert[0], pert[1], pert[2], g, None, reverse) - base) / d
            assert abs(got - grad[idx]) < 1e-6 * (1 + abs(grad[idx])), (which, idx, got, grad[idx])


def test_tanh_affine_vjp_single_trip_and_zero_decay():
    # one trip: h = tanh(x + a h0), so dL/dx = g (1 - h^2), dL/da = g (1 - h^2) h0, dL/dh0 = g (1 - h^2) a
    x, a, h0, g = np.array([[0.3]]), np.array([[0.7]]), np.array([-0.4]), np.array([[2.0]])
    gi, (gx, ga) = oracle.element_scan_vjp("tanh_affine", h0, [x, a], g, axis=0)
    d = 2.0 * (1 - np.tanh(0.3 + 0.7 * -0.4) ** 2)
    assert np.isclose(gx[0, 0], d) and np.isclose(ga[0, 0], d * -0.4) and np.isclose(gi[0], d * 0.7)
    # decay 0: each trip is tanh(x) alone, so grad_x = g (1 - tanh(x)^2) and nothing reaches initial
    rng = _rng(83)
    x = rng.normal(size=(4, 9))
    g = rng.normal(size=(4, 9))
    gi, (gx, ga) = oracle.element_scan_vjp("tanh_affine", rng.normal(size=4), [x, np.zeros_like(x)], g, axis=1)
    np.testing.assert_allclose(gx, g * (1 - np.tanh(x) ** 2), rtol=1e-14)
    assert np.all(gi == 0)


def test_norm_cap_vjp_uncapped_is_the_linear_scan_gradient():
    # when the cap never acts the body is y = a h + x, a gated linear scan: its
    # adjoint is the reverse linear scan of g with the next trip's gate
    rng = _rng(84)
    B, T, n = 2, 8, 5
    x = 0.01 * rng.normal(size=(B, T, n))
    a = rng.uniform(0.2, 0.6, size=(B, T, 1))
    init = 0.01 * rng.normal(size=(B, n))
    g = rng.normal(size=(B, T, n))
    h = oracle.element_scan("norm_cap", init, [x, a], axis=1, state_axis=-1)
    assert np.max(np.linalg.norm(h, axis=-1)) < 0.5
    gi, (gx, ga) = oracle.element_scan_vjp("norm_cap", init, [x, a], g, axis=1, state_axis=-1)
    shifted = np.ones((B, T, 1))
    shifted[:, :-1] = a[:, 1:]
    lam = oracle.linear_scan(np.broadcast_to(shifted, (B, T, n)), g, axis=1, reverse=True)
    np.testing.assert_allclose(gx, lam, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gi, a[:, 0] * lam[:, 0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- matrix-scan :projective
#
# "Tensor operations", the "matrix-scan" section (:projective): every step
# rescales both the accumulated product of the a's (from the identity) and the
# state by that product's largest entry in absolute value. Pinned below: when b
# vanishes after its first step, each state must be the plain scan's state
# scaled by a positive number.


@pytest.mark.parametrize("reverse", [False, True])
def test_projective_with_b_after_first_step_zero_is_h_over_the_product_size(reverse):
    # b zero after its first step: h[t] = (a[t] ... a[first+1] b[first]) / max|a[t] ... a[first]|, the
    # true state divided by the largest entry of the true running product (written with explicit products)
    rng = _rng(91)
    T, n = 9, 4
    a = 0.9 * rng.normal(size=(2, T, n, n))
    b = np.zeros((2, T, n, 2))
    first = T - 1 if reverse else 0
    b[:, first] = rng.normal(size=(2, n, 2))
    got = oracle.matrix_scan_projective(a, b, axis=1, reverse=reverse)
    order = list(range(T - 1, -1, -1)) if reverse else list(range(T))
    for bi in range(2):
        prod = np.eye(n)
        state = b[bi, first]
        for i, t in enumerate(order):
            prod = a[bi, t] @ prod
            if i > 0:
                state = a[bi, t] @ state
            np.testing.assert_allclose(got[bi, t], state / np.max(np.abs(prod)), rtol=1e-12, atol=1e-14)


def test_projective_result_is_h_up_to_a_positive_factor():
    # the page's statement itself: with b zero after its first step, out[t] = c_t * matrix_scan(...)[t], c_t > 0
    rng = _rng(92)
    a = rng.normal(size=(3, 12, 5, 5))
    b = np.zeros((3, 12, 5, 1))
    b[:, 0] = rng.normal(size=(3, 5, 1))
    got = oracle.matrix_scan_projective(a, b, axis=1)
    true = oracle.matrix_scan(a, b, axis=1)
    ratio = np.sum(got * true, axis=(-2, -1)) / np.sum(true * true, axis=(-2, -1))
    assert np.all(ratio > 0)
    np.testing.assert_allclose(got, ratio[..., None, None] * true, rtol=1e-10, atol=1e-300)


@pytest.mark.parametrize("c", [0.5, 2.0, 3.0])
def test_projective_scalar_multiple_of_identity_is_a_scaled_running_sum(c):
    # a[t] = c I: the product after each step is c^k I with largest entry c^k, so every step divides by c:
    # h[t] = h[t-1] + b[t] / c from h[0] = b[0] / c, i.e. cumsum(b) / c -- for any length, where the plain
    # scan would overflow (c = 2 or 3 over 1500 steps is far beyond float64's range)
    rng = _rng(93)
    T, n = 1500, 3
    a = np.broadcast_to(c * np.eye(n), (T, n, n))
    b = rng.normal(size=(T, n, 2))
    got = oracle.matrix_scan_projective(a, b, axis=0)
    np.testing.assert_allclose(got, np.cumsum(b, axis=0) / c, rtol=1e-12, atol=1e-12)


def test_projective_identity_a_is_plain_cumsum_and_reverse_is_flip_scan_flip():
    rng = _rng(94)
    b = rng.normal(size=(2, 30, 4, 3))
    eye = np.broadcast_to(np.eye(4), (2, 30, 4, 4))
    np.testing.assert_allclose(oracle.matrix_scan_projective(eye, b, axis=1), np.cumsum(b, axis=1), rtol=1e-13)
    a = 0.7 * rng.normal(size=(2, 30, 4, 4))
    fwd = oracle.matrix_scan_projective(np.flip(a, 1), np.flip(b, 1), axis=1)
    np.testing.assert_allclose(oracle.matrix_scan_projective(a, b, axis=1, reverse=True), np.flip(fwd, 1),
                               rtol=1e-13, atol=1e-15)


def test_projective_zero_product_divides_by_one():
    a = np.zeros((4, 2, 2))
    b = np.arange(16, dtype=float).reshape(4, 2, 2)
    np.testing.assert_array_equal(oracle.matrix_scan_projective(a, b, axis=0), b)


# ---------------------------------------------------------------- table-scan
#
# "Tensor operations", the "table-scan" section: state = table[previous, symbol]
# along one axis from :start; the page's example is the parity automaton.


def test_table_scan_parity_example_is_running_xor():
    # the page's example: flip = [[0 1] [1 0]] over bits gives the parity so far
    rng = _rng(101)
    bits = rng.integers(0, 2, size=(5, 200)).astype(np.int32)
    got = oracle.table_scan(np.array([[0, 1], [1, 0]], dtype=np.int32), bits)
    np.testing.assert_array_equal(got, np.cumsum(bits, axis=-1) % 2)
    assert got.dtype == np.int32 and got.shape == bits.shape


@pytest.mark.parametrize("k", [3, 7, 16])
def test_table_scan_counter_mod_k_is_cumsum_mod_k(k):
    # table[s, x] = (s + x) mod k from start s0: the states are (s0 + running sum) mod k, along any axis
    rng = _rng(102)
    table = (np.arange(k)[:, None] + np.arange(k)[None, :]) % k
    sym = rng.integers(0, k, size=(4, 30, 6)).astype(np.int32)
    for axis in (0, 1, -1):
        got = oracle.table_scan(table.astype(np.int32), sym, axis=axis, start=2)
        np.testing.assert_array_equal(got, (2 + np.cumsum(sym, axis=axis)) % k)


def test_table_scan_identity_reset_and_composition():
    rng = _rng(103)
    sym = rng.integers(0, 5, size=(3, 40)).astype(np.int32)
    stay = np.repeat(np.arange(4)[:, None], 5, axis=1).astype(np.int32)   # table[s, x] = s
    np.testing.assert_array_equal(oracle.table_scan(stay, sym, start=3), np.full(sym.shape, 3))
    reset = np.repeat((np.arange(5) % 4)[None, :], 4, axis=0).astype(np.int32)  # table[s, x] = x mod 4
    np.testing.assert_array_equal(oracle.table_scan(reset, sym), sym % 4)
    # running the second half from the last state of the first half continues the run
    table = rng.integers(0, 6, size=(6, 5)).astype(np.int32)
    whole = oracle.table_scan(table, sym)
    first = oracle.table_scan(table, sym[:, :17])
    for row in range(3):
        rest = oracle.table_scan(table, sym[row:row + 1, 17:], start=int(first[row, -1]))
        np.testing.assert_array_equal(whole[row:row + 1, 17:], rest)


def test_table_scan_small_hand_run():
    # a 3-state automaton traced by hand: table rows are states, columns symbols
    table = np.array([[1, 2], [0, 0], [2, 1]], dtype=np.int32)
    sym = np.array([0, 1, 1, 0, 1], dtype=np.int32)
    # from 0: t[0,0]=1, t[1,1]=0, t[0,1]=2, t[2,0]=2, t[2,1]=1
    np.testing.assert_array_equal(oracle.table_scan(table, sym), [1, 0, 2, 2, 1])
    # a square table that is not symmetric: rows (the state) and columns (the symbol) cannot be swapped
    table = np.array([[1, 0, 0], [2, 2, 0], [1, 1, 1]], dtype=np.int32)
    # from 0: t[0,1]=0, t[0,0]=1, t[1,2]=0, t[0,1]=0
    np.testing.assert_array_equal(oracle.table_scan(table, np.array([1, 0, 2, 1], dtype=np.int32)), [0, 1, 0, 0])


def test_table_scan_out_of_range_clamped_or_refused():
    table = np.array([[1, 5], [0, -2]], dtype=np.int32)   # entries 5 and -2 are not states
    sym = np.array([[0, 7, -1, 1, 1]], dtype=np.int32)
    # clamped (GPU reading): symbols 7 -> 1, -1 -> 0; reached entries 5 -> 1, -2 -> 0
    # from 0: t[0,0]=1; t[1,clamp 7=1]=-2 -> 0; t[0,clamp -1=0]=1; t[1,1]=-2 -> 0; t[0,1]=5 -> 1
    np.testing.assert_array_equal(oracle.table_scan(table, sym), [[1, 0, 1, 0, 1]])
    with pytest.raises(ValueError):
        oracle.table_scan(table, sym, clamp=False)
    with pytest.raises(ValueError):
        oracle.table_scan(table, np.array([0, 1]), clamp=False)  # reaches 5 at the second symbol
    for bad in (dict(start=2), dict(axis=1)):
        with pytest.raises(ValueError):
            oracle.table_scan(table, np.array([0, 1]), **bad)
    with pytest.raises(ValueError):
        oracle.table_scan(np.zeros((2, 0), dtype=np.int32), np.array([0]))
