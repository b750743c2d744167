"""The pins must fail on plausible mistakes: each case plants one in the oracle.

A mutation replaces one oracle function for the duration of a test (on the
CPU, through pytest's monkeypatch) and then runs the pins written for that
operation. At least one pin has to fail, otherwise the pins would not have
told a correct oracle from a wrong one.
"""

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

_real_es = oracle.element_scan
_real_ms = oracle.matrix_scan
_real_bodies = dict(oracle.BODIES)


def _time_shifted(body, initial, sequences, axis=0, state_axis=None, reverse=False, dtype=np.float64):
    # reads x one trip late: x[t-1] at trip t
    seqs = [np.asarray(s, dtype=np.float64) for s in sequences]
    ax = axis % seqs[0].ndim
    seqs[0] = np.roll(seqs[0], 1, axis=ax)
    return _real_es(body, initial, seqs, axis, state_axis, reverse, dtype)


def _gate_shifted(body, initial, sequences, axis=0, state_axis=None, reverse=False, dtype=np.float64):
    # reads the second sequence (decay or cost) one trip early
    seqs = [np.asarray(s, dtype=np.float64) for s in sequences]
    ax = axis % seqs[0].ndim
    seqs[1] = np.roll(seqs[1], -1, axis=ax)
    return _real_es(body, initial, seqs, axis, state_axis, reverse, dtype)


def _wrong_direction(body, initial, sequences, axis=0, state_axis=None, reverse=False, dtype=np.float64):
    return _real_es(body, initial, sequences, axis, state_axis, not reverse, dtype)


ES_MUTANTS = {
    "tanh drops decay": ("tanh_affine", lambda h, x, a: np.tanh(x + h)),
    "tanh swaps x and a": ("tanh_affine", lambda h, x, a: np.tanh(a + x * h)),
    "tanh drops tanh": ("tanh_affine", lambda h, x, a: x + a * h),
    "norm-cap drops sqrt": ("norm_cap", lambda h, x, a: (lambda y: y / np.maximum(1.0, np.sum(y * y, -1, keepdims=True)))(a * h + x)),
    "norm-cap caps each component": ("norm_cap", lambda h, x, a: (lambda y: y / np.maximum(1.0, np.abs(y)))(a * h + x)),
    "norm-cap drops x": ("norm_cap", lambda h, x, a: (lambda y: y / np.maximum(1.0, np.sqrt(np.sum(y * y, -1, keepdims=True))))(a * h)),
    "max-plus adds cost": ("max_plus", lambda h, x, c: np.maximum(h + c, x)),
    "max-plus takes min": ("max_plus", lambda h, x, c: np.minimum(h - c, x)),
    "max-plus subtracts after max": ("max_plus", lambda h, x, c: np.maximum(h, x) - c),
}

ES_PINS = {
    "tanh_affine": [
        (pins.test_golden_tanh_affine, {}),
        (pins.test_tanh_zero_decay_is_pointwise_tanh, {"axis": 1}),
        (pins.test_tanh_inverse_problem, {"axis": 1, "reverse": False}),
        (pins.test_tanh_inverse_problem, {"axis": 1, "reverse": True}),
    ],
    "norm_cap": [
        (pins.test_golden_norm_cap, {}),
        (pins.test_norm_cap_inverse_problem, {"n": 16, "gate_width": 1, "reverse": False}),
        (pins.test_norm_cap_linear_regime_closed_form, {}),
        (pins.test_norm_cap_saturated_is_unit_norm, {}),
    ],
    "max_plus": [
        (pins.test_golden_max_plus, {"key": "max_plus_reverse", "reverse": True}),
        (pins.test_max_plus_closed_form, {"reverse": True}),
        (pins.test_max_plus_zero_cost_is_reverse_cummax, {}),
    ],
}


def _some_pin_fails(pin_list):
    for fn, kwargs in pin_list:
        try:
            fn(**kwargs)
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(ES_MUTANTS))
def test_element_scan_body_mutants_are_caught(name, monkeypatch):
    body, fn = ES_MUTANTS[name]
    monkeypatch.setitem(oracle.BODIES, body, fn)
    assert _some_pin_fails(ES_PINS[body]), f"no pin caught mutant: {name}"


@pytest.mark.parametrize("mutant", [_time_shifted, _gate_shifted, _wrong_direction])
@pytest.mark.parametrize("body", sorted(ES_PINS))
def test_element_scan_index_mutants_are_caught(mutant, body, monkeypatch):
    monkeypatch.setattr(oracle, "element_scan", mutant)
    assert _some_pin_fails(ES_PINS[body]), f"no {body} pin caught {mutant.__name__}"


def _ms_transposed(a, b, axis=0, reverse=False, dtype=np.float64):
    return _real_ms(np.swapaxes(np.asarray(a, dtype=np.float64), -1, -2), b, axis, reverse, dtype)


def _ms_a_shifted(a, b, axis=0, reverse=False, dtype=np.float64):
    # uses a[t-1] at step t
    a = np.asarray(a, dtype=np.float64)
    lead = len(np.broadcast_shapes(a.shape[:-2], np.shape(b)[:-2]))
    ax = axis % lead
    a_b = np.broadcast_to(a, np.broadcast_shapes(a.shape[:-2], np.shape(b)[:-2]) + a.shape[-2:])
    return _real_ms(np.roll(a_b, 1, axis=ax), b, axis, reverse, dtype)


def _ms_wrong_direction(a, b, axis=0, reverse=False, dtype=np.float64):
    return _real_ms(a, b, axis, not reverse, dtype)


def _ms_starts_from_b0_twice(a, b, axis=0, reverse=False, dtype=np.float64):
    # starts from h = b[first] instead of h = 0, counting the first b twice
    out = _real_ms(a, b, axis, reverse, dtype)
    return out + np.take(np.asarray(b, dtype=np.float64), [-1 if reverse else 0], axis=axis % (np.ndim(b) - 2))


MS_PINS = [
    (pins.test_golden_matrix_scan, {"key": "matrix_scan_forward", "reverse": False}),
    (pins.test_golden_matrix_scan, {"key": "matrix_scan_reverse", "reverse": True}),
    (pins.test_matrix_scan_product_sum, {"n": 4, "m": 2, "reverse": True}),
    (pins.test_matrix_scan_product_sum, {"n": 3, "m": 1, "reverse": False}),
    (pins.test_matrix_scan_inverse_problem, {"reverse": False}),
]


@pytest.mark.parametrize("mutant", [_ms_transposed, _ms_a_shifted, _ms_wrong_direction, _ms_starts_from_b0_twice])
def test_matrix_scan_mutants_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "matrix_scan", mutant)
    assert _some_pin_fails(MS_PINS), f"no matrix-scan pin caught {mutant.__name__}"


def test_unmutated_oracle_passes_the_same_pins():
    for body in ES_PINS:
        assert not _some_pin_fails(ES_PINS[body])
    assert not _some_pin_fails(MS_PINS)


_real_ls = oracle.linear_scan


def _ls_a_shifted(a, b, axis=0, reverse=False, dtype=np.float64):
    # uses a[t-1] at step t
    shape = np.broadcast_shapes(np.shape(a), np.shape(b))
    a_b = np.broadcast_to(np.asarray(a, dtype=np.float64), shape)
    return _real_ls(np.roll(a_b, 1, axis=axis % len(shape)), b, axis, reverse, dtype)


def _ls_swapped(a, b, axis=0, reverse=False, dtype=np.float64):
    return _real_ls(b, a, axis, reverse, dtype)


def _ls_wrong_direction(a, b, axis=0, reverse=False, dtype=np.float64):
    return _real_ls(a, b, axis, not reverse, dtype)


def _ls_starts_from_b0_twice(a, b, axis=0, reverse=False, dtype=np.float64):
    out = _real_ls(a, b, axis, reverse, dtype)
    shape = np.broadcast_shapes(np.shape(a), np.shape(b))
    b_b = np.broadcast_to(np.asarray(b, dtype=np.float64), shape)
    return out + np.take(b_b, [-1 if reverse else 0], axis=axis % len(shape))


def _ls_adds_a(a, b, axis=0, reverse=False, dtype=np.float64):
    # h + a instead of a * h: the number broadcast still shapes the result
    shape = np.broadcast_shapes(np.shape(a), np.shape(b))
    a_b = np.moveaxis(np.broadcast_to(np.asarray(a, dtype=np.float64), shape), axis % len(shape), 0)
    b_b = np.moveaxis(np.broadcast_to(np.asarray(b, dtype=np.float64), shape), axis % len(shape), 0)
    h = np.zeros(a_b.shape[1:])
    out = np.empty_like(b_b)
    for t in (range(len(b_b) - 1, -1, -1) if reverse else range(len(b_b))):
        h = a_b[t] + h + b_b[t]
        out[t] = h
    return np.moveaxis(out, 0, axis % len(shape))


LS_PINS = [
    (pins.test_linear_scan_product_sum, {"reverse": False}),
    (pins.test_linear_scan_product_sum, {"reverse": True}),
    (pins.test_linear_scan_inverse_problem, {"reverse": False}),
    (pins.test_linear_scan_inverse_problem, {"reverse": True}),
    (pins.test_linear_scan_geometric_series, {}),
]


@pytest.mark.parametrize("mutant", [_ls_a_shifted, _ls_swapped, _ls_wrong_direction, _ls_starts_from_b0_twice, _ls_adds_a])
def test_linear_scan_mutants_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "linear_scan", mutant)
    assert _some_pin_fails(LS_PINS), f"no linear-scan pin caught {mutant.__name__}"


def test_unmutated_linear_scan_passes_its_pins():
    assert not _some_pin_fails(LS_PINS)


_real_vjp = oracle.matrix_scan_vjp


def _vjp_mutant(kind):
    """A copy of the gradient loop with one plausible mistake planted."""
    def vjp(a, b, g, axis=0, reverse=False, dtype=np.float64):
        a = np.asarray(a, dtype=dtype)
        b = np.asarray(b, dtype=dtype)
        g = np.asarray(g, dtype=dtype)
        h = oracle.matrix_scan(a, b, axis=axis, reverse=reverse, dtype=dtype)
        n = a.shape[-1]
        lead = h.shape[:-2]
        ax = axis % len(lead)
        a_t = np.moveaxis(np.broadcast_to(a, lead + (n, n)), ax, 0)
        g_t, h_t = np.moveaxis(g, ax, 0), np.moveaxis(h, ax, 0)
        T = lead[ax]
        lam = np.empty(g_t.shape)
        grad_a = np.zeros(a_t.shape)
        order = list(range(T - 1, -1, -1)) if reverse else list(range(T))
        if kind == "wrong_direction":
            order = order[::-1]
        from_later = np.zeros(g_t.shape[1:])
        for i in range(T - 1, -1, -1):
            t = order[i]
            lam[t] = g_t[t] + from_later if kind != "drops_g" or i == T - 1 else from_later
            if i > 0:
                p = order[i - 1]
                hp = h_t[t] if kind == "uses_h_t" else h_t[p]
                grad_a[t] = (hp @ np.swapaxes(lam[t], -1, -2) if kind == "outer_transposed"
                             else lam[t] @ np.swapaxes(hp, -1, -2))
            at = a_t[t] if kind == "no_transpose" else np.swapaxes(a_t[t], -1, -2)
            if kind == "same_step_a" and i > 0:
                at = np.swapaxes(a_t[order[i - 1]], -1, -2)
            from_later = at @ lam[t]
        grad_a = oracle._sum_to_shape(np.moveaxis(grad_a, 0, ax), a.shape)
        grad_b = oracle._sum_to_shape(np.moveaxis(lam, 0, ax), b.shape)
        return grad_a, grad_b
    vjp.__name__ = f"vjp_{kind}"
    return vjp


VJP_PINS = [
    (pins.test_matrix_scan_vjp_exact_by_unit_perturbations, {"axis": 1, "reverse": False}),
    (pins.test_matrix_scan_vjp_exact_by_unit_perturbations, {"axis": 0, "reverse": True}),
    (pins.test_matrix_scan_vjp_grad_b_is_the_transposed_scan_run_backwards, {"reverse": False}),
    (pins.test_matrix_scan_vjp_scalar_closed_form, {}),
]


@pytest.mark.parametrize("kind", ["no_transpose", "same_step_a", "uses_h_t", "outer_transposed", "drops_g",
                                  "wrong_direction"])
def test_matrix_scan_vjp_mutants_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "matrix_scan_vjp", _vjp_mutant(kind))
    assert _some_pin_fails(VJP_PINS), f"no gradient pin caught {kind}"


def test_unmutated_vjp_passes_its_pins():
    assert not _some_pin_fails(VJP_PINS)
    # the planted-mistake copy without a mistake is the oracle
    rng = np.random.default_rng(5)
    a, b, g = rng.normal(size=(2, 5, 3, 3)), rng.normal(size=(2, 5, 3, 2)), rng.normal(size=(2, 5, 3, 2))
    for x, y in zip(_vjp_mutant("none")(a, b, g, axis=1), _real_vjp(a, b, g, axis=1)):
        np.testing.assert_array_equal(x, y)


def _tanh_no_slope(h_prev, x, a, h, lam, branch):
    return a * lam, lam, lam * h_prev


def _tanh_slope_of_input(h_prev, x, a, h, lam, branch):
    dz = lam * (1.0 - h_prev * h_prev)
    return a * dz, dz, dz * h_prev


def _tanh_swapped(h_prev, x, a, h, lam, branch):
    dz = lam * (1.0 - h * h)
    return a * dz, dz * h_prev, dz


def _norm_cap_no_projection(h_prev, x, a, h, lam, capped):
    y = a * h_prev + x
    r = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
    dy = np.where(capped, lam / r, lam)
    return a * dy, dy, dy * h_prev


def _norm_cap_ignores_cap(h_prev, x, a, h, lam, capped):
    return a * lam, lam, lam * h_prev


def _max_plus_swapped_branches(h_prev, x, c, h, lam, x_won):
    zero = np.zeros_like(lam)
    return np.where(x_won, lam, zero), np.where(x_won, zero, lam), np.where(x_won, -lam, zero)


def _max_plus_cost_sign(h_prev, x, c, h, lam, x_won):
    zero = np.zeros_like(lam)
    return np.where(x_won, zero, lam), np.where(x_won, lam, zero), np.where(x_won, zero, lam)


ES_VJP_MUTANTS = {
    "tanh_no_slope": ("tanh_affine", _tanh_no_slope),
    "tanh_slope_of_input": ("tanh_affine", _tanh_slope_of_input),
    "tanh_swapped": ("tanh_affine", _tanh_swapped),
    "norm_cap_no_projection": ("norm_cap", _norm_cap_no_projection),
    "norm_cap_ignores_cap": ("norm_cap", _norm_cap_ignores_cap),
    "max_plus_swapped_branches": ("max_plus", _max_plus_swapped_branches),
    "max_plus_cost_sign": ("max_plus", _max_plus_cost_sign),
}

ES_VJP_PINS = {
    "tanh_affine": [(pins.test_element_scan_vjp_central_differences, {"body": "tanh_affine", "state": None, "reverse": False}),
                    (pins.test_tanh_affine_vjp_single_trip_and_zero_decay, {})],
    "norm_cap": [(pins.test_element_scan_vjp_central_differences, {"body": "norm_cap", "state": 4, "reverse": True})],
    "max_plus": [(pins.test_max_plus_vjp_exact_by_unit_perturbations, {"reverse": True})],
}


@pytest.mark.parametrize("name", sorted(ES_VJP_MUTANTS))
def test_element_scan_vjp_mutants_are_caught(name, monkeypatch):
    body, fn = ES_VJP_MUTANTS[name]
    monkeypatch.setitem(oracle._VJP, body, fn)
    assert _some_pin_fails(ES_VJP_PINS[body]), f"no gradient pin caught {name}"


def _es_vjp_wrong_prev(body, initial, sequences, g, axis=0, state_axis=None, reverse=False, dtype=np.float64):
    # every trip's incoming state taken as its own result (h[t] for h[t-1])
    real_vjp = oracle._VJP[body]
    def vjp(h_prev, x, a, h, lam, branch):
        return real_vjp(h, x, a, h, lam, branch)
    saved = oracle._VJP[body]
    oracle._VJP[body] = vjp
    try:
        return _real_es_vjp(body, initial, sequences, g, axis, state_axis, reverse, dtype)
    finally:
        oracle._VJP[body] = saved


def _es_vjp_wrong_direction(body, initial, sequences, g, axis=0, state_axis=None, reverse=False, dtype=np.float64):
    return _real_es_vjp(body, initial, sequences, g, axis, state_axis, not reverse, dtype)


_real_es_vjp = oracle.element_scan_vjp


@pytest.mark.parametrize("mutant,body", [(_es_vjp_wrong_prev, "tanh_affine"), (_es_vjp_wrong_prev, "norm_cap"),
                                          (_es_vjp_wrong_direction, "tanh_affine"), (_es_vjp_wrong_direction, "norm_cap"),
                                          (_es_vjp_wrong_direction, "max_plus")])
def test_element_scan_vjp_loop_mutants_are_caught(mutant, body, monkeypatch):
    # (max-plus's VJP reads the incoming state only through its branch decision: see the next test)
    monkeypatch.setattr(oracle, "element_scan_vjp", mutant)
    assert _some_pin_fails(ES_VJP_PINS[body]), f"no {body} gradient pin caught {mutant.__name__}"


def test_max_plus_branch_mutant_is_caught(monkeypatch):
    real = oracle._branches
    def wrong_sign(body, h_prev32, x32, s32):
        return x32 >= (h_prev32 + s32) if body == "max_plus" else real(body, h_prev32, x32, s32)
    monkeypatch.setattr(oracle, "_branches", wrong_sign)
    assert _some_pin_fails(ES_VJP_PINS["max_plus"])


def test_unmutated_element_scan_vjp_passes_its_pins():
    for body in ES_VJP_PINS:
        assert not _some_pin_fails(ES_VJP_PINS[body])


_real_proj = oracle.matrix_scan_projective


def _proj_mutant(kind):
    def f(a, b, axis=0, reverse=False, dtype=np.float64):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        n = a.shape[-1]
        lead = np.broadcast_shapes(a.shape[:-2], b.shape[:-2])
        ax = axis % len(lead)
        a_t = np.moveaxis(np.broadcast_to(a, lead + (n, n)), ax, 0)
        b_t = np.moveaxis(np.broadcast_to(b, lead + b.shape[-2:]), ax, 0)
        T = lead[ax]
        out = np.empty(b_t.shape)
        h = np.zeros(b_t.shape[1:])
        P = np.broadcast_to(np.eye(n), a_t.shape[1:]).copy()
        for t in (range(T - 1, -1, -1) if reverse else range(T)):
            P = a_t[t] @ P if kind != "product_transposed" else P @ a_t[t]
            big = np.max(np.abs(P), axis=(-2, -1), keepdims=True)
            if kind == "sum_not_max":
                big = np.sum(np.abs(P), axis=(-2, -1), keepdims=True)
            big = np.where(big > 0, big, 1.0)
            if kind != "product_not_normalised":
                P = P / big
            if kind == "b_not_divided":
                h = a_t[t] @ h / big + b_t[t]
            else:
                h = (a_t[t] @ h + b_t[t]) / big
            out[t] = h
        return np.moveaxis(out, 0, ax)
    f.__name__ = f"proj_{kind}"
    return f


PROJ_PINS = [
    (pins.test_projective_with_b_after_first_step_zero_is_h_over_the_product_size, {"reverse": False}),
    (pins.test_projective_scalar_multiple_of_identity_is_a_scaled_running_sum, {"c": 2.0}),
]


@pytest.mark.parametrize("kind", ["product_transposed", "sum_not_max", "product_not_normalised", "b_not_divided"])
def test_projective_mutants_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "matrix_scan_projective", _proj_mutant(kind))
    assert _some_pin_fails(PROJ_PINS), f"no projective pin caught {kind}"


def test_unmutated_projective_passes_its_pins():
    assert not _some_pin_fails(PROJ_PINS)
    rng = np.random.default_rng(6)
    a, b = rng.normal(size=(2, 7, 3, 3)), rng.normal(size=(2, 7, 3, 2))
    np.testing.assert_allclose(_proj_mutant("none")(a, b, axis=1), _real_proj(a, b, axis=1), rtol=1e-15)


_real_ts = oracle.table_scan


def _ts_transposed(table, symbols, axis=-1, start=0, clamp=True):
    table = np.asarray(table)
    if table.shape[0] != table.shape[1]:
        return _real_ts(table, symbols, axis, start, clamp)  # (only square tables can be swapped)
    return _real_ts(table.T.copy(), symbols, axis, start, clamp)


def _ts_state_before(table, symbols, axis=-1, start=0, clamp=True):
    # stores the state before each symbol instead of after it
    out = _real_ts(table, symbols, axis, start, clamp)
    ax = axis % np.ndim(symbols)
    shifted = np.roll(out, 1, axis=ax)
    idx = [slice(None)] * out.ndim
    idx[ax] = 0
    shifted[tuple(idx)] = start
    return shifted


def _ts_ignores_start(table, symbols, axis=-1, start=0, clamp=True):
    return _real_ts(table, symbols, axis, 0, clamp)


TS_PINS = [
    (pins.test_table_scan_parity_example_is_running_xor, {}),
    (pins.test_table_scan_counter_mod_k_is_cumsum_mod_k, {"k": 7}),
    (pins.test_table_scan_small_hand_run, {}),
]


@pytest.mark.parametrize("mutant", [_ts_transposed, _ts_state_before, _ts_ignores_start])
def test_table_scan_mutants_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "table_scan", mutant)
    assert _some_pin_fails(TS_PINS), f"no table-scan pin caught {mutant.__name__}"


def test_unmutated_table_scan_passes_its_pins():
    assert not _some_pin_fails(TS_PINS)
