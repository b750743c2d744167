"""The C-ABI boundary on the CPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before any device work.

No call here passes arguments the library would accept, so nothing reaches
the GPU (there is none in the build container).
"""

import ctypes
import pathlib
import re

import numpy as np
import pytest
import torch

import scan_primitives_amd as sx
from scan_primitives_amd import _binding as B

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "sx_scan.h"

FAKE = 1 << 40  # a plausible device address; never dereferenced by a rejected call


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sx_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("sx_element_scan", "sx_matrix_scan", "sx_element_scan_workspace_bytes",
                     "sx_matrix_scan_workspace_bytes", "sx_matrix_scan_out_shape", "sx_linear_scan",
                     "sx_linear_scan_out_shape", "sx_matrix_scan_backward", "sx_matrix_scan_backward_workspace_bytes",
                     "sx_element_scan_backward", "sx_element_scan_backward_workspace_bytes", "sx_table_scan",
                     "sx_matrix_scan_workspace_status", "sx_set_lookback_spin_limit",
                     "sx_status_name", "sx_last_error", "sx_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in sx_scan.h but not exported"


def test_status_names_and_version(lib):
    assert lib.sx_status_name(0) == b"OK"
    assert lib.sx_status_name(1) == b"E-DIM-001"
    assert lib.sx_status_name(2) == b"E-DIM-002"
    assert lib.sx_status_name(3) == b"E-DIM-003"
    assert b"gfx950" in lib.sx_version()


def _es(lib, body=2, shape=(4, 8, 3), axis=1, state_axis=B.SX_STATE_SCALAR, x=FAKE, s=FAKE + 4096,
        init=FAKE + 8192, out=FAKE + (1 << 20), x_width=None, s_width=None, rank=None):
    shape = list(shape)
    r = len(shape) if rank is None else rank
    xw = (shape[-1] if shape else 1) if x_width is None else x_width
    sw = (shape[-1] if shape else 1) if s_width is None else s_width
    st = lib.sx_element_scan(body, r, B.i64_array(shape), axis, state_axis, 0, init, None, x, xw, None, s, sw,
                             None, out, None, 0, None)
    return st, lib.sx_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(axis=3), B.SX_E_DIM_001),
    (dict(axis=-4), B.SX_E_DIM_001),
    (dict(shape=(4, 0, 3)), B.SX_E_DIM_001),                        # empty scan axis
    (dict(body=1), B.SX_E_DIM_001),                                 # norm-cap needs a vector state
    (dict(body=1, shape=(2, 5, 17), state_axis=-1), B.SX_E_DIM_001),  # state width above 16
    (dict(body=1, shape=(2, 5, 16), state_axis=-1, x_width=3), B.SX_E_DIM_001),
    (dict(body=1, shape=(2, 5, 16), state_axis=-1, s_width=4), B.SX_E_DIM_001),
    (dict(body=1, shape=(2, 5, 16), state_axis=0), B.SX_E_DIM_001),    # only the last axis is a state axis
    (dict(body=1, shape=(2, 5, 16), state_axis=-1, axis=2), B.SX_E_DIM_001),  # axis is the state axis
    (dict(x=None), B.SX_E_DIM_003),
    (dict(s=None), B.SX_E_DIM_003),
    (dict(init=None), B.SX_E_DIM_003),
    (dict(out=None), B.SX_E_DIM_003),
    (dict(out=FAKE + 16), B.SX_E_ALIAS),                            # out overlaps x
    (dict(body=9), B.SX_E_UNSUPPORTED),
    (dict(shape=(1,) * 9), B.SX_E_UNSUPPORTED),
    (dict(shape=(), rank=0), B.SX_E_DIM_001),
])
def test_element_scan_rejects_on_host(lib, kwargs, code):
    st, msg = _es(lib, **kwargs)
    assert st == code, (st, msg)
    assert msg.startswith(f"error[{B._STATUS_NAMES[code]}]")


def test_element_scan_error_message_names_shapes(lib):
    st, msg = _es(lib, axis=5)
    assert "[4, 8, 3]" in msg and "axis 5" in msg


def test_element_scan_zero_lanes_is_a_no_op(lib):
    # [0, 6, 3] along axis 1 has no lanes: nothing to launch, nothing to check on the device
    st, _ = _es(lib, shape=(0, 6, 3), x=None, s=None, init=None, out=None)
    assert st == B.SX_OK


def test_element_scan_workspace_query(lib):
    assert lib.sx_element_scan_workspace_bytes(2, 3, B.i64_array([4, 8, 3]), 1, B.SX_STATE_SCALAR) >= 0
    assert lib.sx_element_scan_workspace_bytes(2, 3, B.i64_array([4, 8, 3]), 7, B.SX_STATE_SCALAR) == 0


def _ms(lib, a_shape=(2, 5, 4, 4), b_shape=(2, 5, 4, 3), dtype=B.SX_F32, out_dtype=B.SX_F32, axis=1, projective=0,
        a=FAKE, b=FAKE + (1 << 20), out=FAKE + (1 << 22), a_strides=None):
    st = lib.sx_matrix_scan(dtype, len(a_shape), B.i64_array(a_shape),
                            B.i64_array(a_strides) if a_strides else None, a, len(b_shape), B.i64_array(b_shape),
                            None, b, axis, 0, projective, out_dtype, out, None, 0, None)
    return st, lib.sx_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(a_shape=(2, 5, 17, 17), b_shape=(2, 5, 17, 1)), B.SX_E_DIM_001),  # n above 16
    (dict(a_shape=(2, 5, 4, 3)), B.SX_E_DIM_001),                           # a not square
    (dict(b_shape=(2, 5, 5, 3)), B.SX_E_DIM_001),                           # inner dims differ
    (dict(b_shape=(3, 5, 4, 3)), B.SX_E_DIM_001),                           # leading dims do not broadcast
    (dict(axis=2), B.SX_E_DIM_001),
    (dict(axis=-3), B.SX_E_DIM_001),
    (dict(a_shape=(4, 4), b_shape=(4, 3)), B.SX_E_DIM_001),                 # no leading dim to scan
    (dict(dtype=5), B.SX_E_DIM_002),
    (dict(out_dtype=3), B.SX_E_DIM_002),
    (dict(a=None), B.SX_E_DIM_003),
    (dict(b=None), B.SX_E_DIM_003),
    (dict(out=None), B.SX_E_DIM_003),
    (dict(projective=1, out=None), B.SX_E_DIM_003),                         # :projective checks the same
    (dict(a_strides=(80, 16, 1, 4)), B.SX_E_UNSUPPORTED),                    # transposed matrix dims
    (dict(out=FAKE + 64), B.SX_E_ALIAS),
])
def test_matrix_scan_rejects_on_host(lib, kwargs, code):
    st, msg = _ms(lib, **kwargs)
    assert st == code, (st, msg)


def test_matrix_scan_empty_is_a_no_op(lib):
    st, _ = _ms(lib, a_shape=(2, 0, 4, 4), b_shape=(2, 0, 4, 3), a=None, b=None, out=None)
    assert st == B.SX_OK


def test_matrix_scan_out_shape_broadcasts(lib):
    out = B.i64_array([0] * 10)
    r = lib.sx_matrix_scan_out_shape(3, B.i64_array([7, 4, 4]), 4, B.i64_array([2, 7, 4, 3]), out)
    assert r == 4 and list(out[:4]) == [2, 7, 4, 3]
    r = lib.sx_matrix_scan_out_shape(4, B.i64_array([3, 1, 4, 4]), 3, B.i64_array([5, 4, 1]), out)
    assert r == 4 and list(out[:4]) == [3, 5, 4, 1]
    assert lib.sx_matrix_scan_out_shape(3, B.i64_array([2, 4, 4]), 3, B.i64_array([3, 4, 1]), out) == -1


def test_matrix_scan_workspace_status_checks_arguments_on_the_host(lib):
    # refused before any HIP call: no workspace, or one smaller than its header
    assert lib.sx_matrix_scan_workspace_status(None, 1 << 20, None) == B.SX_E_DIM_003
    assert b"NULL" in lib.sx_last_error()
    assert lib.sx_matrix_scan_workspace_status(ctypes.c_void_p(4096), 64, None) == B.SX_E_WORKSPACE
    assert b"256" in lib.sx_last_error()


def test_matrix_scan_workspace_query_is_host_only(lib):
    ws = lib.sx_matrix_scan_workspace_bytes(4, B.i64_array([32, 8192, 16, 16]), 4, B.i64_array([32, 8192, 16, 1]), 1)
    assert ws >= 0
    assert lib.sx_matrix_scan_workspace_bytes(3, B.i64_array([2, 4, 4]), 3, B.i64_array([2, 5, 1]), 0) == 0


def _msb(lib, a_shape=(2, 5, 4, 4), b_shape=(2, 5, 4, 3), dtype=B.SX_F32, grad=B.SX_F32, axis=1, a=FAKE,
         h=FAKE + (1 << 20), g=FAKE + (2 << 20), ga=FAKE + (4 << 20), gb=FAKE + (5 << 20), ws=FAKE + (8 << 20),
         ws_bytes=1 << 30, g_strides=None):
    st = lib.sx_matrix_scan_backward(dtype, len(a_shape), B.i64_array(a_shape), None, a, len(b_shape),
                                     B.i64_array(b_shape), h, B.i64_array(g_strides) if g_strides else None, g, axis,
                                     0, grad, ga, gb, ws, ws_bytes, None)
    return st, lib.sx_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=4), B.SX_E_DIM_002),
    (dict(grad=9), B.SX_E_DIM_002),
    (dict(b_shape=(2, 5, 5, 3)), B.SX_E_DIM_001),                # inner dims differ
    (dict(b_shape=(3, 5, 4, 3)), B.SX_E_DIM_001),                # leading dims do not broadcast
    (dict(axis=2), B.SX_E_DIM_001),
    (dict(a=None), B.SX_E_DIM_003),
    (dict(h=None), B.SX_E_DIM_003),
    (dict(g=None), B.SX_E_DIM_003),
    (dict(ga=None), B.SX_E_DIM_003),
    (dict(gb=None), B.SX_E_DIM_003),
    (dict(ga=FAKE + 64), B.SX_E_ALIAS),                           # grad_a over a
    (dict(gb=FAKE + (2 << 20) + 8), B.SX_E_ALIAS),               # grad_b over g
    (dict(gb=FAKE + (4 << 20) + 16), B.SX_E_ALIAS),              # grad_b over grad_a
    (dict(ws=None), B.SX_E_WORKSPACE),
    (dict(ws_bytes=64), B.SX_E_WORKSPACE),
    (dict(ws=FAKE + (8 << 20) + 4), B.SX_E_WORKSPACE),           # not 256-byte aligned
    (dict(g_strides=(60, 12, 1, 4)), B.SX_E_UNSUPPORTED),        # g's matrix dims transposed
])
def test_matrix_scan_backward_rejects_on_host(lib, kwargs, code):
    st, msg = _msb(lib, **kwargs)
    assert st == code, (st, msg)
    assert msg


def test_matrix_scan_backward_empty_is_a_no_op(lib):
    st, _ = _msb(lib, a_shape=(2, 0, 4, 4), b_shape=(2, 0, 4, 3), a=None, h=None, g=None, ga=None, gb=None, ws=None,
                 ws_bytes=0)
    assert st == B.SX_OK


def test_matrix_scan_backward_workspace_query(lib):
    q = lib.sx_matrix_scan_backward_workspace_bytes
    full = q(4, B.i64_array([32, 8192, 16, 16]), 4, B.i64_array([32, 8192, 16, 1]), 1, B.SX_F32)
    assert full > 0 and full % 256 == 0
    # a broadcast over the batch needs room for the full-shape grad_a before its sum
    shared = q(3, B.i64_array([8192, 16, 16]), 4, B.i64_array([32, 8192, 16, 1]), 1, B.SX_F32)
    assert shared >= full + 32 * 8192 * 256 * 4
    # bf16 gradients with b at the result's shape: the adjoint goes into grad_b itself, rounded
    assert q(4, B.i64_array([32, 8192, 16, 16]), 4, B.i64_array([32, 8192, 16, 1]), 1, B.SX_BF16) == full
    # ... and with a broadcast b it is kept in f32 for the sum
    assert q(4, B.i64_array([32, 8192, 16, 16]), 3, B.i64_array([8192, 16, 1]), 1, B.SX_BF16) >= \
        full + 32 * 8192 * 16 * 4
    assert q(3, B.i64_array([2, 4, 4]), 3, B.i64_array([2, 5, 1]), 0, B.SX_F32) == 0


def _esb(lib, body=2, shape=(4, 8, 3), axis=1, state_axis=B.SX_STATE_SCALAR, ptrs=None, x_width=3, s_width=3,
         ws=None, ws_bytes=0):
    base = {"initial": FAKE, "x": FAKE + (1 << 20), "s": FAKE + (2 << 20), "h": FAKE + (3 << 20), "g": FAKE + (4 << 20),
            "gi": FAKE + (5 << 20), "gx": FAKE + (6 << 20), "gs": FAKE + (7 << 20)}
    base.update(ptrs or {})
    st = lib.sx_element_scan_backward(body, len(shape), B.i64_array(shape), axis, state_axis, 0, base["initial"],
                                      base["x"], x_width, None, base["s"], s_width, None, base["h"], base["g"],
                                      base["gi"], base["gx"], base["gs"], ws, ws_bytes, None)
    return st, lib.sx_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(body=7), B.SX_E_UNSUPPORTED),
    (dict(axis=3), B.SX_E_DIM_001),
    (dict(shape=(4, 0, 3)), B.SX_E_DIM_001),                              # empty scan axis
    (dict(body=1), B.SX_E_DIM_001),                                       # norm-cap needs a vector state
    (dict(ptrs={"initial": None}), B.SX_E_DIM_003),
    (dict(ptrs={"h": None}), B.SX_E_DIM_003),
    (dict(ptrs={"g": None}), B.SX_E_DIM_003),
    (dict(ptrs={"gi": None}), B.SX_E_DIM_003),
    (dict(ptrs={"gx": None}), B.SX_E_DIM_003),
    (dict(ptrs={"gs": None}), B.SX_E_DIM_003),
    (dict(ptrs={"gx": FAKE + (3 << 20) + 8}), B.SX_E_ALIAS),             # grad_x over h
    (dict(ptrs={"gs": FAKE + (6 << 20) + 4}), B.SX_E_ALIAS),             # grad_s over grad_x
    (dict(ptrs={"gi": FAKE + 4}), B.SX_E_ALIAS),                          # grad_initial over initial
    (dict(body=0, shape=(4, 8, 3), state_axis=-1, x_width=3, s_width=1), B.SX_E_WORKSPACE),  # width-1 gate sums
    (dict(body=1, shape=(4, 64, 3), state_axis=-1, x_width=3, s_width=3), B.SX_E_WORKSPACE),  # norm-cap split
])
def test_element_scan_backward_rejects_on_host(lib, kwargs, code):
    st, msg = _esb(lib, **kwargs)
    assert st == code, (st, msg)
    assert msg


def test_element_scan_backward_workspace_query(lib):
    q = lib.sx_element_scan_backward_workspace_bytes
    assert q(0, 3, B.i64_array([4, 64, 32]), 1, B.SX_STATE_SCALAR, 32, 32) == 0
    need = q(0, 4, B.i64_array([8, 1024, 16, 16]), 1, -1, 16, 1)
    assert need >= 8 * 1024 * 16 * 16 * 4 and need % 256 == 0   # the width-1 gate's full-width gradient
    # norm-cap sums a width-one gate's gradient in its kernels: only the split's bounds remain
    # (128 state vectors, 128 chunks of 8 trips: two bounds per vector and group of chunks (8 groups)
    # and one product per chunk and vector)
    assert q(1, 4, B.i64_array([8, 1024, 16, 16]), 1, -1, 16, 1) == (2 * 8 + 128) * 128 * 4
    assert q(1, 4, B.i64_array([8, 1024, 4096, 16]), 1, -1, 1, 1) == 0
    # norm-cap with few state vectors splits the axis
    assert q(1, 4, B.i64_array([8, 1024, 16, 16]), 1, -1, 16, 16) == (2 * 8 + 128) * 128 * 4
    assert q(1, 4, B.i64_array([8, 15, 16, 16]), 1, -1, 16, 16) == 0     # too few trips to split
    assert q(1, 4, B.i64_array([8, 1024, 4096, 16]), 1, -1, 16, 16) == 0  # enough state vectors
    assert q(0, 4, B.i64_array([8, 1024, 16, 16]), 1, -1, 16, 16) == 0   # tanh-affine needs none
    assert q(2, 3, B.i64_array([4, 8, 3]), 5, B.SX_STATE_SCALAR, 3, 3) == 0  # invalid axis


def _ts(lib, states=3, nsym=4, table=FAKE, shape=(5, 9), symbols=FAKE + (1 << 20), axis=-1, start=0,
        out=FAKE + (2 << 20)):
    st = lib.sx_table_scan(states, nsym, table, len(shape), B.i64_array(shape), None, symbols, axis, start, out, None)
    return st, lib.sx_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(nsym=0), B.SX_E_DIM_001),                          # a table with no symbols
    (dict(states=0), B.SX_E_DIM_001),
    (dict(axis=2), B.SX_E_DIM_001),
    (dict(axis=-3), B.SX_E_DIM_001),
    (dict(start=3), B.SX_E_DIM_001),                         # :start is not a state
    (dict(start=-1), B.SX_E_DIM_001),
    (dict(shape=()), B.SX_E_DIM_001),
    (dict(table=None), B.SX_E_DIM_003),
    (dict(symbols=None), B.SX_E_DIM_003),
    (dict(out=None), B.SX_E_DIM_003),
    (dict(out=FAKE + (1 << 20) + 8), B.SX_E_ALIAS),         # out over symbols
    (dict(out=FAKE + 4), B.SX_E_ALIAS),                      # out over the table
])
def test_table_scan_rejects_on_host(lib, kwargs, code):
    st, msg = _ts(lib, **kwargs)
    assert st == code, (st, msg)
    assert msg


def test_table_scan_empty_is_a_no_op(lib):
    assert _ts(lib, shape=(5, 0), table=None, symbols=None, out=None)[0] == B.SX_OK


def test_table_scan_binding_checks_dtypes():
    with pytest.raises(sx.SxError) as e:
        sx.table_scan(torch.zeros((2, 2), dtype=torch.int32), torch.zeros(5, dtype=torch.int32))
    assert e.value.name == "E-UNSUPPORTED"  # host tensors


def _ls(lib, a_shape=(3, 9, 5), b_shape=(3, 9, 5), dtype=B.SX_F32, out_dtype=B.SX_F32, axis=1, a=FAKE,
        b=FAKE + (1 << 20), out=FAKE + (1 << 22), a_strides=None, b_strides=None):
    st = lib.sx_linear_scan(dtype, len(a_shape), B.i64_array(a_shape) if a_shape else None,
                            B.i64_array(a_strides) if a_strides else None, a, len(b_shape),
                            B.i64_array(b_shape) if b_shape else None, B.i64_array(b_strides) if b_strides else None,
                            b, axis, 0, out_dtype, out, None)
    return st, lib.sx_last_error().decode()


@pytest.mark.parametrize("kwargs,code", [
    (dict(b_shape=(3, 8, 5)), B.SX_E_DIM_001),                 # shapes do not broadcast
    (dict(a_shape=(2, 9, 1)), B.SX_E_DIM_001),                 # leading 2 against b's 3
    (dict(axis=3), B.SX_E_DIM_001),
    (dict(axis=-4), B.SX_E_DIM_001),
    (dict(a_shape=(), b_shape=()), B.SX_E_DIM_001),            # two numbers: no axis
    (dict(dtype=2), B.SX_E_DIM_002),
    (dict(out_dtype=7), B.SX_E_DIM_002),
    (dict(a=None), B.SX_E_DIM_003),
    (dict(b=None), B.SX_E_DIM_003),
    (dict(out=None), B.SX_E_DIM_003),
    (dict(out=FAKE + 64), B.SX_E_ALIAS),                        # out over a
    (dict(out=FAKE + (1 << 20) + 4), B.SX_E_ALIAS),            # out over b
    (dict(a_shape=(1, 2, 3, 4, 5, 6, 7, 8, 9)), B.SX_E_UNSUPPORTED),
])
def test_linear_scan_rejects_on_host(lib, kwargs, code):
    st, msg = _ls(lib, **kwargs)
    assert st == code, (st, msg)
    assert msg


def test_linear_scan_empty_is_a_no_op(lib):
    assert _ls(lib, a_shape=(3, 0, 5), b_shape=(3, 0, 5), a=None, b=None, out=None)[0] == B.SX_OK
    assert _ls(lib, a_shape=(), b_shape=(0, 9, 5), a=None, b=None, out=None)[0] == B.SX_OK


def test_linear_scan_out_shape_broadcasts(lib):
    out = B.i64_array([0] * 8)
    assert lib.sx_linear_scan_out_shape(0, None, 3, B.i64_array([4, 6, 2]), out) == 3
    assert list(out[:3]) == [4, 6, 2]
    assert lib.sx_linear_scan_out_shape(2, B.i64_array([6, 1]), 3, B.i64_array([4, 1, 2]), out) == 3
    assert list(out[:3]) == [4, 6, 2]
    assert lib.sx_linear_scan_out_shape(1, B.i64_array([5]), 0, None, out) == 1 and out[0] == 5
    assert lib.sx_linear_scan_out_shape(2, B.i64_array([2, 3]), 2, B.i64_array([3, 3]), out) == -1
    assert lib.sx_linear_scan_out_shape(0, None, 0, None, out) == -1


def test_linear_scan_binding_refuses_before_the_device():
    with pytest.raises(sx.SxError) as e:
        sx.linear_scan(0.5, 2.0)
    assert e.value.name == "E-DIM-001"
    with pytest.raises(sx.SxError) as e:
        sx.cumsum(torch.zeros(4, 3))
    assert e.value.name == "E-UNSUPPORTED"  # a host tensor: the library takes device tensors
    with pytest.raises(sx.SxError) as e:
        sx.linear_scan(torch.zeros(4, 3), [1.0, 2.0])
    assert e.value.name in ("E-UNSUPPORTED", "E-DIM-003")


def test_binding_refuses_host_tensors_and_bad_dtypes():
    x = torch.zeros(2, 3, 4)
    with pytest.raises(sx.SxError) as e:
        sx.element_scan("max_plus", torch.zeros(2, 4), [x, x], axis=1)
    assert e.value.name == "E-UNSUPPORTED"
    with pytest.raises(sx.SxError) as e:
        sx.matrix_scan(torch.zeros(2, 3, 3), torch.zeros(2, 3, 1, dtype=torch.float64))
    assert e.value.code in (B.SX_E_UNSUPPORTED, B.SX_E_DIM_002)
    with pytest.raises(sx.SxError):
        sx.element_scan("no_such_body", torch.zeros(2, 4), [x, x])
    with pytest.raises(sx.SxError) as e:
        sx.element_scan("max_plus", torch.zeros(2, 4), [x, x, x], axis=1)
    assert e.value.name == "E-DIM-001"


def test_workloads_describe_the_standard_configurations():
    from scan_primitives_amd import workloads as W
    w = W.make_tanh()
    assert w.out_shape == (4, 64, 32) and w.algorithmic_bytes == 98816
    w = W.make_norm_cap(B=2, T=8)
    assert w.out_shape == (2, 8, 16, 16)
    w = W.make_matrix(2, 8, 16, 16, torch.bfloat16)
    assert w.tensors["a"].dtype == torch.bfloat16
    # the draws are seeded: the same call gives the same tensors
    assert torch.equal(W.make_tanh().tensors["x"], W.make_tanh().tensors["x"])
    np.testing.assert_array_equal(W.make_max_plus((2, 8, 4)).tensors["s"].numpy() >= 0, True)


def test_algorithmic_bytes_of_the_large_workloads():
    # full sizes, computed from shapes alone (no tensors are drawn here)
    sizes = {
        "norm-cap": (8 * 1024 * 16 * 16 * 4 * 2 + 8 * 1024 * 16 * 4 + 8 * 16 * 16 * 4, 17309696),
        "max-plus": (64 * 4096 * 256 * 4 * 3 + 64 * 256 * 4, 805371904),
        "matrix f32": (32 * 8192 * (256 + 16 + 16) * 4, 301989888),
        "matrix bf16": (16 * 16384 * (256 + 256 + 256) * 2, 402653184),
    }
    for name, (got, want) in sizes.items():
        assert got == want, name


def test_fake_pointer_constant_is_not_null():
    assert ctypes.c_void_p(FAKE).value == FAKE
