"""ctypes binding over libsx_scan.so (C ABI in include/sx_scan.h).

Argument marshalling only: shapes, strides, pointers, the workspace and the
current torch stream go to the C library, whose HIP kernels do every step of
the scan. There is no CPU fallback: without the built library every call
raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# SX_SCAN_LIB selects another build of the same library (the host-sanitized one the
# boundary tests run under); by default the in-tree libsx_scan.so.
LIB_PATH = os.environ.get("SX_SCAN_LIB") or os.path.join(HERE, "libsx_scan.so")

SX_OK = 0
SX_E_DIM_001 = 1
SX_E_DIM_002 = 2
SX_E_DIM_003 = 3
SX_E_UNSUPPORTED = 4
SX_E_ALIAS = 5
SX_E_WORKSPACE = 6
SX_E_DEVICE = 7
SX_STATE_SCALAR = -(2 ** 31)
SX_F32 = 0
SX_BF16 = 1

BODIES = {"tanh_affine": 0, "norm_cap": 1, "max_plus": 2}
_DTYPES = {torch.float32: SX_F32, torch.bfloat16: SX_BF16}
_STATUS_NAMES = {0: "OK", 1: "E-DIM-001", 2: "E-DIM-002", 3: "E-DIM-003", 4: "E-UNSUPPORTED",
                 5: "E-ALIAS", 6: "E-WORKSPACE", 7: "E-DEVICE"}


class SxError(RuntimeError):
    """A call the library (or this binding, before calling it) refused."""

    def __init__(self, code: int, message: str):
        super().__init__(message)
        self.code = code
        self.name = _STATUS_NAMES.get(code, "E-UNKNOWN")


_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsx_scan.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m scan_primitives_amd.build_lib` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    lib.sx_element_scan.restype = c_int
    lib.sx_element_scan.argtypes = [c_int, c_int, _i64p, c_int, c_int, c_int,
                                    vp, _i64p, vp, ctypes.c_int64, _i64p, vp, ctypes.c_int64, _i64p,
                                    vp, vp, c_size, vp]
    lib.sx_element_scan_workspace_bytes.restype = c_size
    lib.sx_element_scan_workspace_bytes.argtypes = [c_int, c_int, _i64p, c_int, c_int]
    lib.sx_matrix_scan.restype = c_int
    lib.sx_matrix_scan.argtypes = [c_int, c_int, _i64p, _i64p, vp, c_int, _i64p, _i64p, vp,
                                   c_int, c_int, c_int, c_int, vp, vp, c_size, vp]
    lib.sx_matrix_scan_noalloc.restype = c_int
    lib.sx_matrix_scan_noalloc.argtypes = [c_int, c_int, _i64p, _i64p, vp, c_int, _i64p, _i64p, vp,
                                           c_int, c_int, c_int, c_int, vp, vp]
    lib.sx_matrix_scan_workspace_bytes.restype = c_size
    lib.sx_matrix_scan_workspace_bytes.argtypes = [c_int, _i64p, c_int, _i64p, c_int]
    lib.sx_matrix_scan_out_shape.restype = c_int
    lib.sx_matrix_scan_out_shape.argtypes = [c_int, _i64p, c_int, _i64p, _i64p]
    lib.sx_element_scan_backward.restype = c_int
    lib.sx_element_scan_backward.argtypes = [c_int, c_int, _i64p, c_int, c_int, c_int, vp, vp, ctypes.c_int64, _i64p,
                                             vp, ctypes.c_int64, _i64p, vp, vp, vp, vp, vp, vp, c_size, vp]
    lib.sx_element_scan_backward_workspace_bytes.restype = c_size
    lib.sx_element_scan_backward_workspace_bytes.argtypes = [c_int, c_int, _i64p, c_int, c_int, ctypes.c_int64,
                                                             ctypes.c_int64]
    lib.sx_matrix_scan_backward.restype = c_int
    lib.sx_matrix_scan_backward.argtypes = [c_int, c_int, _i64p, _i64p, vp, c_int, _i64p, vp, _i64p, vp,
                                            c_int, c_int, c_int, vp, vp, vp, c_size, vp]
    lib.sx_matrix_scan_backward_workspace_bytes.restype = c_size
    lib.sx_matrix_scan_backward_workspace_bytes.argtypes = [c_int, _i64p, c_int, _i64p, c_int, c_int]
    lib.sx_table_scan.restype = c_int
    lib.sx_table_scan.argtypes = [c_int, c_int, vp, c_int, _i64p, _i64p, vp, c_int, ctypes.c_int32, vp, vp]
    lib.sx_linear_scan.restype = c_int
    lib.sx_linear_scan.argtypes = [c_int, c_int, _i64p, _i64p, vp, c_int, _i64p, _i64p, vp,
                                   c_int, c_int, c_int, vp, vp]
    lib.sx_linear_scan_out_shape.restype = c_int
    lib.sx_linear_scan_out_shape.argtypes = [c_int, _i64p, c_int, _i64p, _i64p]
    lib.sx_matrix_scan_workspace_status.restype = c_int
    lib.sx_matrix_scan_workspace_status.argtypes = [vp, c_size, vp]
    lib.sx_set_lookback_spin_limit.restype = None
    lib.sx_set_lookback_spin_limit.argtypes = [ctypes.c_uint32]
    lib.sx_status_name.restype = ctypes.c_char_p
    lib.sx_status_name.argtypes = [c_int]
    lib.sx_last_error.restype = ctypes.c_char_p
    lib.sx_last_error.argtypes = []
    lib.sx_version.restype = ctypes.c_char_p
    lib.sx_version.argtypes = []
    _lib = lib
    return lib


def i64_array(values) -> ctypes.Array:
    values = list(values)
    return (ctypes.c_int64 * max(len(values), 1))(*values)


def _check(status: int) -> None:
    if status != SX_OK:
        msg = load_library().sx_last_error().decode()
        raise SxError(status, msg or _STATUS_NAMES.get(status, str(status)))


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# Matrix-scan workspaces. The library needs each one zero-filled once and then
# leaves it ready for the next call, so no call clears anything. Eager calls get
# one per (device, stream), zero-filled when allocated. Calls captured into a
# graph get one per capture (keyed by the HIP capture id), allocated and
# zero-filled inside that capture: every graph then starts from a zeroed
# workspace of its own in its first replay, and no captured workspace is handed
# to an eager call or to another graph.
_matrix_workspaces: dict = {}
_hip_runtime = None


def _capture_id(stream_handle: int):
    """The id of the capture running on the stream, or None."""
    global _hip_runtime
    if _hip_runtime is None:
        # the HIP runtime torch has loaded (the same soname the library links)
        hip = ctypes.CDLL("libamdhip64.so.7")
        hip.hipStreamGetCaptureInfo.restype = ctypes.c_int
        hip.hipStreamGetCaptureInfo.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int),
                                                ctypes.POINTER(ctypes.c_ulonglong)]
        _hip_runtime = hip
    status, cid = ctypes.c_int(0), ctypes.c_ulonglong(0)
    err = _hip_runtime.hipStreamGetCaptureInfo(stream_handle, ctypes.byref(status), ctypes.byref(cid))
    if err != 0:
        raise SxError(SX_E_DEVICE, f"hipStreamGetCaptureInfo failed with HIP error {err}")
    return int(cid.value) if status.value == 1 else None  # 1: hipStreamCaptureStatusActive


def _matrix_workspace(nbytes: int, device: torch.device):
    if nbytes == 0:
        return None
    handle = torch.cuda.current_stream(device).cuda_stream
    cid = _capture_id(handle) if torch.cuda.is_current_stream_capturing() else None
    key = (device.index, handle, cid)
    entry = _matrix_workspaces.get(key)
    if entry is not None and entry.numel() >= nbytes:
        return entry
    size = (nbytes + (1 << 20) - 1) >> 20 << 20
    if entry is not None:
        size = max(size, entry.numel())
    ws = torch.zeros(size, dtype=torch.uint8, device=device)
    _matrix_workspaces[key] = ws
    return ws


def matrix_scan_status(device=None) -> None:
    """Raise ``SxError`` (E-DEVICE) if a matrix-scan look-back gave up on one of
    this device's eager workspaces since the last check, and clear what it
    found. Waits for the streams those workspaces belong to."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    for (index, handle, cid), ws in list(_matrix_workspaces.items()):
        if index != dev.index or cid is not None:
            continue
        with torch.cuda.device(dev):
            _check(lib.sx_matrix_scan_workspace_status(ws.data_ptr(), ws.numel(), handle))


def set_lookback_spin_limit(limit: int) -> None:
    """Bound on the polls a matrix-scan look-back makes before it gives up and
    records it (0 restores the default). A diagnostic for the give-up report."""
    load_library().sx_set_lookback_spin_limit(int(limit))


def _require_device_tensor(name: str, t) -> None:
    if not isinstance(t, torch.Tensor):
        raise SxError(SX_E_DIM_003, f"{name}: a tensor was expected, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise SxError(SX_E_UNSUPPORTED, f"{name}: the HIP library takes device tensors, got {t.device}")


def element_scan(body: str, initial: torch.Tensor, sequences, axis: int = 0, state_axis=None,
                 reverse: bool = False) -> torch.Tensor:
    """Element scan on the GPU: ``"tanh_affine"``, ``"norm_cap"`` or ``"max_plus"``.

    ``sequences`` is ``[x, decay]`` or ``[x, cost]`` (page order). ``state_axis``
    is ``None`` for a scalar state or ``-1`` for a vector state along the last
    axis. Returns a new f32 tensor of the sequences' shape. When autograd
    records (an input requires grad), the gradient runs through
    ``element_scan_backward``.
    """
    seqs = list(sequences)
    if torch.is_grad_enabled() and any(isinstance(t, torch.Tensor) and t.requires_grad for t in [initial] + seqs):
        if len(seqs) != 2:
            raise SxError(SX_E_DIM_001, f"element-scan: the {body} body takes two sequences, got {len(seqs)}")
        return _ElementScanFunction.apply(body, axis, state_axis, reverse, initial, seqs[0], seqs[1])
    return _element_scan_forward(body, initial, seqs, axis, state_axis, reverse)


def _element_scan_forward(body, initial, sequences, axis, state_axis, reverse) -> torch.Tensor:
    if body not in BODIES:
        raise SxError(SX_E_UNSUPPORTED, f"element-scan: unknown body {body!r}")
    seqs = list(sequences)
    if len(seqs) != 2:
        raise SxError(SX_E_DIM_001, f"element-scan: the {body} body takes two sequences, got {len(seqs)}")
    x, s = seqs
    for name, t in (("initial", initial), ("x", x), ("sequence 2", s)):
        _require_device_tensor(name, t)
        if t.dtype != torch.float32:
            raise SxError(SX_E_DIM_002, f"element-scan: {name} is {t.dtype}, sequences and initial are f32")
    if not (x.device == s.device == initial.device):
        raise SxError(SX_E_UNSUPPORTED, "element-scan: operands on different devices")
    rank = x.dim()
    vec = state_axis is not None
    if vec:
        if rank < 2 or initial.dim() < 1:
            raise SxError(SX_E_DIM_001, "element-scan: a vector state needs sequences of rank >= 2")
        n = initial.shape[-1]
        out_shape = tuple(x.shape[:-1]) + (n,)
        if tuple(s.shape[:-1]) != tuple(x.shape[:-1]):
            raise SxError(SX_E_DIM_001, f"element-scan: sequences {tuple(x.shape)} and {tuple(s.shape)} "
                                        "differ outside the state axis")
        x_width, s_width = x.shape[-1], s.shape[-1]
        sa = state_axis
    else:
        out_shape = tuple(x.shape)
        if tuple(s.shape) != out_shape:
            raise SxError(SX_E_DIM_001, f"element-scan: sequences {tuple(x.shape)} and {tuple(s.shape)} differ")
        x_width = s_width = out_shape[-1] if rank else 1
        sa = SX_STATE_SCALAR
    ax = axis + rank if axis < 0 else axis
    if 0 <= ax < rank:
        expect_init = out_shape[:ax] + out_shape[ax + 1:]
        if tuple(initial.shape) != expect_init:
            raise SxError(SX_E_DIM_001, f"element-scan: initial {tuple(initial.shape)} f32 does not match the "
                                        f"sequence shape {out_shape} without axis {axis}")
    lib = load_library()
    out = torch.empty(out_shape, dtype=torch.float32, device=x.device)
    shape_a = i64_array(out_shape)
    ws_bytes = lib.sx_element_scan_workspace_bytes(BODIES[body], rank, shape_a, axis, sa)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
    with torch.cuda.device(x.device):
        status = lib.sx_element_scan(
            BODIES[body], rank, shape_a, axis, sa, 1 if reverse else 0,
            initial.data_ptr(), i64_array(initial.stride()),
            x.data_ptr(), x_width, i64_array(x.stride()),
            s.data_ptr(), s_width, i64_array(s.stride()),
            out.data_ptr(), ws.data_ptr() if ws is not None else None, ws_bytes,
            _stream_handle(x.device))
    _check(status)
    return out


def element_scan_backward(body: str, initial: torch.Tensor, sequences, h: torch.Tensor, g: torch.Tensor,
                          axis: int = 0, state_axis=None, reverse: bool = False):
    """Gradients ``(grad_initial, [grad_x, grad_s])`` of a loss through
    ``h = element_scan(body, initial, sequences, axis, state_axis, reverse)``,
    given that call's result ``h`` and the loss's gradient ``g`` with respect
    to it. Each gradient has its tensor's shape; all are f32.
    """
    if body not in BODIES:
        raise SxError(SX_E_UNSUPPORTED, f"element-scan gradient: unknown body {body!r}")
    seqs = list(sequences)
    if len(seqs) != 2:
        raise SxError(SX_E_DIM_001, f"element-scan gradient: the {body} body takes two sequences, got {len(seqs)}")
    x, s = seqs
    for name, t in (("initial", initial), ("x", x), ("sequence 2", s), ("h", h), ("g", g)):
        _require_device_tensor(name, t)
        if t.dtype != torch.float32:
            raise SxError(SX_E_DIM_002, f"element-scan gradient: {name} is {t.dtype}; element scans are f32")
    if tuple(g.shape) != tuple(h.shape):
        raise SxError(SX_E_DIM_001, f"element-scan gradient: g {tuple(g.shape)} and h {tuple(h.shape)} differ")
    rank = h.dim()
    vec = state_axis is not None
    x_width = x.shape[-1] if vec else (h.shape[-1] if rank else 1)
    s_width = s.shape[-1] if vec else (h.shape[-1] if rank else 1)
    sa = state_axis if vec else SX_STATE_SCALAR
    initial, h, g = initial.contiguous(), h.contiguous(), g.contiguous()
    lib = load_library()
    shape_a = i64_array(h.shape)
    ws_bytes = lib.sx_element_scan_backward_workspace_bytes(BODIES[body], rank, shape_a, axis, sa, x_width, s_width)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=h.device) if ws_bytes else None
    gi, gx, gs = torch.empty_like(initial), torch.empty(tuple(x.shape), dtype=torch.float32, device=h.device), \
        torch.empty(tuple(s.shape), dtype=torch.float32, device=h.device)
    with torch.cuda.device(h.device):
        status = lib.sx_element_scan_backward(
            BODIES[body], rank, shape_a, axis, sa, 1 if reverse else 0, initial.data_ptr(),
            x.data_ptr(), x_width, i64_array(x.stride()), s.data_ptr(), s_width, i64_array(s.stride()),
            h.data_ptr(), g.data_ptr(), gi.data_ptr(), gx.data_ptr(), gs.data_ptr(),
            ws.data_ptr() if ws is not None else None, ws_bytes, _stream_handle(h.device))
    _check(status)
    return gi, [gx, gs]


class _ElementScanFunction(torch.autograd.Function):
    """element_scan with its gradient from the library: saves the inputs and the result."""

    @staticmethod
    def forward(ctx, body, axis, state_axis, reverse, initial, x, s):
        h = _element_scan_forward(body, initial, [x, s], axis, state_axis, reverse)
        ctx.save_for_backward(initial, x, s, h)
        ctx.args = (body, axis, state_axis, reverse)
        return h

    @staticmethod
    def backward(ctx, g):
        initial, x, s, h = ctx.saved_tensors
        body, axis, state_axis, reverse = ctx.args
        gi, (gx, gs) = element_scan_backward(body, initial, [x, s], h, g, axis=axis, state_axis=state_axis,
                                             reverse=reverse)
        return None, None, None, None, gi, gx, gs


def matrix_scan(a: torch.Tensor, b: torch.Tensor, axis: int = 0, reverse: bool = False,
                out_dtype=None, projective: bool = False) -> torch.Tensor:
    """Matrix scan on the GPU: ``h[t] = a[t] @ h[t-1] + b[t]`` along ``axis``.

    ``a`` is ``[..., n, n]`` and ``b`` ``[..., n, m]`` of one dtype (f32 or
    bf16); the leading dims broadcast. The result has the broadcast leading
    shape plus ``[n, m]`` and ``b``'s dtype unless ``out_dtype`` says
    otherwise. Computation is f32. When autograd records (an input requires
    grad), the gradient runs through ``matrix_scan_backward``.
    """
    if torch.is_grad_enabled() and any(isinstance(t, torch.Tensor) and t.requires_grad for t in (a, b)):
        return _MatrixScanFunction.apply(a, b, axis, reverse, out_dtype, projective)
    return _matrix_scan_forward(a, b, axis, reverse, out_dtype, projective)


def _matrix_scan_forward(a, b, axis, reverse, out_dtype, projective) -> torch.Tensor:
    _require_device_tensor("a", a)
    _require_device_tensor("b", b)
    if a.dtype != b.dtype or a.dtype not in _DTYPES:
        raise SxError(SX_E_DIM_002, f"matrix-scan: a is {a.dtype} and b is {b.dtype}; one float dtype "
                                    "(f32 or bf16) is required")
    if a.device != b.device:
        raise SxError(SX_E_UNSUPPORTED, "matrix-scan: operands on different devices")
    out_dtype = b.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise SxError(SX_E_DIM_002, f"matrix-scan: out dtype {out_dtype} is not f32 or bf16")
    lib = load_library()
    # The library reads the two matrix dims row-major; other layouts are copied to that one here.
    if a.dim() >= 2 and not _matrix_dims_contiguous(a):
        a = a.contiguous()
    if b.dim() >= 2 and not _matrix_dims_contiguous(b):
        b = b.contiguous()
    a_shape, b_shape = i64_array(a.shape), i64_array(b.shape)
    oshape = i64_array([0] * 10)
    r = lib.sx_matrix_scan_out_shape(a.dim(), a_shape, b.dim(), b_shape, oshape)
    if r < 0:
        # let the library produce the precise status and message
        _check(lib.sx_matrix_scan(_DTYPES[a.dtype], a.dim(), a_shape, None, None, b.dim(), b_shape, None, None,
                                  axis, 0, 0, _DTYPES[out_dtype], None, None, 0, None))
        raise SxError(SX_E_DIM_001, "matrix-scan: shapes do not fit")
    out = torch.empty(tuple(oshape[:r]), dtype=out_dtype, device=a.device)
    ws_bytes = lib.sx_matrix_scan_workspace_bytes(a.dim(), a_shape, b.dim(), b_shape, axis)
    ws = _matrix_workspace(ws_bytes, a.device)
    with torch.cuda.device(a.device):
        status = lib.sx_matrix_scan(
            _DTYPES[a.dtype], a.dim(), a_shape, i64_array(a.stride()), a.data_ptr(),
            b.dim(), b_shape, i64_array(b.stride()), b.data_ptr(),
            axis, 1 if reverse else 0, 1 if projective else 0, _DTYPES[out_dtype], out.data_ptr(),
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
            _stream_handle(a.device))
    _check(status)
    return out


def linear_scan(a, b, axis: int = 0, reverse: bool = False, out_dtype=None) -> torch.Tensor:
    """Linear scan on the GPU: ``h[t] = a[t] * h[t-1] + b[t]`` along ``axis`` from ``h = 0``.

    Matrix-scan over one-by-one matrices. ``a`` and ``b`` are tensors of one
    float dtype (f32 or bf16) or numbers, broadcast to one shape (at least one
    of them a tensor of rank >= 1); a number takes the tensor's dtype. The
    result has the broadcast shape and that dtype unless ``out_dtype`` says
    otherwise. Computation is f32.
    """
    ta = a if isinstance(a, torch.Tensor) else None
    tb = b if isinstance(b, torch.Tensor) else None
    if ta is None and tb is None:
        raise SxError(SX_E_DIM_001, "linear-scan: a and b are both numbers; there is no axis to scan along")
    ref = tb if tb is not None else ta
    _require_device_tensor("a" if ref is ta else "b", ref)
    # A number becomes a rank-0 tensor on the device (a fill kernel, no host copy).
    if ta is None:
        ta = torch.full((), float(a), dtype=ref.dtype, device=ref.device)
    if tb is None:
        tb = torch.full((), float(b), dtype=ref.dtype, device=ref.device)
    _require_device_tensor("a", ta)
    _require_device_tensor("b", tb)
    if ta.dtype != tb.dtype or ta.dtype not in _DTYPES:
        raise SxError(SX_E_DIM_002, f"linear-scan: a is {ta.dtype} and b is {tb.dtype}; one float dtype "
                                    "(f32 or bf16) is required")
    if ta.device != tb.device:
        raise SxError(SX_E_UNSUPPORTED, "linear-scan: operands on different devices")
    out_dtype = tb.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise SxError(SX_E_DIM_002, f"linear-scan: out dtype {out_dtype} is not f32 or bf16")
    lib = load_library()
    a_shape, b_shape = i64_array(ta.shape), i64_array(tb.shape)
    oshape = i64_array([0] * 8)
    r = lib.sx_linear_scan_out_shape(ta.dim(), a_shape, tb.dim(), b_shape, oshape)
    if r < 0:
        # let the library produce the precise status and message
        _check(lib.sx_linear_scan(_DTYPES[ta.dtype], ta.dim(), a_shape, None, None, tb.dim(), b_shape, None, None,
                                  axis, 0, _DTYPES[out_dtype], None, None))
        raise SxError(SX_E_DIM_001, "linear-scan: shapes do not fit")
    out = torch.empty(tuple(oshape[:r]), dtype=out_dtype, device=ref.device)
    with torch.cuda.device(ref.device):
        status = lib.sx_linear_scan(
            _DTYPES[ta.dtype], ta.dim(), a_shape, i64_array(ta.stride()), ta.data_ptr(),
            tb.dim(), b_shape, i64_array(tb.stride()), tb.data_ptr(),
            axis, 1 if reverse else 0, _DTYPES[out_dtype], out.data_ptr(), _stream_handle(ref.device))
    _check(status)
    return out


def table_scan(table: torch.Tensor, symbols: torch.Tensor, axis: int = -1, start: int = 0) -> torch.Tensor:
    """Deterministic automaton on the GPU: along ``axis``, reading a symbol
    moves the state to ``table[previous, symbol]``, starting at ``start``. ``table`` is
    ``[states, symbols]``, both int32; returns every state (int32, symbols'
    shape). Out-of-range symbols and reached entries are clamped into range."""
    _require_device_tensor("table", table)
    _require_device_tensor("symbols", symbols)
    if table.dtype != torch.int32 or symbols.dtype != torch.int32:
        raise SxError(SX_E_DIM_002, f"table-scan: table is {table.dtype} and symbols {symbols.dtype}; both must be "
                                    ":i32")
    if table.dim() != 2:
        raise SxError(SX_E_DIM_001, f"table-scan: the table must be [states symbols], got {tuple(table.shape)}")
    if table.device != symbols.device:
        raise SxError(SX_E_UNSUPPORTED, "table-scan: operands on different devices")
    table = table.contiguous()
    lib = load_library()
    out = torch.empty(tuple(symbols.shape), dtype=torch.int32, device=symbols.device)
    with torch.cuda.device(symbols.device):
        status = lib.sx_table_scan(int(table.shape[0]), int(table.shape[1]), table.data_ptr(), symbols.dim(),
                                   i64_array(symbols.shape), i64_array(symbols.stride()), symbols.data_ptr(),
                                   axis, int(start), out.data_ptr(), _stream_handle(symbols.device))
    _check(status)
    return out


def cumsum(x: torch.Tensor, axis: int = 0, reverse: bool = False, out_dtype=None) -> torch.Tensor:
    """Running sum along ``axis`` (from the end when ``reverse``): linear-scan with ``a = 1``."""
    return linear_scan(1.0, x, axis=axis, reverse=reverse, out_dtype=out_dtype)


def matrix_scan_backward(a: torch.Tensor, b_shape, h: torch.Tensor, g: torch.Tensor, axis: int = 0,
                         reverse: bool = False, grad_dtype=None):
    """Gradients ``(grad_a, grad_b)`` of a loss through ``h = matrix_scan(a, b, axis, reverse)``.

    ``h`` is that call's result and ``g`` the loss's gradient with respect to
    it; ``a``, ``h`` and ``g`` share one dtype (f32 or bf16). ``grad_a`` and
    ``grad_b`` have the shapes of ``a`` and ``b`` (summed over broadcast dims)
    and ``grad_dtype`` (default: a's dtype). The adjoint is computed in f32.
    """
    for name, t in (("a", a), ("h", h), ("g", g)):
        _require_device_tensor(name, t)
    if not (a.dtype == h.dtype == g.dtype) or a.dtype not in _DTYPES:
        raise SxError(SX_E_DIM_002, f"matrix-scan gradient: a is {a.dtype}, h {h.dtype} and g {g.dtype}; one float "
                                    "dtype (f32 or bf16) is required")
    if not (a.device == h.device == g.device):
        raise SxError(SX_E_UNSUPPORTED, "matrix-scan gradient: operands on different devices")
    grad_dtype = a.dtype if grad_dtype is None else grad_dtype
    if grad_dtype not in _DTYPES:
        raise SxError(SX_E_DIM_002, f"matrix-scan gradient: grad dtype {grad_dtype} is not f32 or bf16")
    b_shape = tuple(int(d) for d in b_shape)
    if tuple(g.shape) != tuple(h.shape):
        raise SxError(SX_E_DIM_001, f"matrix-scan gradient: g {tuple(g.shape)} and h {tuple(h.shape)} differ")
    lib = load_library()
    if a.dim() >= 2 and not _matrix_dims_contiguous(a):
        a = a.contiguous()
    if g.dim() >= 2 and not _matrix_dims_contiguous(g):
        g = g.contiguous()
    h = h.contiguous()
    a_shape, bs = i64_array(a.shape), i64_array(b_shape)
    ws_bytes = lib.sx_matrix_scan_backward_workspace_bytes(a.dim(), a_shape, len(b_shape), bs, axis,
                                                           _DTYPES[grad_dtype])
    ws = _matrix_workspace(ws_bytes, a.device)
    grad_a = torch.empty(tuple(a.shape), dtype=grad_dtype, device=a.device)
    grad_b = torch.empty(b_shape, dtype=grad_dtype, device=a.device)
    with torch.cuda.device(a.device):
        status = lib.sx_matrix_scan_backward(
            _DTYPES[a.dtype], a.dim(), a_shape, i64_array(a.stride()), a.data_ptr(),
            len(b_shape), bs, h.data_ptr(), i64_array(g.stride()), g.data_ptr(),
            axis, 1 if reverse else 0, _DTYPES[grad_dtype], grad_a.data_ptr(), grad_b.data_ptr(),
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
            _stream_handle(a.device))
    _check(status)
    return grad_a, grad_b


class _MatrixScanFunction(torch.autograd.Function):
    """matrix_scan with its gradient from the library: saves a and the result."""

    @staticmethod
    def forward(ctx, a, b, axis, reverse, out_dtype, projective):
        h = _matrix_scan_forward(a, b, axis, reverse, out_dtype, projective)
        ctx.save_for_backward(a, h)
        ctx.b_shape, ctx.b_dtype, ctx.axis, ctx.reverse = tuple(b.shape), b.dtype, axis, reverse
        ctx.projective = projective
        return h

    @staticmethod
    def backward(ctx, g):
        if ctx.projective:  # "Tensor operations", matrix-scan: the :projective result has no gradient
            raise SxError(SX_E_UNSUPPORTED, "matrix-scan: :projective true has no gradient; differentiating "
                                            "through it is an error")
        a, h = ctx.saved_tensors
        g = g.to(h.dtype)
        # The gradient scan takes a, h and g of one dtype. With an out_dtype other than the
        # operands' one, widen to f32 (exact): a for bf16 operands with an f32 result; h and g
        # for f32 operands with a bf16 result (grad_a then uses the result as rounded to bf16,
        # a relative change of at most 2^-9 per element). Gradients take the operands' dtype.
        if a.dtype != h.dtype:
            if h.dtype == torch.float32:
                a = a.float()
            else:
                h, g = h.float(), g.float()
        grad_a, grad_b = matrix_scan_backward(a, ctx.b_shape, h, g, axis=ctx.axis, reverse=ctx.reverse,
                                              grad_dtype=ctx.b_dtype)
        return grad_a, grad_b, None, None, None, None


def _matrix_dims_contiguous(t: torch.Tensor) -> bool:
    rows, cols = t.shape[-2], t.shape[-1]
    st = t.stride()
    return (cols <= 1 or st[-1] == 1) and (rows <= 1 or cols == 0 or st[-2] == cols)
