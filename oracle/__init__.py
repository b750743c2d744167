"""Plain CPU oracle for element-scan and matrix-scan.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this package. It imports nothing from ``scan_primitives_amd``
and the HIP library never reaches it: the two implementations share no code.

What it computes is the plain definition of each scan, written out as a
serial loop over the scanned axis, one trip at a time, with numpy doing the
arithmetic of one trip for every lane at once. There is no chunking, no
reassociation and no fusion. Arithmetic is float64 by default: inputs given
as float32 or bfloat16 widen to float64 exactly, so the result is the exact
recurrence up to float64 rounding. ``dtype=np.float32`` runs the same loop
in float32 with one rounding per numpy operation (no fused multiply-add);
for the max-plus body, whose subtract and maximum are correctly rounded,
that mode reproduces a serial float32 evaluation bit for bit.

Sources, all from the SexpGPU documentation pages:

* "Nonlinear element scans", introduction: the tanh-affine body
  ``h[t] = tanh(x[t] + decay[t] * h[t-1])`` from ``h[-1] = initial``, every
  output position holding the state after its own trip; the vector state
  (``:state-axis -1``) with the norm-capped body
  ``h[t] = y / max(1, |y|)``, ``y = decay[t] * h[t-1] + x[t]``; ``:reverse``
  running ``h[t] = f(h[t+1], x[t])`` from ``h[time] = initial``; the
  right-to-left max-plus sweep ``max(h - c, x)``.
* "Nonlinear element scans", "Arguments and body": operand shapes, the
  axis rules, and the width-one sequence acting as a gate for the whole
  vector state.
* "Tensor operations", Operations table (matrix-scan row) and the
  "matrix-scan" section: ``h[t] = a[t] @ h[t-1] + b[t]`` from ``h = 0``,
  ``:reverse`` running from the end, NumPy broadcasting of the leading dims,
  ``:axis`` counted among the leading dims, result in ``b``'s shape.
* "Tensor operations", the "matrix-scan" section, on its gradient: the
  same scan run backwards on the transposes of ``a``; and the "gradient"
  section: a gradient has the shape (and dtype) of the tensor it is taken
  with respect to, so a broadcast operand's gradient sums over the dims it
  was broadcast along.
* "Tensor operations", the "table-scan" section: a deterministic automaton
  ``state = table[previous, symbol]`` along one axis from ``start``; an
  out-of-range symbol or reached entry is refused on the CPU and clamped on
  the GPU (both are here; the GPU's is the default).
* "Tensor operations", the "matrix-scan" section, on the prelude's
  ``linear-scan``: the same recurrence over one-by-one matrices, with ``a``
  and ``b`` (tensors or plain numbers) broadcast together; ``cumsum`` is
  defined through it, so it is the linear scan with ``a = 1``.

Readings where the pages leave a point open (each is listed with its reason
in the design notes of the repository):

* matrix-scan ``:reverse`` is ``h[t] = a[t] @ h[t+1] + b[t]`` from
  ``h[T] = 0``: the step at position t uses position t's operands, as the
  reverse element scan does, so the result equals flipping, scanning forward
  and flipping back.
* the result shape of matrix-scan is the broadcast leading shape followed
  by ``[n, m]``; this is ``b``'s shape whenever ``b`` already has the full
  leading shape.
* a matrix-scan over an axis of length zero returns an empty result; an
  element scan over one is refused, since the pages require length >= 1.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, inverse problems, invariants the pages state, and worked
examples under ``tests/golden/``.
"""

from __future__ import annotations

import numpy as np

__all__ = ["element_scan", "element_scan_vjp", "matrix_scan", "matrix_scan_projective", "matrix_scan_vjp",
           "linear_scan", "cumsum", "table_scan", "BODIES"]


# --- element-scan bodies ----------------------------------------------------
# Each body maps (incoming state, sequence values at this trip) to the new
# state, in the operation order the page writes it.


def _tanh_affine(h, x, a):
    # "Nonlinear element scans", introduction: (tanh (+ x (* a h)))
    return np.tanh(x + a * h)


def _norm_cap(h, x, a):
    # "Nonlinear element scans", introduction, vector state:
    # y = (+ (* a h) x); y / (maximum 1.0 (sqrt (sum (* y y) :axes [-1])))
    y = a * h + x
    norm = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
    return y / np.maximum(1.0, norm)


def _max_plus(h, x, c):
    # "Nonlinear element scans", introduction, :reverse: (maximum (- h c) x)
    return np.maximum(h - c, x)


BODIES = {
    "tanh_affine": _tanh_affine,
    "norm_cap": _norm_cap,
    "max_plus": _max_plus,
}

# Bodies that reduce over the state vector need a vector state: by the page's
# "Arguments and body" section, a reduction over components has nothing to
# reduce when the state is a single number.
_REDUCING = {"norm_cap"}


def element_scan(body, initial, sequences, axis=0, state_axis=None,
                 reverse=False, dtype=np.float64):
    """Run an element scan the plain way: one trip at a time, all lanes at once.

    ``body`` is one of ``BODIES``; ``sequences`` is the list of the body's
    sequence arguments in page order (``[x, decay]`` or ``[x, cost]``).
    ``state_axis`` is ``None`` (scalar state) or ``-1`` (the last axis
    holds the components of a vector state). Returns an array of the sequences' shape
    (with the last axis equal to the state's width under ``state_axis``).

    Follows "Nonlinear element scans", introduction and "Arguments and body".
    """
    step = BODIES[body]
    seqs = [np.asarray(s, dtype=dtype) for s in sequences]
    h = np.array(initial, dtype=dtype, copy=True)
    if not seqs:
        raise ValueError("element_scan: sequences must be nonempty")
    rank = seqs[0].ndim
    if rank < 1:
        raise ValueError("element_scan: sequences need at least one axis")
    ax = axis + rank if axis < 0 else axis
    if not 0 <= ax < rank:
        raise ValueError(f"element_scan: axis {axis} out of range for rank {rank}")

    if state_axis is None:
        if body in _REDUCING:
            raise ValueError(f"element_scan: body {body!r} reduces, so it needs a vector state")
        shape = seqs[0].shape
        for s in seqs:
            if s.shape != shape:
                raise ValueError("element_scan: sequences must share one shape")
    else:
        if state_axis not in (-1, rank - 1):
            raise ValueError("element_scan: the state axis is the last axis")
        if ax == rank - 1:
            raise ValueError("element_scan: the scan axis cannot be the state axis")
        n = h.shape[-1]
        widened = []
        for s in seqs:
            if s.shape[:-1] != seqs[0].shape[:-1] or s.shape[-1] not in (1, n):
                raise ValueError("element_scan: a sequence's last axis is 1 or the state width")
            # A width-one sequence broadcasts over the whole state vector.
            widened.append(np.broadcast_to(s, s.shape[:-1] + (n,)))
        seqs = widened
        shape = seqs[0].shape

    expected_init = shape[:ax] + shape[ax + 1:]
    if h.shape != expected_init:
        raise ValueError(f"element_scan: initial has shape {h.shape}, expected {expected_init}")
    T = shape[ax]
    if T < 1:
        raise ValueError("element_scan: the scan axis has length at least one")

    # Time-major views: seq_t[t] is every lane's value at trip t.
    seq_t = [np.moveaxis(s, ax, 0) for s in seqs]
    out = np.empty((T,) + expected_init, dtype=dtype)
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        h = step(h, *(s[t] for s in seq_t))
        out[t] = h  # the state reached at position t is stored at t
    return np.moveaxis(out, 0, ax)


# --- element-scan gradients ------------------------------------------------
# Each body's vector-Jacobian product at one trip: given the state it started
# from, its sequence values, the state it produced and the adjoint lam of that
# state, the adjoints of (incoming state, x, second sequence). Written from the
# chain rule on the body as the page writes it.


def _tanh_affine_vjp(h_prev, x, a, h, lam, branch):
    # h = tanh(z), z = x + a h_prev; dtanh/dz = 1 - h^2
    dz = lam * (1.0 - h * h)
    return a * dz, dz, dz * h_prev


def _norm_cap_vjp(h_prev, x, a, h, lam, capped):
    # y = a h_prev + x; h = y when |y| <= 1, else y / |y|, whose Jacobian is
    # (I - h h^T) / |y| (symmetric)
    y = a * h_prev + x
    r = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
    dy_capped = (lam - h * np.sum(h * lam, axis=-1, keepdims=True)) / np.where(capped, r, 1.0)
    dy = np.where(capped, dy_capped, lam)
    return a * dy, dy, dy * h_prev


def _max_plus_vjp(h_prev, x, c, h, lam, x_won):
    # h = max(h_prev - c, x): the adjoint goes to the branch that gave h
    zero = np.zeros_like(lam)
    return np.where(x_won, zero, lam), np.where(x_won, lam, zero), np.where(x_won, zero, -lam)


_VJP = {"tanh_affine": _tanh_affine_vjp, "norm_cap": _norm_cap_vjp, "max_plus": _max_plus_vjp}


def _branches(body, h_prev32, x32, s32):
    """Which branch each lane's trip took, decided in float32 from the float32
    forward pass (the precision the scan computes in): for max-plus, x wins
    when x >= h_prev - c (ties go to x); for norm-cap, the cap acts when
    |y|^2 > 1 with y = a h_prev + x. None for tanh-affine, which has none."""
    if body == "max_plus":
        return x32 >= (h_prev32 - s32)
    if body == "norm_cap":
        y = s32 * h_prev32 + x32
        return np.sum(y * y, axis=-1, keepdims=True, dtype=np.float32) > np.float32(1.0)
    return None


def element_scan_vjp(body, initial, sequences, g, axis=0, state_axis=None, reverse=False, dtype=np.float64):
    """Gradient of ``sum(g * element_scan(body, initial, sequences, ...))``.

    Returns ``(grad_initial, [grad_x, grad_s])`` in the shapes of ``initial``
    and of each sequence (a width-one sequence under a vector state gets the
    sum over the state of its broadcast gradient). With lam[t] the adjoint of
    the state after trip t and s / p the trips after / before t in scan order,

      lam[t] = g[t] + (adjoint of the incoming state from trip s's VJP)

    and each trip's VJP gives its sequences' gradients; trip 0's incoming
    adjoint is grad_initial. Values are computed in ``dtype`` (float64 by
    default); branch decisions (max-plus's winner, norm-cap's cap) are taken
    in float32 from a float32 forward pass, as the scan computes them.

    Follows "Nonlinear element scans", introduction (the bodies) and the
    chain rule; the pages' gradient section gives each gradient its tensor's
    shape.
    """
    seqs_in = [np.asarray(s_, dtype=dtype) for s_ in sequences]
    init = np.asarray(initial, dtype=dtype)
    h = element_scan(body, init, seqs_in, axis=axis, state_axis=state_axis, reverse=reverse, dtype=dtype)
    h32 = element_scan(body, np.asarray(initial, dtype=np.float32), [np.asarray(s_, dtype=np.float32) for s_ in sequences],
                       axis=axis, state_axis=state_axis, reverse=reverse, dtype=np.float32)
    g = np.asarray(g, dtype=dtype)
    if g.shape != h.shape:
        raise ValueError(f"element_scan_vjp: g has shape {g.shape}, the result has {h.shape}")
    rank = h.ndim
    ax = axis + rank if axis < 0 else axis
    n = h.shape[-1]
    wide = [np.broadcast_to(s_, s_.shape[:-1] + (n,)) if state_axis is not None else s_ for s_ in seqs_in]
    wide32 = [w.astype(np.float32) for w in wide]
    x_t, s_t = (np.moveaxis(w, ax, 0) for w in wide)
    x32_t, s32_t = (np.moveaxis(w, ax, 0) for w in wide32)
    h_t, h32_t, g_t = np.moveaxis(h, ax, 0), np.moveaxis(h32, ax, 0), np.moveaxis(g, ax, 0)
    T = h_t.shape[0]
    order = list(range(T - 1, -1, -1)) if reverse else list(range(T))  # scan order
    vjp = _VJP[body]
    gx = np.zeros(x_t.shape, dtype=dtype)
    gs = np.zeros(s_t.shape, dtype=dtype)
    from_later = np.zeros(h_t.shape[1:], dtype=dtype)  # adjoint reaching the state from the trip after
    g_init = None
    for i in range(T - 1, -1, -1):
        t = order[i]
        lam = g_t[t] + from_later
        if i > 0:
            p = order[i - 1]
            h_prev, h_prev32 = h_t[p], h32_t[p]
        else:
            h_prev, h_prev32 = init, np.asarray(initial, dtype=np.float32)
        branch = _branches(body, h_prev32, x32_t[t], s32_t[t])
        d_prev, gx[t], gs[t] = vjp(h_prev, x_t[t], s_t[t], h_t[t], lam, branch)
        if i > 0:
            from_later = d_prev
        else:
            g_init = d_prev
    grads = []
    for gt, s_ in zip((gx, gs), seqs_in):
        full = np.moveaxis(gt, 0, ax)
        if state_axis is not None and s_.shape[-1] == 1 and n != 1:
            full = np.sum(full, axis=-1, keepdims=True)
        grads.append(full.reshape(s_.shape))
    return g_init.reshape(init.shape), grads


def matrix_scan(a, b, axis=0, reverse=False, dtype=np.float64):
    """Run a matrix scan the plain way: one matrix product per step.

    ``a`` is ``[..., n, n]`` and ``b`` ``[..., n, m]``; the leading dims
    broadcast (NumPy rules) and ``axis`` counts among them. Forward:
    ``h[t] = a[t] @ h[t-1] + b[t]`` from ``h[-1] = 0``. Reverse:
    ``h[t] = a[t] @ h[t+1] + b[t]`` from ``h[T] = 0``.

    Follows "Tensor operations", Operations table (matrix-scan row) and the
    "matrix-scan" section.
    """
    a = np.asarray(a, dtype=dtype)
    b = np.asarray(b, dtype=dtype)
    if a.ndim < 2 or b.ndim < 2:
        raise ValueError("matrix_scan: a and b need two matrix dims")
    n = a.shape[-1]
    if a.shape[-2] != n or b.shape[-2] != n:
        raise ValueError("matrix_scan: a must be [.., n, n] and b [.., n, m]")
    if n > 16:
        raise ValueError("matrix_scan: n is at most 16")
    m = b.shape[-1]
    lead = np.broadcast_shapes(a.shape[:-2], b.shape[:-2])
    if len(lead) < 1:
        raise ValueError("matrix_scan: the scan axis is one of the leading dims")
    ax = axis + len(lead) if axis < 0 else axis
    if not 0 <= ax < len(lead):
        raise ValueError(f"matrix_scan: axis {axis} out of range for leading rank {len(lead)}")
    a = np.broadcast_to(a, lead + (n, n))
    b = np.broadcast_to(b, lead + (n, m))

    a_t = np.moveaxis(a, ax, 0)
    b_t = np.moveaxis(b, ax, 0)
    T = lead[ax]
    out = np.empty((T,) + b_t.shape[1:], dtype=dtype)
    h = np.zeros(b_t.shape[1:], dtype=dtype)
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        h = a_t[t] @ h + b_t[t]
        out[t] = h
    return np.moveaxis(out, 0, ax)


def matrix_scan_projective(a, b, axis=0, reverse=False, dtype=np.float64):
    """matrix-scan with ``:projective true``: the plain way, one step at a time.

    A running product P of the a's starts at the identity. Each step (in scan
    order) replaces P by ``a[t] @ P``, takes m = the largest magnitude of its
    entries, divides P by m, and sets ``h = (a[t] @ h + b[t]) / m`` (h from
    0). A product whose entries are all zero divides by 1. Operands, axis,
    broadcasting and result shape are those of ``matrix_scan``.

    Follows "Tensor operations", the "matrix-scan" section (``:projective``).
    """
    a = np.asarray(a, dtype=dtype)
    b = np.asarray(b, dtype=dtype)
    if a.ndim < 2 or b.ndim < 2:
        raise ValueError("matrix_scan_projective: a and b need two matrix dims")
    n = a.shape[-1]
    if a.shape[-2] != n or b.shape[-2] != n or n > 16:
        raise ValueError("matrix_scan_projective: a must be [.., n, n] and b [.., n, m] with n <= 16")
    m = b.shape[-1]
    lead = np.broadcast_shapes(a.shape[:-2], b.shape[:-2])
    if len(lead) < 1:
        raise ValueError("matrix_scan_projective: the scan axis is one of the leading dims")
    ax = axis + len(lead) if axis < 0 else axis
    if not 0 <= ax < len(lead):
        raise ValueError(f"matrix_scan_projective: axis {axis} out of range for leading rank {len(lead)}")
    a_t = np.moveaxis(np.broadcast_to(a, lead + (n, n)), ax, 0)
    b_t = np.moveaxis(np.broadcast_to(b, lead + (n, m)), ax, 0)
    T = lead[ax]
    out = np.empty((T,) + b_t.shape[1:], dtype=dtype)
    h = np.zeros(b_t.shape[1:], dtype=dtype)
    P = np.broadcast_to(np.eye(n, dtype=dtype), a_t.shape[1:]).copy()
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        P = a_t[t] @ P
        big = np.max(np.abs(P), axis=(-2, -1), keepdims=True)
        big = np.where(big > 0, big, 1.0)
        P = P / big
        h = (a_t[t] @ h + b_t[t]) / big
        out[t] = h
    return np.moveaxis(out, 0, ax)


def _sum_to_shape(x, shape):
    """Sum ``x`` over the dims that broadcasting ``shape`` up to ``x.shape`` added or stretched."""
    extra = x.ndim - len(shape)
    if extra:
        x = x.sum(axis=tuple(range(extra)))
    stretched = tuple(i for i, d in enumerate(shape) if d == 1 and x.shape[i] != 1)
    if stretched:
        x = x.sum(axis=stretched, keepdims=True)
    return x.reshape(shape)


def matrix_scan_vjp(a, b, g, axis=0, reverse=False, dtype=np.float64):
    """Gradient of ``sum(g * matrix_scan(a, b))`` with respect to ``a`` and ``b``.

    Returns ``(grad_a, grad_b)`` in the shapes of ``a`` and ``b``; ``g`` has
    the result's shape. Chain rule through one step ``h[t] = a[t] @ h[p] + b[t]``
    (``p`` the step before in scan order, ``h[p] = 0`` at the first step):
    with ``lam[t]`` the total derivative with respect to ``h[t]``,

      lam[t]    = g[t] + a[s]^T @ lam[s]     (``s`` the step after t in scan
                                             order; no second term at the last)
      grad_b[t] = lam[t]
      grad_a[t] = lam[t] @ h[p]^T            (zero at the first step)

    so ``lam`` is the same scan run in the other direction on the transposes
    of ``a``, one step shifted. Written as a plain loop over the steps, last
    to first, after the forward scan above has produced ``h``.

    Follows "Tensor operations", the "matrix-scan" section (its gradient) and
    the "gradient" section (a gradient takes its operand's shape).
    """
    a = np.asarray(a, dtype=dtype)
    b = np.asarray(b, dtype=dtype)
    g = np.asarray(g, dtype=dtype)
    h = matrix_scan(a, b, axis=axis, reverse=reverse, dtype=dtype)  # validates the operands
    if g.shape != h.shape:
        raise ValueError(f"matrix_scan_vjp: g has shape {g.shape}, the result has {h.shape}")
    n, m = a.shape[-1], b.shape[-1]
    lead = h.shape[:-2]
    ax = axis + len(lead) if axis < 0 else axis
    a_t = np.moveaxis(np.broadcast_to(a, lead + (n, n)), ax, 0)
    g_t = np.moveaxis(g, ax, 0)
    h_t = np.moveaxis(h, ax, 0)
    T = lead[ax]
    lam = np.empty(g_t.shape, dtype=dtype)
    grad_a = np.zeros(a_t.shape, dtype=dtype)
    order = list(range(T - 1, -1, -1)) if reverse else list(range(T))  # scan order of the forward pass
    from_later = np.zeros(g_t.shape[1:], dtype=dtype)  # a[s]^T @ lam[s], s the step after
    for i in range(T - 1, -1, -1):
        t = order[i]
        lam[t] = g_t[t] + from_later
        if i > 0:
            p = order[i - 1]
            grad_a[t] = lam[t] @ np.swapaxes(h_t[p], -1, -2)
        from_later = np.swapaxes(a_t[t], -1, -2) @ lam[t]
    grad_a = _sum_to_shape(np.moveaxis(grad_a, 0, ax), a.shape)
    grad_b = _sum_to_shape(np.moveaxis(lam, 0, ax), b.shape)
    return grad_a, grad_b


def table_scan(table, symbols, axis=-1, start=0, clamp=True):
    """Run a deterministic automaton the plain way, one symbol at a time.

    ``table`` is ``[states, symbols]`` of integers and ``symbols`` any shape of
    integers; along ``axis`` (the last by default) each symbol moves the
    state to ``table[previous, symbol]``, starting at ``start`` (0 by default).
    Returns every state, in ``symbols``' shape (int32).

    Out-of-range values: with ``clamp`` (the GPU reading) a symbol is clamped
    into ``[0, symbols)`` and a table entry the run reaches into
    ``[0, states)``; without it, either raises ``ValueError`` (the CPU
    reading).

    Follows "Tensor operations", the "table-scan" section.
    """
    table = np.asarray(table)
    symbols = np.asarray(symbols)
    if not (np.issubdtype(table.dtype, np.integer) and np.issubdtype(symbols.dtype, np.integer)):
        raise TypeError("table_scan: table and symbols are integers")
    if table.ndim != 2 or table.shape[0] < 1 or table.shape[1] < 1:
        raise ValueError("table_scan: the table is [states, symbols] with at least one of each")
    n_states, n_syms = table.shape
    if symbols.ndim < 1:
        raise ValueError("table_scan: symbols need at least one axis")
    ax = axis + symbols.ndim if axis < 0 else axis
    if not 0 <= ax < symbols.ndim:
        raise ValueError(f"table_scan: axis {axis} out of range for rank {symbols.ndim}")
    if not 0 <= start < n_states:
        raise ValueError(f"table_scan: start {start} is not a state")
    sym_t = np.moveaxis(symbols, ax, 0).astype(np.int64)
    out = np.empty(sym_t.shape, dtype=np.int32)
    state = np.full(sym_t.shape[1:], start, dtype=np.int64)
    for t in range(sym_t.shape[0]):
        x = sym_t[t]
        if clamp:
            x = np.clip(x, 0, n_syms - 1)
        elif np.any((x < 0) | (x >= n_syms)):
            raise ValueError("table_scan: a symbol is outside [0, symbols)")
        state = table[state, x].astype(np.int64)
        if clamp:
            state = np.clip(state, 0, n_states - 1)
        elif np.any((state < 0) | (state >= n_states)):
            raise ValueError("table_scan: the run reached a table entry outside [0, states)")
        out[t] = state
    return np.moveaxis(out, 0, ax)


def linear_scan(a, b, axis=0, reverse=False, dtype=np.float64):
    """Run a linear scan the plain way: one multiply-add per step, every
    position of the broadcast shape outside ``axis`` its own recurrence.

    ``a`` and ``b`` are numbers or arrays broadcast (NumPy rules) to one
    shape, in which ``axis`` counts. Forward: ``h[t] = a[t] * h[t-1] + b[t]``
    from ``h[-1] = 0``; reverse: ``h[t] = a[t] * h[t+1] + b[t]`` from
    ``h[T] = 0``. The result has the broadcast shape.

    Follows "Tensor operations", the "matrix-scan" section: the matrix
    recurrence over one-by-one matrices, operands broadcast to one shape.
    """
    a = np.asarray(a, dtype=dtype)
    b = np.asarray(b, dtype=dtype)
    shape = np.broadcast_shapes(a.shape, b.shape)
    if len(shape) < 1:
        raise ValueError("linear_scan: the operands broadcast to a number; there is no axis to scan")
    ax = axis + len(shape) if axis < 0 else axis
    if not 0 <= ax < len(shape):
        raise ValueError(f"linear_scan: axis {axis} out of range for rank {len(shape)}")
    a_t = np.moveaxis(np.broadcast_to(a, shape), ax, 0)
    b_t = np.moveaxis(np.broadcast_to(b, shape), ax, 0)
    T = shape[ax]
    out = np.empty((T,) + b_t.shape[1:], dtype=dtype)
    h = np.zeros(b_t.shape[1:], dtype=dtype)
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        h = a_t[t] * h + b_t[t]
        out[t] = h
    return np.moveaxis(out, 0, ax)


def cumsum(x, axis=0, reverse=False, dtype=np.float64):
    """Running sum along ``axis`` (from the end when ``reverse``): the linear
    scan with ``a = 1``, as the "matrix-scan" section builds cumsum on it."""
    return linear_scan(1.0, x, axis=axis, reverse=reverse, dtype=dtype)
