"""Seeded synthetic inputs for element-scan, matrix-scan and linear-scan.

This module only draws random numbers (torch CPU generators, fixed seeds);
it holds none of the scans' arithmetic. Tests, the bench and the smoke check
build their inputs here and hand the same host tensors to the HIP library
and to the CPU oracle.

The five standard workloads follow the sizes and distributions below; the
``make_*`` functions take other sizes for the parity tests. linear-scan
(``make_linear``) has no standard workload of its own: it is measured on the
max-plus shape, [64,4096,256] along axis 1.

  tanh-affine       x [4,64,32] ~ N(0,1), decay [4,64,32] ~ U(0,1),
                    initial [4,32] ~ N(0,1), axis 1, forward
  norm-cap          x [8,1024,16,16] ~ N(0,1), decay [8,1024,16,1] ~ U(0.8,1),
                    initial zeros [8,16,16], axis 1, state axis -1, forward
  max-plus          x [64,4096,256] ~ N(0,1), cost [64,4096,256] ~ U(0,0.1),
                    initial [64,256] ~ N(0,1), axis 1, reverse
  matrix f32        a [32,8192,16,16] = 0.9 I + 0.01 N(0,1),
                    b [32,8192,16,1] ~ N(0,1), f32, axis 1, forward
  matrix bf16       a [16,16384,16,16] = 0.9 I + 0.01 N(0,1),
                    b [16,16384,16,16] ~ N(0,1), drawn in f32 and rounded to
                    bf16 (nearest even), axis 1, reverse
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass
class Workload:
    name: str
    op: str                      # "element_scan", "matrix_scan", "matrix_scan_backward", "linear_scan", ...
    tensors: dict                # host tensors, in the order the op takes them
    axis: int = 1
    reverse: bool = False
    body: str | None = None      # element-scan body
    state_axis: int | None = None
    out_dtype: torch.dtype | None = None
    meta: dict = field(default_factory=dict)

    def on(self, device) -> dict:
        return {k: v.to(device) for k, v in self.tensors.items()}

    @property
    def out_shape(self) -> tuple:
        t = self.tensors
        if self.op == "element_scan":
            x = t["x"]
            if self.state_axis is None:
                return tuple(x.shape)
            return tuple(x.shape[:-1]) + (t["initial"].shape[-1],)
        if self.op == "linear_scan":
            return tuple(torch.broadcast_shapes(t["b"].shape, t["a"].shape if "a" in t else ()))
        if self.op == "matrix_scan_backward":  # the outputs are grad_a and grad_b
            return tuple(t["a"].shape)
        if self.op == "element_scan_backward":  # the outputs are the gradients of initial, x and s
            return tuple(t["x"].shape)
        if self.op == "table_scan":
            return tuple(t["symbols"].shape)
        lead = torch.broadcast_shapes(t["a"].shape[:-2], t["b"].shape[:-2])
        return tuple(lead) + tuple(t["b"].shape[-2:])

    @property
    def out_numel(self) -> int:
        n = 1
        for d in self.out_shape:
            n *= d
        return n

    @property
    def out_elem_bytes(self) -> int:
        if self.op in ("element_scan", "table_scan"):
            return 4
        dt = self.out_dtype or self.tensors["b"].dtype
        return torch.tensor([], dtype=dt).element_size()

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: every input read once, the output written once.

        For the matrix-scan gradient the inputs are a, the forward result h and
        its gradient g (g's shape and dtype are h's), and the outputs grad_a and
        grad_b (b's values are not read)."""
        t = self.tensors
        if self.op == "matrix_scan_backward":
            e = t["a"].element_size()
            return (2 * t["a"].numel() + 2 * t["g"].numel() + t["b"].numel()) * e
        if self.op == "element_scan_backward":  # initial, x, s, h, g read; their gradients written (f32)
            return 4 * (2 * (t["initial"].numel() + t["x"].numel() + t["s"].numel()) + 2 * t["g"].numel())
        ins = sum(v.numel() * v.element_size() for v in t.values())
        return ins + self.out_numel * self.out_elem_bytes


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def make_tanh(shape=(4, 64, 32), axis=1, reverse=False, seed=1) -> Workload:
    g = _gen(seed)
    x = torch.randn(shape, generator=g)
    decay = torch.rand(shape, generator=g)
    ax = axis % len(shape)
    initial = torch.randn(shape[:ax] + shape[ax + 1:], generator=g)
    return Workload(f"tanh-affine {list(shape)} axis {axis}{' reverse' if reverse else ''}", "element_scan",
                    {"initial": initial, "x": x, "s": decay}, axis=axis, reverse=reverse, body="tanh_affine")


def make_norm_cap(B=8, T=1024, H=16, n=16, gate_width=1, axis=1, reverse=False, seed=2,
                  zero_initial=True, x_scale=1.0) -> Workload:
    g = _gen(seed)
    x = x_scale * torch.randn((B, T, H, n), generator=g)
    decay = 0.8 + 0.2 * torch.rand((B, T, H, gate_width), generator=g)
    initial = torch.zeros((B, H, n)) if zero_initial else torch.randn((B, H, n), generator=g)
    return Workload(f"norm-cap [{B},{T},{H},{n}] gate width {gate_width}{' reverse' if reverse else ''}",
                    "element_scan", {"initial": initial, "x": x, "s": decay}, axis=axis, reverse=reverse,
                    body="norm_cap", state_axis=-1)


def make_max_plus(shape=(64, 4096, 256), axis=1, reverse=True, seed=3) -> Workload:
    g = _gen(seed)
    x = torch.randn(shape, generator=g)
    cost = 0.1 * torch.rand(shape, generator=g)
    ax = axis % len(shape)
    initial = torch.randn(shape[:ax] + shape[ax + 1:], generator=g)
    return Workload(f"max-plus {list(shape)} axis {axis}{' reverse' if reverse else ''}", "element_scan",
                    {"initial": initial, "x": x, "s": cost}, axis=axis, reverse=reverse, body="max_plus")


def make_matrix(B=32, T=8192, n=16, m=1, dtype=torch.float32, axis=1, reverse=False, seed=4,
                noise=0.01, out_dtype=None, projective=False) -> Workload:
    g = _gen(seed)
    eye = torch.eye(n)
    a = 0.9 * eye + noise * torch.randn((B, T, n, n), generator=g)
    b = torch.randn((B, T, n, m), generator=g)
    a, b = a.to(dtype), b.to(dtype)
    name = f"matrix-scan {str(dtype).replace('torch.', '')} [{B},{T}] n={n} m={m}{' reverse' if reverse else ''}"
    if projective:
        name = name.replace("matrix-scan", "matrix-scan :projective")
    return Workload(name, "matrix_scan", {"a": a, "b": b}, axis=axis, reverse=reverse, out_dtype=out_dtype,
                    meta={"projective": projective})


def make_linear(shape=(64, 4096, 256), axis=1, reverse=False, dtype=torch.float32, a_kind="decay",
                a_shape=None, seed=6, out_dtype=None) -> Workload:
    """linear-scan inputs: b ~ N(0,1) of ``shape``; a by ``a_kind``:

    "decay"  a ~ U(0.9, 1) of ``a_shape`` (default ``shape``; a shape that
             broadcasts against it tests broadcasting),
    "signed" a ~ U(-1, 1) of ``a_shape``,
    "ones"   the number 1 (cumsum),
    "number" the number 0.95.
    Tensors are drawn in f32 and rounded to ``dtype`` (nearest even for bf16).
    """
    g = _gen(seed)
    b = torch.randn(shape, generator=g)
    tensors, meta = {"b": b.to(dtype)}, {}
    ash = tuple(shape) if a_shape is None else tuple(a_shape)
    if a_kind == "decay":
        tensors["a"] = (0.9 + 0.1 * torch.rand(ash, generator=g)).to(dtype)
    elif a_kind == "signed":
        tensors["a"] = (2.0 * torch.rand(ash, generator=g) - 1.0).to(dtype)
    elif a_kind == "ones":
        meta["a_number"] = 1.0
    elif a_kind == "number":
        meta["a_number"] = 0.95
    else:
        raise ValueError(f"unknown a_kind {a_kind!r}")
    what = "cumsum" if a_kind == "ones" else f"linear-scan a {a_kind}"
    name = f"{what} {str(dtype).replace('torch.', '')} {list(shape)} axis {axis}{' reverse' if reverse else ''}"
    if a_shape is not None:
        name += f" a {list(a_shape)}"
    return Workload(name, "linear_scan", tensors, axis=axis, reverse=reverse, out_dtype=out_dtype, meta=meta)


def standard_workloads(which=None) -> list[Workload]:
    """The five standard workloads, in order (or those whose index is in ``which``)."""
    makers = [
        lambda: make_tanh(),
        lambda: make_norm_cap(),
        lambda: make_max_plus(),
        lambda: make_matrix(32, 8192, 16, 1, torch.float32, reverse=False, seed=4),
        lambda: make_matrix(16, 16384, 16, 16, torch.bfloat16, reverse=True, seed=5),
    ]
    idx = range(len(makers)) if which is None else which
    return [makers[i]() for i in idx]


def make_matrix_grad(B=32, T=8192, n=16, m=1, dtype=torch.float32, axis=1, reverse=False, seed=4) -> Workload:
    """The gradient of a matrix workload: a and b as ``make_matrix`` draws them
    (same seed, so the same tensors), and g ~ N(0,1) of the result's shape,
    drawn after them in f32 and rounded to ``dtype``."""
    w = make_matrix(B, T, n, m, dtype, axis=axis, reverse=reverse, seed=seed)
    g = torch.randn(tuple(w.out_shape), generator=_gen(seed + 100)).to(dtype)
    name = "gradient of " + w.name
    return Workload(name, "matrix_scan_backward", {"a": w.tensors["a"], "b": w.tensors["b"], "g": g}, axis=axis,
                    reverse=reverse)


def make_table(kind="parity", B=4096, T=16384, axis=-1, start=0, seed=8) -> Workload:
    """table-scan inputs, int32: "parity" is the pages' example (table
    [[0 1] [1 0]] over bits, 0 and 1 with equal odds); "dfa16" a random
    automaton of 16 states over 16 symbols, table entries and symbols
    uniform."""
    g = _gen(seed)
    if kind == "parity":
        table = torch.tensor([[0, 1], [1, 0]], dtype=torch.int32)
        symbols = torch.randint(0, 2, (B, T), generator=g, dtype=torch.int32)
    elif kind == "dfa16":
        table = torch.randint(0, 16, (16, 16), generator=g, dtype=torch.int32)
        symbols = torch.randint(0, 16, (B, T), generator=g, dtype=torch.int32)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    return Workload(f"table-scan {kind} [{B},{T}]", "table_scan", {"table": table, "symbols": symbols}, axis=axis,
                    meta={"start": start})


def make_element_grad(w: Workload, seed: int) -> Workload:
    """The gradient of an element-scan workload: its tensors and g ~ N(0,1) of
    the result's shape."""
    g = torch.randn(tuple(w.out_shape), generator=_gen(seed))
    return Workload("gradient of " + w.name, "element_scan_backward", dict(w.tensors, g=g), axis=w.axis,
                    reverse=w.reverse, body=w.body, state_axis=w.state_axis)


def extra_workloads() -> list[Workload]:
    """Timed beside the step, not part of it: linear-scan and cumsum on the
    max-plus shape, [64,4096,256] along axis 1, f32; the gradients of the two
    matrix workloads and of the three element-scan workloads; the f32 matrix
    workload with :projective; table-scan on [4096,16384] int32 symbols (the
    parity automaton and a random 16-state one)."""
    return [make_linear(a_kind="decay", seed=6), make_linear(a_kind="ones", seed=7),
            make_matrix_grad(32, 8192, 16, 1, torch.float32, reverse=False, seed=4),
            make_matrix_grad(16, 16384, 16, 16, torch.bfloat16, reverse=True, seed=5),
            make_element_grad(make_tanh(), seed=11), make_element_grad(make_norm_cap(), seed=12),
            make_element_grad(make_max_plus(), seed=13),
            make_matrix(32, 8192, 16, 1, torch.float32, seed=4, projective=True),
            make_table("parity", seed=8), make_table("dfa16", seed=9)]
