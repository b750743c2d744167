"""Repeated calls give the same bits.

Element-scan, linear-scan and table-scan kernels fix every rounding order in
code. Matrix-scan's look-back may start from any published leaving state of an
earlier unit, but the result does not depend on which: a unit's published
leaving state is its map applied to its entering state (one MFMA sequence), and
a look-back applies the published maps of the units in between to the state it
starts from, one at a time, in scan order, with that same sequence. By
induction over the units, every route to a unit's entering state performs the
same operations on the same values as the route through every unit in turn,
so the entering state (and everything formed from it) has the same bits
whichever route is taken. This file checks that across calls whose timing is
disturbed (other calls, a large fill between them), for the pipelined and the
per-unit kernels, :projective and the gradients, including the matrix-scan
workloads at full size.
"""

import pytest
import torch

import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CALLS = 6


def _disturb(i):
    # other work between calls: another matrix-scan shape (the binding's shared
    # workspace moves to a new epoch) or a large fill that changes the timing
    if i % 2 == 0:
        w = W.make_matrix(2, 500 + 37 * i, 16, 1, torch.float32, seed=900 + i)
        t = w.on(DEV)
        sx.matrix_scan(t["a"], t["b"], axis=w.axis)
    else:
        torch.empty(32 << 20, device=DEV).fill_(float(i))


FORWARD = {
    "f32 m=1 [32,8192] (standard workload)": lambda: W.make_matrix(32, 8192, 16, 1, torch.float32, seed=4),
    "bf16 m=16 [16,16384] reverse (standard workload)": lambda: W.make_matrix(16, 16384, 16, 16, torch.bfloat16,
                                                                              reverse=True, seed=5),
    "f32 m=1 [3,3001] ragged": lambda: W.make_matrix(3, 3001, 16, 1, torch.float32, seed=41),
    "f32 m=4 [5,3000] per-unit kernel": lambda: W.make_matrix(5, 3000, 16, 4, torch.float32, seed=42),
    "f32 m=16 [4,5000] per-unit kernel": lambda: W.make_matrix(4, 5000, 16, 16, torch.float32, seed=43),
    "bf16 m=32 [4,5000] pipelined": lambda: W.make_matrix(4, 5000, 16, 32, torch.bfloat16, seed=44),
    "f32 n=7 m=3 [6,2000] per-unit kernel": lambda: W.make_matrix(6, 2000, 7, 3, torch.float32, seed=45),
    "f32 m=1 [8,4000] :projective": lambda: W.make_matrix(8, 4000, 16, 1, torch.float32, seed=46, projective=True),
}


@pytest.mark.parametrize("name", sorted(FORWARD))
def test_matrix_scan_repeats_bit_for_bit(name):
    w = FORWARD[name]()
    print(f"\n[case] determinism: {w.name}", flush=True)
    t = w.on(DEV)
    proj = bool(w.meta.get("projective", False))
    first = sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse, projective=proj)
    for i in range(CALLS):
        _disturb(i)
        again = sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse, projective=proj)
        torch.cuda.synchronize()
        assert torch.equal(again, first), f"call {i + 1} differs from the first"


GRADS = {
    "f32 m=1 [8,3000]": lambda: W.make_matrix_grad(8, 3000, 16, 1, torch.float32, seed=51),
    "bf16 m=16 [4,4000] reverse": lambda: W.make_matrix_grad(4, 4000, 16, 16, torch.bfloat16, reverse=True, seed=52),
    "f32 m=4 [3,2000]": lambda: W.make_matrix_grad(3, 2000, 16, 4, torch.float32, seed=53),
}


@pytest.mark.parametrize("name", sorted(GRADS))
def test_matrix_scan_gradient_repeats_bit_for_bit(name):
    w = GRADS[name]()
    print(f"\n[case] determinism: {w.name}", flush=True)
    t = w.on(DEV)
    h = sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse)
    ga0, gb0 = sx.matrix_scan_backward(t["a"], tuple(t["b"].shape), h, t["g"], axis=w.axis, reverse=w.reverse)
    for i in range(CALLS):
        _disturb(i)
        ga, gb = sx.matrix_scan_backward(t["a"], tuple(t["b"].shape), h, t["g"], axis=w.axis, reverse=w.reverse)
        torch.cuda.synchronize()
        assert torch.equal(ga, ga0) and torch.equal(gb, gb0), f"call {i + 1} differs from the first"


ELEMENT = {
    "max-plus [64,4096,256] reverse (standard workload)": lambda: W.make_max_plus(seed=3),
    "norm-cap [8,1024,16,16] (standard workload)": lambda: W.make_norm_cap(seed=2),
    "linear-scan [33,600,256]": lambda: W.make_linear((33, 600, 256), a_kind="decay", seed=61),
}


@pytest.mark.parametrize("name", sorted(ELEMENT))
def test_element_and_linear_scan_repeat_bit_for_bit(name):
    w = ELEMENT[name]()
    print(f"\n[case] determinism: {w.name}", flush=True)
    t = w.on(DEV)

    def call():
        if w.op == "linear_scan":
            return sx.linear_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse)
        return sx.element_scan(w.body, t["initial"], [t["x"], t["s"]], axis=w.axis, state_axis=w.state_axis,
                               reverse=w.reverse)

    first = call()
    for i in range(3):
        _disturb(i)
        again = call()
        torch.cuda.synchronize()
        assert torch.equal(again, first), f"call {i + 1} differs from the first"
