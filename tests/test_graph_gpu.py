"""The library's calls inside a captured HIP graph give the eager results.

The bench replays captured graphs, so every kernel path is captured here (the
forward scans, and the calls timed beside the step: linear-scan, cumsum,
table-scan, :projective and the gradients) and
replayed several times, with eager calls of the same workload in between,
and each replay's output is checked against the eager output (and the
oracle). Every kernel here is deterministic (matrix-scan's look-back included:
whichever published state it starts from, it applies the same unit maps in
scan order with the same instructions; tests/test_determinism_gpu.py), so
replays must agree with the eager call bit for bit.
"""

import pytest
import torch

import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W
from tests.helpers import MS_TOL_BF16, MS_TOL_F32, assert_element_close, assert_matrix_close, run_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = {
    "tanh lane kernel": lambda: W.make_tanh((3, 70, 40), seed=300),
    "norm-cap row kernel": lambda: W.make_norm_cap(2, 17, 5, 16, seed=301),
    "norm-cap chunked": lambda: W.make_norm_cap(2, 300, 5, 16, seed=302, zero_initial=False),
    "max-plus lane kernel": lambda: W.make_max_plus((3, 200, 19), seed=303),
    "max-plus slab kernel": lambda: W.make_max_plus((33, 600, 256), seed=304),
    "matrix f32 m=1": lambda: W.make_matrix(3, 300, 16, 1, torch.float32, seed=305),
    "matrix bf16 m=16 reverse": lambda: W.make_matrix(2, 300, 16, 16, torch.bfloat16, reverse=True, seed=306),
}


def _call(w, t):
    if w.op == "element_scan":
        return sx.element_scan(w.body, t["initial"], [t["x"], t["s"]], axis=w.axis, state_axis=w.state_axis,
                               reverse=w.reverse)
    return sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse, out_dtype=w.out_dtype)


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replay_matches_eager(name):
    w = CASES[name]()
    print(f"\n[case] graph replay: {w.name}", flush=True)
    t = w.on(DEV)  # inputs staged before capture: only the library call is captured
    eager = _call(w, t)
    torch.cuda.synchronize()
    ref = run_oracle(w)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = _call(w, t)
    for _ in range(3):
        _call(w, t)  # eager work between replays
        torch.cuda.synchronize()
        captured.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(captured, eager)
        if w.op == "element_scan":
            assert_element_close(captured, ref)
        else:
            tol = MS_TOL_F32 if w.tensors["a"].dtype == torch.float32 else MS_TOL_BF16
            assert_matrix_close(captured, ref, tol)


# The calls timed beside the step: each returns a tensor or a tuple of tensors, and every replay must
# give the eager call's bits.
def _other_cases():
    nc = W.make_norm_cap(2, 600, 5, 16, seed=311)
    mp = W.make_max_plus((33, 600, 256), seed=312)
    return {
        "linear-scan slab": W.make_linear((33, 600, 256), a_kind="decay", seed=313),
        "cumsum": W.make_linear((9, 700, 64), a_kind="ones", seed=314),
        "cumsum slab": W.make_linear((2, 777, 4163), a_kind="ones", reverse=True, seed=322),
        "table-scan parity": W.make_table("parity", 64, 3000, seed=315),
        "table-scan 16 states": W.make_table("dfa16", 64, 3000, seed=316),
        "projective f32": W.make_matrix(3, 700, 16, 1, torch.float32, seed=317, projective=True),
        "matrix gradient f32 m=1": W.make_matrix_grad(3, 400, 16, 1, torch.float32, seed=318),
        "matrix gradient bf16 m=16": W.make_matrix_grad(2, 300, 16, 16, torch.bfloat16, reverse=True, seed=319),
        "norm-cap gradient split": W.make_element_grad(nc, seed=320),
        "max-plus gradient slab": W.make_element_grad(mp, seed=321),
    }


def _call_other(w, t, h):
    if w.op == "linear_scan":
        a = t["a"] if "a" in t else w.meta["a_number"]
        return (sx.linear_scan(a, t["b"], axis=w.axis, reverse=w.reverse, out_dtype=w.out_dtype),)
    if w.op == "table_scan":
        return (sx.table_scan(t["table"], t["symbols"], axis=w.axis, start=w.meta.get("start", 0)),)
    if w.op == "matrix_scan":
        return (sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse, projective=True),)
    if w.op == "matrix_scan_backward":
        ga, gb = sx.matrix_scan_backward(t["a"], tuple(t["b"].shape), h, t["g"], axis=w.axis, reverse=w.reverse)
        return ga, gb
    gi, (gx, gs) = sx.element_scan_backward(w.body, t["initial"], [t["x"], t["s"]], h, t["g"], axis=w.axis,
                                            state_axis=w.state_axis, reverse=w.reverse)
    return gi, gx, gs


def _forward_h(w, t):
    if w.op == "matrix_scan_backward":
        return sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse)
    if w.op == "element_scan_backward":
        return sx.element_scan(w.body, t["initial"], [t["x"], t["s"]], axis=w.axis, state_axis=w.state_axis,
                               reverse=w.reverse)
    return None


@pytest.mark.parametrize("name", sorted(_other_cases()))
def test_graph_replay_other_calls(name):
    w = _other_cases()[name]
    print(f"\n[case] graph replay: {w.name}", flush=True)
    t = w.on(DEV)
    h = _forward_h(w, t)  # the forward result a gradient takes, computed before capture
    eager = _call_other(w, t, h)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = _call_other(w, t, h)
    for _ in range(3):
        _call_other(w, t, h)  # eager work between replays
        torch.cuda.synchronize()
        for c in captured:
            c.zero_()
        g.replay()
        torch.cuda.synchronize()
        for c, e in zip(captured, eager):
            assert torch.equal(c, e)
