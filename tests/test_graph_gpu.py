"""The library's calls inside a captured HIP graph give the eager results.

The bench replays captured graphs, so every kernel path is captured here and
replayed several times, with eager calls of the same workload in between,
and each replay's output is checked against the eager output (and the
oracle). Element-scan kernels are deterministic, so replays must agree bit for
bit. Matrix-scan's look-back may compose from whichever published state it
finds first, which can change the rounding order from run to run; those are
held to the f32 tolerance.
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
        if w.op == "element_scan":
            assert torch.equal(captured, eager)
            assert_element_close(captured, ref)
        else:
            tol = MS_TOL_F32 if w.tensors["a"].dtype == torch.float32 else MS_TOL_BF16
            assert_matrix_close(captured, ref, tol)
            assert_matrix_close(captured, eager.double().cpu().numpy(), MS_TOL_F32)
