"""Parity of the HIP table-scan with the CPU oracle: bit-exact (integer states).

The oracle (``oracle.table_scan``, clamping as the pages' GPU backend does)
runs the automaton one symbol at a time. Cases cover the wave kernel (tables
of at most 16 states and 2048 symbols, maps of 8 or 16 bytes: full slabs of 1024 steps, a ragged tail, one step,
strided and non-last axes, clamped symbols and entries, every start) and the
serial kernel (larger tables, in LDS or not), and the two measured workloads
at full size on sampled sequences (a sequence is an exact sub-problem).
"""

import numpy as np
import pytest
import torch

import oracle
import scan_primitives_amd as sx
from scan_primitives_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(table, symbols, axis=-1, start=0):
    print(f"\n[case] table-scan table {tuple(table.shape)} symbols {tuple(symbols.shape)} axis {axis} start {start}",
          flush=True)
    got = sx.table_scan(table.to(DEV), symbols.to(DEV), axis=axis, start=start)
    torch.cuda.synchronize()
    ref = oracle.table_scan(table.numpy(), symbols.numpy(), axis=axis, start=start)
    g = got.cpu().numpy()
    assert g.dtype == np.int32 and g.shape == ref.shape
    bad = np.argwhere(g != ref)
    assert bad.size == 0, f"{len(bad)} states differ; first at {tuple(bad[0])}: got {g[tuple(bad[0])]}, " \
                          f"ref {ref[tuple(bad[0])]}"


def _rand(states, nsym, shape, seed, lo=None, hi=None):
    g = torch.Generator().manual_seed(seed)
    table = torch.randint(0 if lo is None else lo, states if hi is None else hi, (states, nsym), generator=g,
                          dtype=torch.int32)
    symbols = torch.randint(0, nsym, shape, generator=g, dtype=torch.int32)
    return table, symbols


@pytest.mark.parametrize("states,nsym", [(2, 2), (3, 5), (8, 8), (9, 3), (16, 16), (16, 300), (7, 2048)])
@pytest.mark.parametrize("shape", [(5, 3000), (64, 1024), (3, 1), (130, 2049), (1, 777)])
def test_wave_kernel(states, nsym, shape):
    table, symbols = _rand(states, nsym, shape, seed=301 + states + nsym + shape[1])
    _check(table, symbols)


def test_parity_example():
    g = torch.Generator().manual_seed(302)
    bits = torch.randint(0, 2, (9, 5000), generator=g, dtype=torch.int32)
    table = torch.tensor([[0, 1], [1, 0]], dtype=torch.int32)
    got = sx.table_scan(table.to(DEV), bits.to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, np.cumsum(bits.numpy(), axis=-1) % 2)


@pytest.mark.parametrize("start", [0, 4, 9])
def test_every_start(start):
    table, symbols = _rand(10, 6, (20, 1500), seed=303)
    _check(table, symbols, start=start)


@pytest.mark.parametrize("axis", [0, 1, -3])
def test_other_axes_and_strides(axis):
    table, symbols = _rand(5, 3, (40, 33, 7), seed=304)
    _check(table, symbols, axis=axis)
    # a strided view: every other column of a wider tensor (not 16-byte aligned per sequence)
    wide = torch.randint(0, 3, (40, 2100), generator=torch.Generator().manual_seed(305), dtype=torch.int32)
    view = wide.to(DEV)[:, 1::2]
    got = sx.table_scan(table.to(DEV), view).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.table_scan(table.numpy(), view.cpu().numpy()))


def test_clamping():
    # symbols outside [0, nsym) and table entries outside [0, states) are clamped into range
    table, symbols = _rand(6, 4, (17, 2500), seed=306, lo=-3, hi=9)
    symbols[::3] -= 2
    symbols[1::5] += 3
    _check(table, symbols)


@pytest.mark.parametrize("states,nsym", [(17, 8), (200, 60), (300, 100), (5, 4096)])
def test_serial_kernel(states, nsym):
    # more than 16 states, or more symbols than the wave kernel keeps; tables of 30000 and more entries do not
    # fit the LDS copy
    table, symbols = _rand(states, nsym, (300, 700), seed=307 + states)
    _check(table, symbols)


def test_empty_and_errors():
    t = torch.tensor([[0, 1], [1, 0]], dtype=torch.int32, device=DEV)
    assert sx.table_scan(t, torch.zeros((3, 0), dtype=torch.int32, device=DEV)).shape == (3, 0)
    with pytest.raises(sx.SxError) as e:
        sx.table_scan(t, torch.zeros((3, 4), dtype=torch.int64, device=DEV))
    assert e.value.name == "E-DIM-002"
    with pytest.raises(sx.SxError) as e:
        sx.table_scan(t, torch.zeros((3, 4), dtype=torch.int32, device=DEV), start=2)
    assert e.value.name == "E-DIM-001"
    with pytest.raises(sx.SxError) as e:
        sx.table_scan(t[0], torch.zeros((3, 4), dtype=torch.int32, device=DEV))
    assert e.value.name == "E-DIM-001"


@pytest.mark.parametrize("kind", ["parity", "dfa16"])
def test_measured_workloads_sampled_sequences(kind):
    w = W.make_table(kind)
    print(f"\n[case] {w.name} (sampled sequences)", flush=True)
    got = sx.table_scan(w.tensors["table"].to(DEV), w.tensors["symbols"].to(DEV))
    torch.cuda.synchronize()
    rows = np.random.default_rng(308).integers(0, w.tensors["symbols"].shape[0], 6)
    ref = oracle.table_scan(w.tensors["table"].numpy(), w.tensors["symbols"].numpy()[rows])
    np.testing.assert_array_equal(got.cpu().numpy()[rows], ref)
