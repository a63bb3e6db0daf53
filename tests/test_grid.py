"""The workgroup -> tile map (host evaluation of the device code).

* Bijection: every order maps [0, G) onto the G tiles exactly once, including
  short last windows, grids smaller than a window, group_m that does not
  divide the tile rows, and nxcd = 1.
* Locality: under the dispatch model the map is built for (ids [nW, (n+1)W)
  resident together, id r of a window on chiplet r mod 8), count the distinct
  A row-panels and B column-panels each chiplet touches per window (its L2
  working set) and per whole window (the shared cache's).  The chiplet-aware
  order must never be worse than row-major and must be strictly better where
  row-major scatters a chiplet's tiles (wide N).
"""
import itertools

import numpy as np
import pytest

import fp8_gemm_02_amd as hk


def _map(order, Gm, Gn, group_m=8, window=256, nxcd=8):
    G = Gm * Gn
    tm, tn = hk.hk_grid_map(order, Gm, Gn, group_m, window, nxcd, np.arange(G))
    return tm, tn


@pytest.mark.parametrize("order", ["row_major", "xcd"])
@pytest.mark.parametrize("Gm,Gn", [(1, 1), (1, 7), (7, 1), (3, 5), (16, 16), (32, 32), (32, 112),
                                   (13, 29), (33, 17), (5, 300)])
@pytest.mark.parametrize("group_m,window,nxcd", [(8, 256, 8), (1, 256, 8), (3, 100, 8),
                                                 (16, 64, 8), (4, 7, 8), (8, 256, 1), (5, 33, 3)])
def test_bijection(order, Gm, Gn, group_m, window, nxcd):
    tm, tn = _map(order, Gm, Gn, group_m, window, nxcd)
    assert tm.min() >= 0 and tm.max() < Gm and tn.min() >= 0 and tn.max() < Gn
    ids = tm * Gn + tn
    assert np.array_equal(np.sort(ids), np.arange(Gm * Gn))


def test_row_major_is_identity():
    tm, tn = _map("row_major", 4, 6)
    assert np.array_equal(tm * 6 + tn, np.arange(24))


def test_xcd_slots_are_consecutive_per_chiplet():
    # full window of 256 over a 16 x 16 grid: chiplet x gets slots 32x..32x+31,
    # which the grouped order (group_m = 8) lays out as an 8 x 4 tile block
    tm, tn = _map("xcd", 16, 16, group_m=8, window=256, nxcd=8)
    for x in range(8):
        ids = np.arange(x, 256, 8)
        rows, cols = set(tm[ids].tolist()), set(tn[ids].tolist())
        assert len(rows) == 8 and len(cols) == 4
        assert max(rows) - min(rows) == 7 and max(cols) - min(cols) == 3


def _panels(order, Gm, Gn, window=256, nxcd=8, group_m=8):
    tm, tn = _map(order, Gm, Gn, group_m, window, nxcd)
    G = Gm * Gn
    per_xcd, per_window = [], []
    for n0 in range(0, G, window):
        ids = np.arange(n0, min(G, n0 + window))
        per_window.append(len(set(tm[ids])) + len(set(tn[ids])))
        for x in range(nxcd):
            sel = ids[(ids - n0) % nxcd == x]
            if sel.size:
                per_xcd.append((len(set(tm[sel])) + len(set(tn[sel]))) / sel.size)
    return float(np.mean(per_xcd)), float(np.mean(per_window))


@pytest.mark.parametrize("Gm,Gn", [(16, 16), (32, 32), (32, 112)])
def test_xcd_order_never_worse_than_row_major(Gm, Gn):
    x_l2, x_llc = _panels("xcd", Gm, Gn)
    r_l2, r_llc = _panels("row_major", Gm, Gn)
    assert x_l2 <= r_l2 + 1e-12
    assert x_llc <= r_llc + 1e-12


def test_xcd_order_better_on_the_wide_mlp_grid():
    # 8192 x 28672 output in 256-tiles: row-major deals each chiplet 14
    # different column panels per row; the grouped order gives an 8 x 4 block
    x_l2, x_llc = _panels("xcd", 32, 112)
    r_l2, r_llc = _panels("row_major", 32, 112)
    assert x_l2 < 0.8 * r_l2
    assert x_llc < 0.5 * r_llc


def test_grid_map_rejects_bad_input():
    with pytest.raises(hk.HKError):
        hk.hk_grid_map("xcd", 2, 2, 8, 256, 8, [4])
    with pytest.raises(hk.HKError):
        hk.hk_grid_map("xcd", 2, 2, 0, 256, 8, [0])
    with pytest.raises(hk.HKError):
        hk.hk_grid_map(7, 2, 2, 8, 256, 8, [0])
