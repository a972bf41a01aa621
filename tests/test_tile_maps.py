"""The tile orders of the prefill kernels, evaluated on the host by the
library's own map functions (moe_tile_map; the kernels call the same
functions): over many shapes every tile is run by exactly one workgroup,
padding workgroups get no tile, and the XCD dealing keeps what it is for
(a dense XCD's tiles contiguous in the grouped order; an expert row tile's
column tiles, and the LDS-staged kernel's row-tile pairs, on one XCD)."""
from __future__ import annotations

import ctypes
import itertools

import numpy as np
import pytest

from latent_mixture_experts_amd import binding as B

DENSE, EXPERT, TILED = 0, 1, 2


def _map(kind, a, b):
    lib = B.lib()
    lib.moe_tile_map.restype = ctypes.c_int
    lib.moe_tile_map.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    G = lib.moe_tile_map(kind, a, b, None, 0)
    assert G > 0, (kind, a, b, G)
    out = np.empty(2 * G, np.int32)
    assert lib.moe_tile_map(kind, a, b, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2 * G) == G
    return out.reshape(G, 2)


@pytest.mark.parametrize("M,N", list(itertools.product([1, 100, 128, 129, 512, 1600, 4096, 4097],
                                                       [256, 1024, 1280, 4096, 8192])))
def test_dense_every_tile_exactly_once(M, N):
    t = _map(DENSE, M, N)
    n_row, n_col = (M + 127) // 128, N // 256
    G = t.shape[0]
    assert G % 8 == 0 and G - n_row * n_col < 8
    real = t[t[:, 0] >= 0]
    pad = t[t[:, 0] < 0]
    assert (pad == -1).all() and len(real) == n_row * n_col
    assert (real[:, 0] < n_row).all() and (real[:, 1] >= 0).all() and (real[:, 1] < n_col).all()
    ids = real[:, 0] * n_col + real[:, 1]
    assert len(np.unique(ids)) == len(ids)


def test_dense_small_padding_case():
    """The shape that once sent padding workgroups past the weights: 1600 x
    1024 outputs (52 tiles in a grid of 56)."""
    t = _map(DENSE, 1600, 1024)
    assert t.shape[0] == 56 and (t[t[:, 0] < 0] == -1).all() and (t[:, 0] >= 0).sum() == 52
    assert (t[:, 1] < 4).all()


@pytest.mark.parametrize("kind", [EXPERT, TILED])
@pytest.mark.parametrize("rows,cols", list(itertools.product([1, 2, 3, 7, 16, 377, 513, 1000],
                                                             [1, 2, 16, 32, 64])))
def test_expert_orders_every_tile_once_and_xcd_locality(kind, rows, cols):
    t = _map(kind, rows, cols)
    G = t.shape[0]
    chunk = (2 if kind == EXPERT else 1) * cols
    assert G % (8 * chunk) == 0 and G >= rows * cols
    logical = t[:, 0] * cols + t[:, 1]
    assert np.array_equal(np.sort(logical), np.arange(G))          # a bijection on the grid
    assert (t[:, 1] >= 0).all() and (t[:, 1] < cols).all()
    live = t[:, 0] < rows                                           # the tiles a call can have
    assert live.sum() == rows * cols
    xcd = np.arange(G) % 8
    group = t[:, 0] // (2 if kind == EXPERT else 1)                 # row tile (pair) of each workgroup
    for gr in np.unique(group):
        assert len(np.unique(xcd[group == gr])) == 1, (gr, "split over XCDs")
    # every XCD gets work while only a prefix of the row tiles exists
    if rows * cols >= 8 * chunk:
        assert len(np.unique(xcd[live])) == 8
