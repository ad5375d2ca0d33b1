"""The causal tile set of nanhubrain.csdn.net §三.1 "调度问题建模":
S = {(i, j) | j*Bc <= i*Br + Br - 1} is exactly the set of (Br x Bc) tiles
that hold at least one visible element (key <= query), and a tile is free of
masked elements exactly when j*Bc + Bc - 1 <= i*Br (a derived bound the
kernels use to skip the per-element mask). Brute force over small tilings."""
import itertools

import numpy as np
import pytest


@pytest.mark.parametrize("Br,Bc", [(1, 1), (2, 3), (4, 4), (8, 2), (3, 8), (16, 64), (64, 16), (128, 64), (64, 128)])
def test_tile_set_matches_brute_force(Br, Bc):
    N = 3 * max(Br, Bc) + 5
    vis = np.tril(np.ones((N, N), bool))
    Tr, Tc = -(-N // Br), -(-N // Bc)
    for i, j in itertools.product(range(Tr), range(Tc)):
        block = vis[i * Br:(i + 1) * Br, j * Bc:(j + 1) * Bc]
        in_S = j * Bc <= i * Br + Br - 1
        full = j * Bc + Bc - 1 <= i * Br
        assert in_S == bool(block.any()), (i, j)
        rows = min(Br, N - i * Br)
        cols = min(Bc, N - j * Bc)
        if rows == Br and cols == Bc:
            assert full == bool(block.all()), (i, j)
