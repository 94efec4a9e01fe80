"""Host logic of bench.py (no GPU): which stage-2 launches a workload's step issues, and which tile
each takes. Equal-shape neighbours are grouped only when one launch needs fewer rounds of 256 tiles
than separate launches; the tile is 512 rows when the launch's layers together give every one of
the 256 CUs a 512 x 128 tile."""
from collections import namedtuple

import pytest

import bench
from sparse_rank_linear_prune24_amd import configs

Shape = namedtuple("Shape", "name n_in n_out M r")


def layers(cfg):
    c = configs.get(cfg)
    return [Shape(n, k, o, c.M, c.r) for n, k, o in c.layers]


@pytest.mark.parametrize("cfg,want", [
    ("C1", [[0]]), ("C2", [[0]]), ("C3", [[0]]),
    ("C4", [[0, 1], [2]]),                      # gate + up: 896 tiles each (3.5 rounds), 7 rounds together
    ("C5", [[0], [1, 2], [3], [4], [5], [6]]),  # k + v: 128 tiles of 512 rows each, 256 together
])
def test_stage2_units(cfg, want):
    assert bench.stage2_units(layers(cfg), cfg == "C3") == want


def test_tile_rule_and_rounds():
    q, k = layers("C5")[0], layers("C5")[1]
    assert bench.wide_tile(q) and not bench.wide_tile(k) and bench.wide_tile(k, 2)
    assert bench.tile_rounds(q) == 2 and bench.tile_rounds(k) == 1 and bench.tile_rounds(k, 2) == 1
    gate = layers("C4")[0]
    assert bench.tile_rounds(gate) == 4 and bench.tile_rounds(gate, 2) == 7
    gate5 = layers("C5")[4]
    assert bench.tile_rounds(gate5) == 7 and bench.tile_rounds(gate5, 2) == 14   # no gain: separate


def test_group_needs_equal_neighbours():
    a = Shape("a", 4096, 1024, 8192, 128)
    b = Shape("b", 4096, 1024, 8192, 64)       # other rank: not groupable with a
    assert bench.stage2_units([a, b, a], False) == [[0], [1], [2]]
    assert bench.stage2_units([a, a, a, a, a], False)[0] == [0, 1, 2, 3]   # at most four per launch
    assert bench.stage2_units([a, a], True) == [[0], [1]]                  # decode: one layer per launch
