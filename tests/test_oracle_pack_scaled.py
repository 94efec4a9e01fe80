"""Pins of the oracle's activation-aware 2:4 projection + pack.

With a diagonal Hessian the sparse step hard-thresholds the residual scaled column by column by D
(HASSLE-free page, §4.1.2: the result is Wanda's score |W_ij| * ||X_j||), and the entries kept are
the residual's own. Per group of four that keeps the two entries of largest |R[n][k]| * |d[k]|,
which is the 2:4 matrix S minimising the column-weighted error sum_k d_k^2 (R[n][k] - S[n][k])^2.
Pins:
  * brute force over the six keep patterns, minimising the weighted discarded energy in exact
    rational arithmetic, ties to the lexicographically smallest pattern;
  * unit scales reproduce the plain projection bit for bit;
  * power-of-two rescaling of d or of R leaves the selection unchanged;
  * hand-written outcomes for ties, zero scales and special values
    (tests/golden/pack_scaled_groups.txt).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_rank_linear_prune24_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
PATTERNS = [(a, b) for a in range(4) for b in range(a + 1, 4)]
NP = {"fp32": np.float32, "bf16": np.uint16}


def logical(R, d, dtype):
    values, meta = oracle.prune24_pack_scaled(R, d, dtype)
    kept, nib = oracle.unpack(values, meta, R.shape[0], R.shape[1], dtype)
    return kept, nib.astype(np.uint32)


def brute_force_group(vals, scales):
    """Pattern (a, b) minimising sum over discarded k of (d_k x_k)^2, exactly; ties -> smallest."""
    best = None
    for a, b in PATTERNS:
        discarded = sum((s * v) ** 2 for i, (v, s) in enumerate(zip(vals, scales)) if i not in (a, b))
        if best is None or discarded < best[0]:
            best = (discarded, a, b)
    return best[1], best[2]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_brute_force_weighted(dtype):
    n_out, n_in = 24, 64
    # small integers (many exact ties) and random scales with zeros and repeats
    R = inputs.small_integers((n_out, n_in), -4, 4, dtype, seed=21)
    g = np.random.default_rng(5)
    d = g.choice(np.array([0.0, 0.5, 1.0, 2.0, 3.0, 0.25], np.float32), size=n_in)
    kept, nib = logical(R, d, dtype)
    x = inputs.to_f64(R, dtype)
    for n in range(n_out):
        for gi in range(n_in // 4):
            vals = [Fraction(float(v)) for v in x[n, 4 * gi:4 * gi + 4]]
            scales = [Fraction(float(s)) for s in d[4 * gi:4 * gi + 4]]
            a, b = brute_force_group(vals, scales)
            assert nib[n, gi] == (a | (b << 2)), (n, gi, vals, scales)
            want = R[n, [4 * gi + a, 4 * gi + b]]
            assert np.array_equal(kept[n, 2 * gi:2 * gi + 2].view(NP[dtype]), want.view(NP[dtype]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_random_gaussian_brute_force(dtype):
    n_out, n_in = 16, 128
    R = inputs.gaussian((n_out, n_in), 0.02, dtype, seed=3)
    X = inputs.activations(64, n_in, dtype, 4, 20.0, seed=3, config_id=9, layer_id=0)
    d = inputs.column_scales(X, dtype)
    kept, nib = logical(R, d, dtype)
    x = inputs.to_f64(R, dtype)
    for n in range(n_out):
        for gi in range(n_in // 4):
            vals = [Fraction(float(v)) for v in x[n, 4 * gi:4 * gi + 4]]
            scales = [Fraction(float(s)) for s in d[4 * gi:4 * gi + 4]]
            a, b = brute_force_group(vals, scales)
            assert nib[n, gi] == (a | (b << 2))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_unit_scales_are_the_plain_projection(dtype):
    R = inputs.gaussian((48, 256), 0.02, dtype, seed=8)
    R[3, :16] = 0  # whole zero groups
    v1, m1 = oracle.prune24_pack(R, dtype)
    v2, m2 = oracle.prune24_pack_scaled(R, np.ones(256, np.float32), dtype)
    assert np.array_equal(v1.view(np.uint8), v2.view(np.uint8)) and np.array_equal(m1, m2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_power_of_two_rescaling(dtype):
    R = inputs.gaussian((32, 128), 0.02, dtype, seed=11)
    X = inputs.activations(32, 128, dtype, 2, 20.0, seed=11, config_id=9, layer_id=1)
    d = inputs.column_scales(X, dtype)
    _, nib = logical(R, d, dtype)
    _, nib_d = logical(R, d * np.float32(8.0), dtype)
    R2 = inputs.from_f64(inputs.to_f64(R, dtype) * 0.25, dtype)
    kept2, nib_r = logical(R2, d, dtype)
    _, nib_neg = logical(R, -d, dtype)  # the score uses |d|
    assert np.array_equal(nib, nib_d) and np.array_equal(nib, nib_r) and np.array_equal(nib, nib_neg)


def test_scaled_fixture():
    cases = []
    with open(os.path.join(HERE, "golden", "pack_scaled_groups.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                p = [int(t, 16) for t in line.split()]
                cases.append((p[0:4], p[4:8], p[8]))
    assert len(cases) >= 12
    for shift in range(2):
        groups = [[0, 0, 0, 0]] * shift + [c[0] for c in cases]
        scales = [[0, 0, 0, 0]] * shift + [c[1] for c in cases]
        pad = (-len(groups)) % 8
        groups += [[0, 0, 0, 0]] * pad
        scales += [[0, 0, 0, 0]] * pad
        R = np.array(groups, dtype=np.uint32).view(np.float32).reshape(-1, 32)
        d_rows = np.array(scales, dtype=np.uint32).view(np.float32).reshape(-1, 32)
        for row in range(R.shape[0]):  # one row at a time: d is per column
            _, nib = logical(R[row:row + 1].copy(), d_rows[row].copy(), "fp32")
            for j in range(8):
                i = row * 8 + j - shift
                if 0 <= i < len(cases):
                    assert nib[0, j] == cases[i][2], ([hex(x) for x in cases[i][0]], [hex(x) for x in cases[i][1]],
                                                       hex(nib[0, j]), hex(cases[i][2]))


def test_scaled_errors():
    R = np.zeros((4, 32), np.float32)
    with pytest.raises(ValueError):
        oracle.prune24_pack_scaled(R, np.ones(31, np.float32), "fp32")
