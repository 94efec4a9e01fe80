"""Pins of the oracle's 2:4 projection + pack against what the pages and the mathematics fix.

The projection is the sparse step with identity Hessian, solved exactly by hard thresholding
(HASSLE-free page, §4.1.1), under the constraint that at most two of every four consecutive
weights are nonzero (3BASiL article, "A three-block ADMM replaces alternating minimization").
So it must return the Euclidean-nearest 2:4 matrix. The pins:
  * brute force over all six keep patterns per group, minimising the discarded energy in exact
    rational arithmetic, ties to the lexicographically smallest pattern;
  * hand-written outcomes for ties and special values (tests/golden/pack_special_groups.txt);
  * invariants: <= 2 nonzeros per group, idempotence, sign and power-of-two equivariance,
    equivariance under permutations of whole groups, kept energy >= half the group's energy.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_rank_linear_prune24_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
PATTERNS = [(a, b) for a in range(4) for b in range(a + 1, 4)]      # the six ways to keep two of four
VALID_NIBBLES = {a | (b << 2) for a, b in PATTERNS}
NP = {"fp32": np.float32, "bf16": np.uint16}


def exact(x_bits, dtype):
    """Exact rational value of a stored (finite) element."""
    return Fraction(float(inputs.to_f64(np.array([x_bits], dtype=NP[dtype]), dtype)[0]))


def brute_force_group(group_bits, dtype):
    """Pattern (a, b) minimising the discarded energy, exactly; ties -> lexicographically smallest."""
    vals = [exact(x, dtype) for x in group_bits]
    best = None
    for a, b in PATTERNS:           # PATTERNS is in lexicographic order, so `<` keeps the smallest
        discarded = sum(v * v for i, v in enumerate(vals) if i not in (a, b))
        if best is None or discarded < best[0]:
            best = (discarded, a, b)
    return best[1], best[2]


def pack_logical(R, dtype):
    """Oracle pack, returned as its logical view: kept [n_out x n_in/2], nibbles [n_out x n_in/4]."""
    values, meta = oracle.prune24_pack(R, dtype)
    kept, nib = oracle.unpack(values, meta, R.shape[0], R.shape[1], dtype)
    return kept, nib.astype(np.uint32), values, meta


def groups_to_matrix(groups, dtype):
    """Lay out 4-element groups (a storage-dtype array) as rows of 32 columns, zero padded."""
    g = np.asarray(groups).reshape(-1, 4)
    assert g.dtype == NP[dtype]
    pad = (-len(g)) % 8
    if pad:
        g = np.concatenate([g, np.zeros((pad, 4), dtype=NP[dtype])])
    return g.reshape(-1, 32), len(groups)


def check_against_brute_force(R, dtype):
    values, nib, _, _ = pack_logical(R, dtype)
    n_out, n_in = R.shape
    for n in range(n_out):
        for g in range(n_in // 4):
            grp = R[n, 4 * g:4 * g + 4]
            a, b = brute_force_group(grp, dtype)
            assert nib[n, g] == (a | (b << 2)), (n, g, grp, nib[n, g], (a, b))
            assert values[n, 2 * g] == grp[a] and values[n, 2 * g + 1] == grp[b]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_exhaustive_small_integer_groups(dtype):
    # every 4-tuple over {-2..2}: all tie shapes, zeros of both signs excluded (no -0 integers)
    groups = list(itertools.product(range(-2, 3), repeat=4))
    f = np.array(groups, dtype=np.float64)
    R, _ = groups_to_matrix(inputs.from_f64(f, dtype), dtype)
    check_against_brute_force(R, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_random_groups_brute_force(dtype):
    g = np.random.default_rng(7)
    f = g.standard_normal((40, 64)) * 0.02
    # sprinkle exact ties, zeros and sign flips
    f[:, 5] = f[:, 6]
    f[:, 9] = -f[:, 10]
    f[::3, 20:24] = 0.0
    f[1::4, 33] = f[1::4, 35]
    R = inputs.from_f64(f, dtype)
    check_against_brute_force(R, dtype)


def test_special_value_fixture():
    rows = {"fp32": [], "bf16": []}
    with open(os.path.join(HERE, "golden", "pack_special_groups.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            dtype = parts[0]
            xs = [int(t, 16) for t in parts[1:5]]
            rows[dtype].append((xs, int(parts[5], 16), int(parts[6], 16), int(parts[7], 16)))
    assert len(rows["fp32"]) >= 15 and len(rows["bf16"]) >= 10
    for dtype, cases in rows.items():
        # place the cases at every group slot of a 32-wide row, twice over with an offset, so the
        # nibble position inside the metadata word is exercised
        for shift in range(2):
            groups = [[0, 0, 0, 0]] * shift + [c[0] for c in cases]
            bits = np.array(groups, dtype=np.uint32 if dtype == "fp32" else np.uint16)
            R, ng = groups_to_matrix(bits.view(NP[dtype]), dtype)
            values, nib, _, _ = pack_logical(R, dtype)
            nib = nib.reshape(-1)
            vals = values.reshape(-1, 2)
            for i, (xs, want_nib, v0, v1) in enumerate(cases):
                k = i + shift
                assert nib[k] == want_nib, (dtype, [hex(x) for x in xs], hex(nib[k]), hex(want_nib))
                got = vals[k].view(np.uint32 if dtype == "fp32" else np.uint16)
                assert int(got[0]) == v0 and int(got[1]) == v1, (dtype, [hex(x) for x in xs])


def _dense_of(values, meta, shape, dtype):
    """The packed matrix scattered back to storage dtype (exact: S entries are stored values)."""
    return inputs.from_f64(oracle.dense_reconstruct(values, meta, shape[0], shape[1], None, None, dtype), dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_invariants_gaussian(dtype):
    g = np.random.default_rng(11)
    R = inputs.from_f64(g.standard_normal((96, 256)) * 0.02, dtype)
    values, nib, pv, pm = pack_logical(R, dtype)
    assert set(np.unique(nib).tolist()) <= VALID_NIBBLES

    S = _dense_of(pv, pm, R.shape, dtype)
    Sf = inputs.to_f64(S, dtype)
    nz = (Sf.reshape(96, -1, 4) != 0).sum(axis=2)
    assert nz.max() <= 2
    # kept entries are bit copies of R
    kept = Sf != 0
    assert np.array_equal(S[kept], R[kept])

    # idempotence: projecting an already-2:4 matrix changes nothing
    v2, m2 = oracle.prune24_pack(S, dtype)
    assert np.array_equal(v2, pv) and np.array_equal(m2, pm)

    # sign equivariance: same positions, negated values (sign bit flipped)
    sign = np.uint32(0x80000000) if dtype == "fp32" else np.uint16(0x8000)
    Rb = R.view(np.uint32) if dtype == "fp32" else R
    Rneg = (Rb ^ sign).view(R.dtype) if dtype == "fp32" else Rb ^ sign
    vn, nn, _, _ = pack_logical(Rneg, dtype)
    assert np.array_equal(nn, nib)
    vb = values.view(np.uint32) if dtype == "fp32" else values
    vnb = vn.view(np.uint32) if dtype == "fp32" else vn
    assert np.array_equal(vnb, vb ^ sign)

    # power-of-two scaling changes no decision (no overflow / underflow at these magnitudes)
    for e in (-6, 3):
        Rs = inputs.from_f64(inputs.to_f64(R, dtype) * 2.0 ** e, dtype)
        vs, ns, _, _ = pack_logical(Rs, dtype)
        assert np.array_equal(ns, nib)
        assert np.array_equal(inputs.to_f64(vs, dtype), inputs.to_f64(values, dtype) * 2.0 ** e)

    # permuting whole groups permutes the nibbles and value pairs the same way
    perm = g.permutation(256 // 4)
    Rp = R.reshape(96, -1, 4)[:, perm, :].reshape(96, 256)
    vp, np_, _, _ = pack_logical(Rp, dtype)
    assert np.array_equal(np_, nib[:, perm])
    assert np.array_equal(vp.reshape(96, -1, 2), values.reshape(96, -1, 2)[:, perm, :])

    # kept energy is at least half of every group's energy (top two of four squares)
    Rf = inputs.to_f64(R, dtype).reshape(96, -1, 4)
    kept_e = (Sf.reshape(96, -1, 4) ** 2).sum(axis=2)
    assert np.all(kept_e >= 0.5 * (Rf ** 2).sum(axis=2))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_optimal_against_every_pattern_vectorised(dtype):
    """Large-scale brute force: the kept pattern discards no more energy than any of the six."""
    g = np.random.default_rng(3)
    R = inputs.from_f64(g.standard_normal((128, 512)) * 0.02, dtype)
    values, nib, _, _ = pack_logical(R, dtype)
    x2 = inputs.to_f64(R, dtype).reshape(128, -1, 4) ** 2
    a = nib & 3
    b = nib >> 2
    total = x2.sum(axis=2)
    chosen = total - np.take_along_axis(x2, a[..., None], 2)[..., 0] - np.take_along_axis(x2, b[..., None], 2)[..., 0]
    for pa, pb in PATTERNS:
        other = total - x2[..., pa] - x2[..., pb]
        assert np.all(chosen <= other)


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.prune24_pack(np.zeros((4, 48), dtype=np.float32), "fp32")   # 48 % 32 != 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_tiled_layout_positions(dtype):
    """Physical placement of the packed layout, checked at hand-derived positions.

    Layout (our reading; the pages fix no storage format): tiles of 16 rows x 64 input columns;
    group g of row n lives in tile (n // 16, g // 16), at slot L = n % 16 + 16 * ((g % 16) // 4),
    entries 2 * (g % 4) and 2 * (g % 4) + 1. Metadata: blocks of 8 tile columns per tile row,
    meta[tile row, tk // 8, L, (tk % 8) // 2], nibble at bits 16 * (tk % 2) + 4 * (g % 4).
    Padding is zero."""
    n_out, n_in = 17, 96                   # 2 x 2 tiles, ragged in both directions; one block
    g = np.random.default_rng(5)
    f = g.standard_normal((n_out, n_in)) + 3.0  # all positive, no ties
    R = inputs.from_f64(f, dtype)
    kept, nib, values, meta = pack_logical(R, dtype)
    assert values.shape == (2, 2, 64, 8) and meta.shape == (2, 1, 64, 4)
    cases = [  # (row, group) -> (tile row, tile col, slot, entry, meta block, meta word, nibble shift)
        ((0, 0), (0, 0, 0, 0, 0, 0, 0)),
        ((5, 13), (0, 0, 53, 2, 0, 0, 4)),
        ((16, 17), (1, 1, 0, 2, 0, 0, 20)),
        ((3, 20), (0, 1, 19, 0, 0, 0, 16)),
        ((9, 7), (0, 0, 25, 6, 0, 0, 12)),
    ]
    for (n, grp), (tr, tk, slot, e, tb, w, sh) in cases:
        assert values[tr, tk, slot, e] == kept[n, 2 * grp] and values[tr, tk, slot, e + 1] == kept[n, 2 * grp + 1]
        assert (meta[tr, tb, slot, w] >> sh) & 0xF == nib[n, grp]
    # column padding: the second tile column holds groups 16..23 only (slots 0..31); tile columns
    # 2..7 of the block do not exist
    assert not values[:, 1, 32:, :].any() and not (meta[:, 0, 32:, 0] >> 16).any()
    assert not meta[:, :, :, 1:].any()
    # row padding: only row 16 exists in the second tile row
    rows_used = np.zeros(64, dtype=bool)
    rows_used[[0, 16, 32, 48]] = True
    assert not values[1][:, ~rows_used, :].any()
    assert not meta[1][:, ~rows_used, :].any()

    # a second block and the upper words of a slot: 9 tile columns
    R2 = inputs.from_f64(g.standard_normal((16, 576)) + 3.0, dtype)
    kept2, nib2, _, meta2 = pack_logical(R2, dtype)
    assert meta2.shape == (1, 2, 64, 4)
    for (n, grp), (tb, slot, w, sh) in [((2, 86), (0, 18, 2, 24)), ((7, 143), (1, 55, 0, 12)),
                                        ((15, 127), (0, 63, 3, 28)), ((0, 48), (0, 0, 1, 16))]:
        assert (meta2[0, tb, slot, w] >> sh) & 0xF == nib2[n, grp]
    assert not (meta2[0, 1, :, 0] >> 16).any() and not meta2[0, 1, :, 1:].any()


def _fixture_cases():
    rows = {"fp32": [], "bf16": []}
    with open(os.path.join(HERE, "golden", "pack_special_groups.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                p = line.split()
                rows[p[0]].append(([int(t, 16) for t in p[1:5]], int(p[5], 16), int(p[6], 16), int(p[7], 16)))
    return rows


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_reconstruct_without_low_rank_is_the_stored_entries(dtype):
    """With no low-rank part the reconstruction is S itself (LoSparse page, §3: W ~ UV + S with the
    low-rank part absent): the fixture's two stored entries, widened exactly to float32, at the
    positions of its hand-written nibble, and +0 at the other two. The fixture keeps -0 in several
    groups (e.g. 80000000 00000000 00000000 00000001 -> 80000000 at position 0), so an
    implementation that adds an empty low-rank sum (-0 + 0 = +0) fails here."""
    cases = _fixture_cases()[dtype]
    width = np.uint32 if dtype == "fp32" else np.uint16
    R, ng = groups_to_matrix(np.array([c[0] for c in cases], dtype=width).view(NP[dtype]), dtype)
    values, meta = oracle.prune24_pack(R, dtype)
    W = oracle.dense_reconstruct(values, meta, R.shape[0], R.shape[1], None, None, dtype)
    got = W.astype(np.float32).view(np.uint32).reshape(-1, 4)
    widen = (lambda b: b) if dtype == "fp32" else (lambda b: b << 16)
    for i, (xs, nibble, v0, v1) in enumerate(cases):
        a, b = nibble & 3, nibble >> 2
        want = [0, 0, 0, 0]
        want[a], want[b] = widen(v0), widen(v1)
        # NaN payloads do not survive the float64 round trip bit for bit; compare them as NaN
        for q in range(4):
            wq = np.array([want[q]], dtype=np.uint32).view(np.float32)[0]
            if np.isnan(wq):
                assert np.isnan(got[i, q].view(np.float32)), (dtype, i, q)
            else:
                assert int(got[i, q]) == want[q], (dtype, [hex(x) for x in xs], q, hex(int(got[i, q])), hex(want[q]))
    assert any(c[2] in (0x80000000, 0x8000) or c[3] in (0x80000000, 0x8000) for c in cases), "fixture keeps a -0"
