"""Pins of the oracle's N:M projection (and its storage in the 2:4 packed layout).

N:M sparsity keeps at most N of every M consecutive weights (HASSLE-free page, §1 and §2: the
framework targets N:M sparsity; 3BASiL article, "A three-block ADMM replaces alternating
minimization": N:M structures such as 2:4, and its 2:8 + rank-64 result after LoRA fine-tuning).
With identity Hessian the sparse step is hard thresholding (HASSLE-free page, §4.1.1), so the
projection must return the Euclidean-nearest N:M matrix. The pins:
  * brute force over every keep-set of every group, maximising the kept energy in exact integer
    arithmetic, ties to the lexicographically smallest set (the lower columns);
  * 2:4 through this path is the 2:4 pack itself, bit for bit, special values included;
  * invariants: at most N nonzeros per group of M, kept entries are bit copies, dropped entries
    +0, idempotence, nesting (the 1:M set lies inside the 2:M set);
  * stored in the 2:4 layout (N <= 2, 4 | M) the packed S unpacks to exactly the projection.
"""
import itertools

import numpy as np
import pytest

import oracle
from sparse_rank_linear_prune24_amd import inputs

BITS = {"fp32": np.uint32, "bf16": np.uint16}
PATTERNS_NM = [(1, 4), (2, 4), (1, 8), (2, 8), (1, 16), (2, 16)]


def small_ints(shape, seed, dtype):
    """Integers in [-3, 3] (many ties) in the storage type."""
    v = np.random.default_rng(seed).integers(-3, 4, size=shape).astype(np.float32)
    return v if dtype == "fp32" else inputs.f32_to_bf16_bits(v)


def as_f32(a, dtype):
    return a if dtype == "fp32" else inputs.bf16_bits_to_f32(a)


def brute_force(R, n, m):
    """Nearest N:M matrix by enumeration: per group the keep-set of size n with the largest kept
    energy (integers: exact), ties to the lexicographically smallest set; dropped entries +0."""
    out = np.zeros_like(R)
    n_out, n_in = R.shape
    for row in range(n_out):
        for g0 in range(0, n_in, m):
            grp = R[row, g0:g0 + m].astype(np.int64)
            best, best_e = None, -1
            for keep in itertools.combinations(range(m), n):   # lexicographic order
                e = int(sum(grp[i] * grp[i] for i in keep))
                if e > best_e:
                    best, best_e = keep, e
            for i in best:
                out[row, g0 + i] = R[row, g0 + i]
    return out


@pytest.mark.parametrize("n,m", PATTERNS_NM)
def test_brute_force(n, m):
    R = small_ints((7, 64), seed=10 * n + m, dtype="fp32")
    got = oracle.prune_nm(R, n, m, "fp32")
    want = brute_force(R, n, m)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_two_four_is_the_pack(dtype):
    R = inputs.gaussian((33, 256), 1.0, dtype, seed=4, config_id=3300, tensor_id=1)
    b = R.view(np.uint32 if dtype == "fp32" else np.uint16)
    specials = [0x7FC00000, 0xFF800000, 0x80000000, 0x7F800000] if dtype == "fp32" else [0x7FC0, 0xFF80, 0x8000, 0x7F80]
    for i, v in enumerate(specials):
        b[i, 4 * i:4 * i + 4] = [v, v, 0, v]                     # ties among specials and a zero
    b[5, 8:12] = 0                                               # an all-zero group
    b[6, 12:16] = b[6, 12]                                       # four equal entries
    v1, m1 = oracle.prune_nm_pack(R, 2, 4, dtype)
    v2, m2 = oracle.prune24_pack(R, dtype)
    assert np.array_equal(m1, m2)
    assert np.array_equal(v1.view(BITS[dtype]), v2.view(BITS[dtype]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,m", PATTERNS_NM)
def test_invariants(dtype, n, m):
    R = inputs.gaussian((24, 192), 1.0, dtype, seed=n + m, config_id=3300, tensor_id=2)
    bits = R.view(np.uint32 if dtype == "fp32" else np.uint16)
    bits[3, :16] = bits[3, 0]                                    # ties
    Rp = oracle.prune_nm(R, n, m, dtype)
    pb = Rp.view(bits.dtype)
    kept = pb != 0
    assert (kept.reshape(24, -1, m).sum(axis=2) <= n).all()
    assert np.array_equal(pb[kept], bits[kept])                  # bit copies
    assert (pb[~kept] == 0).all()                                # +0, no negative zeros
    # Gaussian entries are nonzero: exactly n kept per group, the n largest magnitudes
    f = np.abs(as_f32(R, dtype)).reshape(24, -1, m)
    kf = kept.reshape(24, -1, m)
    assert (kf.sum(axis=2)[np.arange(24) != 3] == n).all()
    assert (np.where(kf, f, np.inf).min(axis=2) >= np.where(kf, -np.inf, f).max(axis=2)).all()
    assert np.array_equal(oracle.prune_nm(Rp, n, m, dtype).view(bits.dtype), pb)   # idempotent
    if n == 2:
        inner = oracle.prune_nm(R, 1, m, dtype).view(bits.dtype) != 0
        assert not (inner & ~kept).any()                          # 1:M inside 2:M


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,m", [(1, 4), (1, 8), (2, 8), (2, 16)])
def test_packed_layout_holds_the_projection(dtype, n, m):
    R = inputs.gaussian((20, 320), 1.0, dtype, seed=7 * m + n, config_id=3300, tensor_id=3)
    Rp = oracle.prune_nm(R, n, m, dtype)
    values, meta = oracle.prune_nm_pack(R, n, m, dtype)
    S = oracle.dense_reconstruct(values, meta, 20, 320, None, None, dtype)
    assert np.array_equal(S, as_f32(Rp, dtype).astype(np.float64))


def test_rejects_patterns_denser_than_two_four():
    R = np.zeros((1, 32), np.float32)
    for n, m in [(3, 4), (4, 8), (3, 8), (2, 6)]:
        with pytest.raises(ValueError):
            oracle.prune_nm_pack(R, n, m, "fp32")
    with pytest.raises(ValueError):
        oracle.prune_nm(np.zeros((1, 36), np.float32), 1, 8, "fp32")   # 8 does not divide 36
