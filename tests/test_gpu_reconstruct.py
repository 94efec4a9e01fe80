"""GPU parity of splr_dense_reconstruct: S part bit-exact, S + U V within 1e-6 rms (float32)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, inputs
from tests._helpers import from_dev, meta_from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_out,n_in,r", [(1, 32, 16), (33, 96, 16), (256, 1024, 64), (100, 4096, 128)])
def test_reconstruct(dtype, n_out, n_in, r):
    print(f"[reconstruct] dtype={dtype} {n_out}x{n_in} r={r}", flush=True)
    L = inputs.random_case(4, n_in, n_out, r, dtype, seed=n_out + r)
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    v, m = from_dev(vd, dtype), meta_from_dev(md)
    # S only: exact (kept entries widened, +0 elsewhere, signed zeros preserved)
    W0 = binding.dense_reconstruct(vd, md, None, None, n_out=n_out, n_in=n_in).cpu().numpy()
    ref0 = oracle.dense_reconstruct(v, m, n_out, n_in, None, None, dtype).astype(np.float32)
    assert np.array_equal(W0.view(np.uint32), ref0.view(np.uint32))
    # S + U V
    W = binding.dense_reconstruct(vd, md, to_dev(L.U, dtype), to_dev(L.V, dtype)).cpu().numpy()
    ref = oracle.dense_reconstruct(v, m, n_out, n_in, L.U, L.V, dtype)
    assert rel_err(W, ref) <= 1e-6


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_signed_zeros_survive(dtype):
    """Kept -0 entries come back as -0 without a low-rank part, bit for bit as the oracle's."""
    print(f"[reconstruct signed zeros] dtype={dtype}", flush=True)
    neg0 = 0x80000000 if dtype == "fp32" else 0x8000
    one = 0x3F800000 if dtype == "fp32" else 0x3F80
    width = np.uint32 if dtype == "fp32" else np.uint16
    bits = np.zeros((2, 64), dtype=width)
    bits[0, 0] = neg0            # -0 kept at position 0 of the first group (nibble 0xC)
    bits[0, 3] = one
    bits[1, 4:8] = [neg0, neg0, 0, neg0]   # all zeros: the two lowest positions, -0 and -0
    bits[1, 9] = neg0            # one -0 beside three +0: positions 0 and 1
    R = bits.view(np.float32) if dtype == "fp32" else bits
    vd, md = binding.prune24_pack(to_dev(R, dtype))
    W = binding.dense_reconstruct(vd, md, None, None, n_out=2, n_in=64).cpu().numpy().view(np.uint32)
    v, m = oracle.prune24_pack(R, dtype)
    ref = oracle.dense_reconstruct(v, m, 2, 64, None, None, dtype).astype(np.float32).view(np.uint32)
    assert np.array_equal(W, ref)
    assert W[0, 0] == 0x80000000 and W[0, 3] == 0x3F800000 and W[0, 1] == 0 and W[0, 2] == 0
