"""GPU parity of splr_linear_ex with a bfloat16 Y.

The bfloat16 output is the float32 result of the same kernels rounded to nearest even, so two
checks: (1) bit for bit equal to round-to-nearest-even (done here on the host) of splr_linear's
float32 Y on the same inputs; (2) against the float64 oracle,
    |Y_bf16 - Y_ref| <= TAU * rms(Y_ref) + |Y_ref| * 2^-8   (half an ulp of bfloat16),
for prefill and decode shapes, float32 and bfloat16 inputs, ragged sizes and ranks 0 / 64 / 80."""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, inputs
from tests._helpers import TAU, rms, to_dev

pytestmark = pytest.mark.gpu


def rne_bf16_bits(y32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = y32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,n_in,n_out,r", [(16, 4096, 256, 64), (40, 1056, 100, 80), (300, 2080, 258, 64),
                                            (128, 512, 96, 0), (2048, 1024, 512, 64)])
def test_bf16_output(dtype, M, n_in, n_out, r):
    print(f"[linear bf16 Y] dtype={dtype} M={M} n_in={n_in} n_out={n_out} r={r}", flush=True)
    L = inputs.random_case(M, n_in, n_out, r, dtype, seed=M + n_out + r, n_outliers=2)
    Xd = to_dev(L.X, dtype)
    Ud = to_dev(L.U, dtype) if r else None
    Vd = to_dev(L.V, dtype) if r else None
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    y16 = binding.linear_ex(Xd, vd, md, Ud, Vd, y_dtype=torch.bfloat16, n_out=n_out)
    y32 = binding.linear(Xd, vd, md, Ud, Vd, n_out=n_out)
    torch.cuda.synchronize()
    bits16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits16, rne_bf16_bits(y32.cpu().numpy()))
    v_ref, m_ref = oracle.prune24_pack(L.R, dtype)
    y_ref = oracle.linear(L.X, v_ref, m_ref, n_out, L.U if r else None, L.V if r else None, dtype)
    y = inputs.bf16_bits_to_f32(bits16).astype(np.float64)
    bound = TAU[dtype] * rms(y_ref) + np.abs(y_ref) * 2.0 ** -8
    assert np.all(np.abs(y - y_ref) <= bound)


def test_bf16_output_full_mlp_layer():
    """The 8192-token MLP gate layer at rank 128 (the block workload's largest output): its
    bfloat16 Y (235 MB) is stored non-temporally. Bit for bit against the host's rounding of the
    float32 Y (also non-temporal, 470 MB) of the same kernels, and sampled token rows against the
    oracle within TAU * rms + half an ulp."""
    L = inputs.make_layer("C5", 4)
    assert (L.M, L.n_in, L.n_out, L.r) == (8192, 4096, 14336, 128)
    print(f"[linear bf16 Y] C5/{L.name} M={L.M} n_in={L.n_in} n_out={L.n_out} r={L.r}", flush=True)
    Xd, Ud, Vd = to_dev(L.X, "bf16"), to_dev(L.U, "bf16"), to_dev(L.V, "bf16")
    vd, md = binding.prune24_pack(to_dev(L.R, "bf16"))
    y16 = binding.linear_ex(Xd, vd, md, Ud, Vd, y_dtype=torch.bfloat16, n_out=L.n_out)
    y32 = binding.linear(Xd, vd, md, Ud, Vd, n_out=L.n_out)
    torch.cuda.synchronize()
    bits16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    y32h = y32.cpu().numpy()
    del y16, y32
    assert np.array_equal(bits16, rne_bf16_bits(y32h))
    rows = np.array([0, 1, 127, 128, 4095, 8191])
    v_ref, m_ref = oracle.prune24_pack(L.R, "bf16")
    y_ref = oracle.linear(L.X, v_ref, m_ref, L.n_out, L.U, L.V, "bf16", rows=rows)
    y = inputs.bf16_bits_to_f32(bits16[rows]).astype(np.float64)
    bound = TAU["bf16"] * rms(y_ref) + np.abs(y_ref) * 2.0 ** -8
    assert np.all(np.abs(y - y_ref) <= bound)
