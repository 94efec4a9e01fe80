"""splr_linear_noalloc (the layer product with the library's built-in workspace, for callers that
cannot allocate) through the C ABI, against splr_linear with a caller workspace: the two run the
same kernels, so Y must agree bit for bit. Two calls in a row on the built-in buffer, the second
with a smaller input than the first (it reads only what it wrote), for each storage type and for
the prefill and decode kernels."""
import numpy as np
import pytest
import torch

from sparse_rank_linear_prune24_amd import binding, inputs
from tests._helpers import meta_to_dev, to_dev

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402  (the packs come from the oracle, so both calls read identical S)

CASES = {
    "bf16": [(1100, 2080, 300, 128), (200, 512, 130, 64), (16, 4096, 64, 64), (5, 96, 40, 16)],
    "fp32": [(70, 160, 33, 32), (3, 64, 20, 16)],
}


def _layer(M, n_in, n_out, r, dtype, seed):
    L = inputs.random_case(M, n_in, n_out, r, dtype, seed=seed, n_outliers=2 if dtype == "bf16" else 0)
    v, m = oracle.prune24_pack(L.R, dtype)
    return L, to_dev(v, dtype), meta_to_dev(m)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_linear(dtype):
    for i, (M, n_in, n_out, r) in enumerate(CASES[dtype]):
        print(f"[noalloc] dtype={dtype} call {i}: M={M} n_in={n_in} n_out={n_out} r={r}", flush=True)
        L, vd, md = _layer(M, n_in, n_out, r, dtype, seed=100 + i)
        Xd, Ud, Vd = to_dev(L.X, dtype), to_dev(L.U, dtype), to_dev(L.V, dtype)
        need = binding.workspace_bytes(M, n_out, n_in, r, Xd.dtype)
        assert need <= 32 << 20
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        Y_ref = binding.linear(Xd, vd, md, Ud, Vd, n_out=n_out, workspace=ws)
        Y = torch.full((M, n_out), float("nan"), dtype=torch.float32, device="cuda")
        binding.linear_noalloc(Xd, vd, md, Ud, Vd, n_out=n_out, out=Y)
        torch.cuda.synchronize()
        a, b = Y.cpu().numpy(), Y_ref.cpu().numpy()
        assert np.all(np.isfinite(a))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {i}: differs from splr_linear"


def test_noalloc_rejects_oversized():
    X = torch.zeros((16384, 64), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros((1024, 64), dtype=torch.bfloat16, device="cuda")
    U = torch.zeros((16, 1024), dtype=torch.bfloat16, device="cuda")
    TR, TK = binding.tiles(16, 64)
    vals = torch.zeros((TR, TK, 64, 8), dtype=torch.bfloat16, device="cuda")
    meta = torch.zeros(binding.meta_shape(16, 64), dtype=torch.int32, device="cuda")
    Y = torch.empty((16384, 16), dtype=torch.float32, device="cuda")
    assert binding.workspace_bytes(16384, 16, 64, 1024, torch.bfloat16) > 32 << 20
    with pytest.raises(binding.SplrError, match="SPLR_ERR_SCRATCH"):
        binding.linear_noalloc(X, vals, meta, U, V, n_out=16, out=Y)
