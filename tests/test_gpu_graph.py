"""The hot path captured in a HIP graph (as bench.py replays it) gives the eager results on every
replay, with eager work and synchronisations between the replays."""
import pytest
import torch

from sparse_rank_linear_prune24_amd import binding, inputs
from tests._helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,r", [(16, 64), (300, 64)])
def test_graph_replays_match_eager(M, r):
    print(f"[graph] M={M} n_in=1024 n_out=512 r={r}", flush=True)
    L = inputs.random_case(M, 1024, 512, r, "bf16", seed=5, n_outliers=4)
    R, X, U, V = (to_dev(a, "bf16") for a in (L.R, L.X, L.U, L.V))
    values, meta = binding.prune24_pack(R)
    ws = binding.new_workspace(M, 512, 1024, r, torch.bfloat16, X.device)
    Y = torch.empty((M, 512), dtype=torch.float32, device=X.device)

    def step(stream):
        binding.prune24_pack(R, values, meta, stream=stream)
        binding.linear_stage1(X, V, ws, stream=stream)
        binding.linear_stage2(X, values, meta, U, ws, n_out=512, out=Y, stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.synchronize()
    v_ref, m_ref, y_ref = values.clone(), meta.clone(), Y.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    for rep in range(3):
        values.zero_()
        meta.zero_()
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(values.view(torch.int16), v_ref.view(torch.int16)), rep
        assert torch.equal(meta, m_ref), rep
        assert torch.equal(Y.view(torch.int32), y_ref.view(torch.int32)), rep
