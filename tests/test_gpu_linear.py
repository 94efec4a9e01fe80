"""GPU parity of splr_linear against the float64 oracle.

Bar (written here, checked on every case): max|Y_gpu - Y_ref| <= tau * rms(Y_ref) with tau = 1e-5 for
float32 inputs and 1e-2 for bfloat16 inputs (float32 accumulation), Y_ref computed by the oracle on
the same rounded inputs. Both sides pack their own S from the same residual R; the packs are
compared bit for bit first.

The bf16 cases also check a tighter bound, TIGHT = 2e-4: products of bfloat16 values are exact in
float32 and sums over at most 14336 terms keep the float32 error near 1e-5 rms; the first low-rank
stage is carried as a bfloat16 pair (relative error <= 2^-18 per element). A dropped term or a misplaced index
shows up far above this bound, while the 1e-2 bar alone could miss the small rank-r term.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, configs, inputs
from tests._helpers import TAU, from_dev, meta_from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu
TIGHT = 2e-4


def run_gpu(L, dtype, pack_on_gpu=True):
    Xd, Ud, Vd = to_dev(L.X, dtype), to_dev(L.U if L.r else None, dtype), to_dev(L.V if L.r else None, dtype)
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    Y = binding.linear(Xd, vd, md, Ud, Vd, n_out=L.n_out)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), from_dev(vd, dtype), meta_from_dev(md)


def check_layer(L, dtype, tag, rows=None, tight=True):
    print(f"[linear] {tag} dtype={dtype} M={L.M} n_in={L.n_in} n_out={L.n_out} r={L.r}", flush=True)
    Y, v, m = run_gpu(L, dtype)
    v_ref, m_ref = oracle.prune24_pack(L.R, dtype)
    bits = np.uint32 if dtype == "fp32" else np.uint16
    assert np.array_equal(m, m_ref) and np.array_equal(v.view(bits), v_ref.view(bits)), f"{tag}: pack differs"
    U, V = (L.U, L.V) if L.r else (None, None)
    Y_ref = oracle.linear(L.X, v_ref, m_ref, L.n_out, U, V, dtype, rows=rows)
    Yg = Y if rows is None else Y[rows]
    assert np.all(np.isfinite(Yg))
    err = rel_err(Yg, Y_ref)
    print(f"[linear] {tag}: max|dY|/rms = {err:.3e}", flush=True)
    assert err <= TAU[dtype], f"{tag}: {err:.3e} > {TAU[dtype]}"
    if dtype == "bf16" and tight:
        assert err <= TIGHT, f"{tag}: {err:.3e} above the expected float32-accumulation error"
    return err


# shapes spanning several tiles, ragged in every dimension; M <= 64 takes the decode kernel
SHAPES = [
    (1, 64, 16, 16), (5, 32, 40, 16), (16, 256, 48, 32), (17, 96, 33, 16), (33, 512, 130, 48),
    (64, 320, 64, 0), (65, 1024, 129, 64), (130, 96, 257, 16), (200, 2080, 300, 64), (257, 512, 513, 128),
    (1024, 1024, 384, 64),
    # low-rank pre-pass: many K slices (decode), rank counts that are not a multiple of 64
    (16, 4096, 64, 64), (40, 1056, 100, 80), (128, 4096, 256, 192),
    # first stage with 128 ranks per workgroup (r > 64) at its three token blocks (16 / 32 / 64 by
    # M), partial rank blocks, the largest rank on both paths
    (1100, 2080, 300, 128), (4100, 320, 72, 144), (96, 512, 80, 1024), (16, 256, 64, 1024),
    # decode-sized inputs at longer K: one and a few tokens, ragged rows, no low-rank part
    (1, 2048, 48, 16), (5, 3584, 100, 64), (16, 2560, 33, 0), (11, 4096, 130, 48),
]


@pytest.mark.parametrize("M,n_in,n_out,r", SHAPES)
def test_bf16_shapes(M, n_in, n_out, r):
    L = inputs.random_case(M, n_in, n_out, r, "bf16", seed=M + n_in + n_out + r, n_outliers=2)
    check_layer(L, "bf16", f"bf16 {M}x{n_in}->{n_out} r{r}")


@pytest.mark.parametrize("M,n_in,n_out,r", [(32, 512, 512, 16), (3, 64, 20, 16), (70, 160, 33, 32), (16, 96, 8, 0)])
def test_fp32_shapes(M, n_in, n_out, r):
    L = inputs.random_case(M, n_in, n_out, r, "fp32", seed=M * n_in + r)
    check_layer(L, "fp32", f"fp32 {M}x{n_in}->{n_out} r{r}")


@pytest.mark.parametrize("cfg", ["C1", "C2", "C3"])
def test_named_full(cfg):
    c = configs.get(cfg)
    L = inputs.make_layer(cfg, 0)
    check_layer(L, c.dtype, cfg)


def sampled_rows(M, seed, tile=128):
    """Token rows the oracle evaluates on a full-size layer: at least one row in every 128-token
    tile of the prefill kernel (its position inside the tile varies from tile to tile, so every
    16-token fragment row and every lane position is met), the edges of the first and last tiles,
    and a few random rows. Every output column of a sampled row is compared."""
    g = np.random.default_rng(seed)
    per_tile = [t * tile + (37 * t + 5) % min(tile, M - t * tile) for t in range((M + tile - 1) // tile)]
    edges = [0, 1, 15, 16, 127, 128, 255, M - 129, M - 128, M - 1]
    return np.unique(np.clip(np.concatenate([per_tile, edges, g.integers(0, M, size=16)]), 0, M - 1))


def test_sampled_rows_cover_every_tile():
    rows = sampled_rows(8192, 5)
    assert set(rows // 128) == set(range(64))
    assert len(set(rows % 16)) == 16


@pytest.mark.parametrize("cfg", ["C4", "C5"])
def test_named_sampled_rows(cfg):
    """Full-size layers (the benchmark's launch configuration); the oracle evaluates sampled token
    rows (one or more in every 128-token tile, tile edges, random ones), each compared element by
    element over all output columns."""
    c = configs.get(cfg)
    rows = sampled_rows(c.M, c.config_id)
    for li in range(len(c.layers)):
        L = inputs.make_layer(cfg, li)
        check_layer(L, c.dtype, f"{cfg}/{L.name}", rows=rows)


# shapes that take the 512-row prefill tile (at least 256 tiles of 512 rows x 128 tokens): ragged
# tokens, rows and K (a 32-column tail), K shorter than the unrolled loop (padding steps), partial
# rank blocks; compared on one row in every 128-token tile
# the 512-row tile: ragged rows and tokens, K tails, rank 0, one and two 64-rank blocks before the
# main loop (16, 80, 128) and further blocks after it (144: a partial one; 192), both Y epilogues
WIDE = [(4100, 2080, 4100, 80), (8192, 96, 4104, 16), (4096, 448, 8192, 0), (4224, 4096, 4096, 128),
        (4096, 1056, 4100, 192), (4160, 544, 4096, 144),
        # Y above 96 MiB (also the second and third shape): non-temporal token-row stores through LDS;
        # a 4-row last tile, and rows
        # not a multiple of 4 (every store per element)
        (8192, 96, 6148, 16), (8200, 96, 6150, 16)]


@pytest.mark.parametrize("M,n_in,n_out,r", WIDE)
def test_bf16_wide_tile(M, n_in, n_out, r):
    assert -(-n_out // 512) * -(-M // 128) >= 256
    L = inputs.random_case(M, n_in, n_out, r, "bf16", seed=M + n_in + n_out + r, n_outliers=2)
    check_layer(L, "bf16", f"bf16 wide {M}x{n_in}->{n_out} r{r}", rows=sampled_rows(M, 11))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("M", [16, 200])
def test_special_cases(dtype, M):
    n_in, n_out, r = 512, 192, 32
    L = inputs.random_case(M, n_in, n_out, r, dtype, seed=77)
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    v, m = from_dev(vd, dtype), meta_from_dev(md)
    Xd, Ud, Vd = to_dev(L.X, dtype), to_dev(L.U, dtype), to_dev(L.V, dtype)

    # S = 0: only the low-rank path. float32 operands: the 1e-5 bar. bfloat16 operands: T = X V^T
    # is carried as a bfloat16 pair hi + lo with |T - hi - lo| <= 2^-18 |T| per element, so the
    # largest output error is a small multiple of 2^-18 rms(Y); 4e-5 (~10 x 2^-18) bounds it.
    zv = torch.zeros_like(vd)
    Y = binding.linear(Xd, zv, md, Ud, Vd).cpu().numpy()
    ref = oracle.linear(L.X, np.zeros_like(v), m, n_out, L.U, L.V, dtype)
    assert rel_err(Y, ref) <= (1e-5 if dtype == "fp32" else 4e-5), "S = 0"
    # U = 0 and r = 0: only the sparse product
    Y0 = binding.linear(Xd, vd, md, torch.zeros_like(Ud), Vd).cpu().numpy()
    Yr0 = binding.linear(Xd, vd, md, None, None, n_out=n_out).cpu().numpy()
    ref = oracle.linear(L.X, v, m, n_out, None, None, dtype)
    assert rel_err(Y0, ref) <= (1e-5 if dtype == "fp32" else TIGHT), "U = 0"
    assert np.array_equal(Y0, Yr0), "U = 0 and r = 0 differ"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_identity_input(dtype):
    """X = I (M = n_in): Y is the transposed reconstruction S + U V."""
    n_in, n_out, r = 128, 96, 16
    L = inputs.random_case(n_in, n_in, n_out, r, dtype, seed=5)
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    eye = to_dev(inputs.from_f64(np.eye(n_in), dtype), dtype)
    Y = binding.linear(eye, vd, md, to_dev(L.U, dtype), to_dev(L.V, dtype)).cpu().numpy()
    W = oracle.dense_reconstruct(from_dev(vd, dtype), meta_from_dev(md), n_out, n_in, L.U, L.V, dtype)
    assert rel_err(Y, W.T) <= 1e-5


@pytest.mark.parametrize("M,n_in", [(16, 512), (48, 512), (256, 512), (16, 2048), (3, 4096)])
def test_integer_exact_bitwise(M, n_in):
    """Small integers make every product and partial sum exact in float32 (all < 2^24): the GPU
    result must equal the oracle exactly, for both kernels (decode M <= 64, prefill above) and
    K up to 4096."""
    dtype, n_out, r = "bf16", 160, 16
    X = inputs.small_integers((M, n_in), -4, 4, dtype, seed=M, tensor_id=0)
    U = inputs.small_integers((n_out, r), -2, 2, dtype, seed=M, tensor_id=2)
    V = inputs.small_integers((r, n_in), -2, 2, dtype, seed=M, tensor_id=3)
    R = inputs.small_integers((n_out, n_in), -4, 4, dtype, seed=M, tensor_id=1)
    v_ref, m_ref = oracle.prune24_pack(R, dtype)
    ref = oracle.linear(X, v_ref, m_ref, n_out, U, V, dtype)
    vd, md = binding.prune24_pack(to_dev(R, dtype))
    Y = binding.linear(to_dev(X, dtype), vd, md, to_dev(U, dtype), to_dev(V, dtype)).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), ref)


@pytest.mark.parametrize("r", [16, 80, 144, 256])
def test_integer_exact_bitwise_wide_tile(r):
    """The 512-row prefill tile on small integers (every sum exact in float32): sampled rows equal
    the oracle exactly, and two runs agree bit for bit."""
    dtype, M, n_in, n_out = "bf16", 4096, 544, 4096
    print(f"[linear] integer wide tile r={r}", flush=True)
    X = inputs.small_integers((M, n_in), -4, 4, dtype, seed=r, tensor_id=0)
    U = inputs.small_integers((n_out, r), -2, 2, dtype, seed=r, tensor_id=2)
    V = inputs.small_integers((r, n_in), -2, 2, dtype, seed=r, tensor_id=3)
    R = inputs.small_integers((n_out, n_in), -4, 4, dtype, seed=r, tensor_id=1)
    rows = sampled_rows(M, 12)
    v_ref, m_ref = oracle.prune24_pack(R, dtype)
    ref = oracle.linear(X, v_ref, m_ref, n_out, U, V, dtype, rows=rows)
    vd, md = binding.prune24_pack(to_dev(R, dtype))
    Xd, Ud, Vd = to_dev(X, dtype), to_dev(U, dtype), to_dev(V, dtype)
    Y = binding.linear(Xd, vd, md, Ud, Vd).cpu().numpy()
    Y2 = binding.linear(Xd, vd, md, Ud, Vd).cpu().numpy()
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32))
    assert np.array_equal(Y[rows].astype(np.float64), ref)


def test_balanced_scale_lowrank():
    """U V as large as W: the rank-r term is no longer a small correction."""
    dtype, M, n_in, n_out, r = "bf16", 256, 1024, 320, 64
    uv_std = np.sqrt(0.02) / r ** 0.25
    L = inputs.random_case(M, n_in, n_out, r, dtype, seed=9, uv_std=uv_std, n_outliers=8)
    check_layer(L, dtype, "balanced")


def test_deterministic():
    L = inputs.random_case(300, 1024, 256, 64, "bf16", seed=3)
    Xd, Ud, Vd = to_dev(L.X, "bf16"), to_dev(L.U, "bf16"), to_dev(L.V, "bf16")
    vd, md = binding.prune24_pack(to_dev(L.R, "bf16"))
    Y1 = binding.linear(Xd, vd, md, Ud, Vd)
    Y2 = binding.linear(Xd, vd, md, Ud, Vd)
    assert torch.equal(Y1, Y2)
    Xs = Xd[:16].contiguous()
    Y3 = binding.linear(Xs, vd, md, Ud, Vd)
    Y4 = binding.linear(Xs, vd, md, Ud, Vd)
    assert torch.equal(Y3, Y4)


def test_workspace_errors():
    L = inputs.random_case(64, 256, 64, 32, "bf16", seed=1)
    Xd, Ud, Vd = to_dev(L.X, "bf16"), to_dev(L.U, "bf16"), to_dev(L.V, "bf16")
    vd, md = binding.prune24_pack(to_dev(L.R, "bf16"))
    need = binding.workspace_bytes(64, 64, 256, 32, torch.bfloat16)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.SplrError) as e:
        binding.linear(Xd, vd, md, Ud, Vd, workspace=small)
    assert e.value.status == 6


@pytest.mark.parametrize("dtype,M,n_in,n_out,r", [("bf16", 200, 2080, 300, 64), ("bf16", 16, 4096, 64, 64),
                                                  ("bf16", 65, 512, 96, 0), ("fp32", 70, 160, 33, 32)])
def test_stages_equal_linear(dtype, M, n_in, n_out, r):
    """splr_linear_stage1 then splr_linear_stage2 give splr_linear's Y bit for bit."""
    print(f"[stages] dtype={dtype} M={M} n_in={n_in} n_out={n_out} r={r}", flush=True)
    L = inputs.random_case(M, n_in, n_out, r, dtype, seed=77, n_outliers=2)
    Xd, Ud, Vd = to_dev(L.X, dtype), to_dev(L.U if r else None, dtype), to_dev(L.V if r else None, dtype)
    vd, md = binding.prune24_pack(to_dev(L.R, dtype))
    Y1 = binding.linear(Xd, vd, md, Ud, Vd, n_out=n_out)
    ws = binding.new_workspace(M, n_out, n_in, r, Xd.dtype, Xd.device)
    binding.linear_stage1(Xd, Vd, ws)
    Y2 = binding.linear_stage2(Xd, vd, md, Ud, ws, n_out=n_out)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int32), Y2.view(torch.int32))


def test_workspace_reuse_across_shapes():
    """One workspace serves calls of different shapes in a row (K split into slices or not, ragged
    token counts): each gives the same Y, bit for bit, as a call with a fresh workspace, whatever
    the previous call left in it."""
    shapes = [(2048, 4096, 256, 64), (16, 4096, 128, 64), (40, 1056, 100, 80), (300, 2080, 96, 128),
              (128, 4096, 256, 192), (16, 4096, 128, 64)]
    need = max(binding.workspace_bytes(M, n_out, n_in, r, torch.bfloat16) for M, n_in, n_out, r in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage: NaN-like floats
    for i, (M, n_in, n_out, r) in enumerate(shapes):
        print(f"[reuse] call {i}: M={M} n_in={n_in} n_out={n_out} r={r}", flush=True)
        L = inputs.random_case(M, n_in, n_out, r, "bf16", seed=100 + i, n_outliers=2)
        Xd, Ud, Vd = to_dev(L.X, "bf16"), to_dev(L.U, "bf16"), to_dev(L.V, "bf16")
        vd, md = binding.prune24_pack(to_dev(L.R, "bf16"))
        Y_shared = binding.linear(Xd, vd, md, Ud, Vd, n_out=n_out, workspace=ws)
        Y_fresh = binding.linear(Xd, vd, md, Ud, Vd, n_out=n_out)
        torch.cuda.synchronize()
        assert torch.equal(Y_shared.view(torch.int32), Y_fresh.view(torch.int32))
