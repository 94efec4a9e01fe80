"""GPU parity of splr_prune24_pack: values and metadata bit-identical to the oracle's."""
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_rank_linear_prune24_amd import binding, configs, inputs
from tests._helpers import from_dev, meta_from_dev, to_dev

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
NP = {"fp32": np.float32, "bf16": np.uint16}


def gpu_pack(R, dtype):
    v, m = binding.prune24_pack(to_dev(R, dtype))
    torch.cuda.synchronize()
    return from_dev(v, dtype), meta_from_dev(m)


def assert_pack_equal(R, dtype, tag=""):
    print(f"[pack] {tag} dtype={dtype} shape={R.shape}", flush=True)
    v_ref, m_ref = oracle.prune24_pack(R, dtype)
    v, m = gpu_pack(R, dtype)
    bits = np.uint32 if dtype == "fp32" else np.uint16
    assert np.array_equal(m, m_ref), f"{tag}: metadata differs at {np.argwhere(m != m_ref)[:5]}"
    assert np.array_equal(v.view(bits), v_ref.view(bits)), f"{tag}: values differ"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_out,n_in", [(1, 32), (3, 96), (17, 64), (64, 512), (129, 4128), (1000, 320)])
def test_ragged_shapes(dtype, n_out, n_in):
    R = inputs.gaussian((n_out, n_in), 0.02, dtype, seed=n_out * 7 + n_in, config_id=3000)
    assert_pack_equal(R, dtype, f"gaussian {n_out}x{n_in}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ties_and_special_values(dtype):
    g = np.random.default_rng(1)
    bits_t = np.uint32 if dtype == "fp32" else np.uint16
    # small integers: dense ties, zeros of both signs
    f = g.integers(-2, 3, size=(64, 256)).astype(np.float64)
    R = inputs.from_f64(f, dtype).view(bits_t).copy()
    neg0 = bits_t(0x80000000) if dtype == "fp32" else bits_t(0x8000)
    R[g.random(R.shape) < 0.1] = neg0
    # special values sprinkled in
    specials = ([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x00000001, 0x80000002, 0x7F7FFFFF, 0x00800000]
                if dtype == "fp32" else [0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8002, 0x7F7F, 0x0080])
    idx = g.integers(0, R.size, size=2000)
    R.reshape(-1)[idx] = np.array(specials, dtype=bits_t)[g.integers(0, len(specials), size=idx.size)]
    R[5, :] = 0                      # all-zero row
    R[6, :] = neg0                   # all negative zeros
    assert_pack_equal(R.view(NP[dtype]), dtype, "ties+specials")


def test_fixture_groups():
    for dtype in ("fp32", "bf16"):
        groups = []
        with open(os.path.join(HERE, "golden", "pack_special_groups.txt")) as fh:
            for line in fh:
                line = line.split("#", 1)[0].strip()
                if line and line.split()[0] == dtype:
                    groups.append([int(t, 16) for t in line.split()[1:5]])
        bits = np.array(groups, dtype=np.uint32 if dtype == "fp32" else np.uint16).reshape(-1)
        pad = (-bits.size) % 32
        bits = np.concatenate([bits, np.zeros(pad, dtype=bits.dtype)]).reshape(-1, 32)
        assert_pack_equal(bits.view(NP[dtype]), dtype, "fixture")


@pytest.mark.parametrize("cfg", ["C1", "C2", "C4", "C5"])
def test_named_workloads(cfg):
    """Every layer of every named workload (C3 shares C2's layer), full size, bit-exact."""
    c = configs.get(cfg)
    for li in range(len(c.layers)):
        L = inputs.make_layer(cfg, li, with_x=False)
        assert_pack_equal(L.R, c.dtype, f"{cfg}/{L.name}")


def test_deterministic_and_stream_ordered():
    R = inputs.gaussian((512, 1024), 0.02, "bf16", seed=4, config_id=3001)
    Rd = to_dev(R, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        v1, m1 = binding.prune24_pack(Rd)
        v2, m2 = binding.prune24_pack(Rd)
    s.synchronize()
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16)) and torch.equal(m1, m2)


def test_validation_on_device():
    R = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.SplrError) as e:
        binding.prune24_pack(R)
    assert e.value.status == 2
    R = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        binding.prune24_pack(R)
