"""End-to-end parity of the HIP path (through the C-ABI) with the oracle."""
import numpy as np
import pytest

from kv_cached_flow_amd import configs, inputs
from oracle import wam_oracle as O
from tests._util import gpu_cache_layer, print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu


def _run_gpu(cfg, inp):
    import torch
    from kv_cached_flow_amd.runner import DeviceChunk
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


def _oracle(cfg, inp):
    return O.run_chunk(cfg, inp, keep_cache=True)


def test_c0_fp32_every_output():
    cfg = configs.get("C0")
    print_case("C0 fp32 end-to-end")
    inp = inputs.generate(cfg)
    ref = _oracle(cfg, inp)
    dc = _run_gpu(cfg, inp)
    T = cfg.tokens_valid
    assert int(dc.cache.len[0]) == T
    for l in range(cfg.L):
        k, v = gpu_cache_layer(dc, l, 0, T)
        assert rel_l2(k, ref["cache"][0][l][0].numpy()) <= 1e-5
        assert rel_l2(v, ref["cache"][0][l][1].numpy()) <= 1e-5
    assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= 1e-5
    assert rel_l2(to_np(dc.vhat), ref["vhat"]) <= 1e-5
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= 1e-5


SMALL = dict(L=2, D=256, Hh=4, Fm=512, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4),
             pad_frames=1, V=2, N=3, read_map=(0, 1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_ragged(dtype):
    # several tiles on every axis with ragged tails (P = 100, one padded frame)
    cfg = configs.small("S", dtype=dtype, **SMALL)
    print_case(f"small ragged {dtype}")
    inp = inputs.generate(cfg)
    ref = _oracle(cfg, inp)
    dc = _run_gpu(cfg, inp)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= tol
    T = cfg.tokens_valid
    for l in range(cfg.L):
        k, v = gpu_cache_layer(dc, l, 0, T)
        assert rel_l2(k, ref["cache"][0][l][0].numpy()) <= (1e-5 if dtype == "f32" else 1e-2)
        assert rel_l2(v, ref["cache"][0][l][1].numpy()) <= (1e-5 if dtype == "f32" else 1e-2)
