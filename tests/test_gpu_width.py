"""Experts of different widths over one attention interface (the action
expert narrower or wider than Hh x dh, its own MLP width) against the oracle,
for the IDM chunk and for co-denoising."""
import json
import os

import numpy as np
import pytest
import torch

from kv_cached_flow_amd import configs, inputs
from kv_cached_flow_amd.runner import DeviceChunk
from oracle import wam_oracle as O
from tests._util import gpu_cache_layer, print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu

SMALL = dict(L=2, D=256, Hh=4, dh=64, Fm=512, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4),
             pad_frames=1, V=2, N=3, read_map=(0, 1))


def _run(cfg, inp):
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


@pytest.mark.parametrize("dtype,Da,Fma", [("f32", 128, 384), ("bf16", 512, 768), ("bf16", 1024, 256)])
def test_chunk_with_an_action_expert_of_its_own_width(dtype, Da, Fma):
    cfg = configs.small("W", dtype=dtype, **dict(SMALL, Da=Da, Fma=Fma))
    print_case(f"action width {Da}, MLP {Fma}, {dtype}")
    inp = inputs.generate(cfg)
    assert inp["action"]["layers"][0]["wqkv"].shape == (3 * cfg.Dq, Da)
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    dc = _run(cfg, inp)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= tol
    assert rel_l2(to_np(dc.vhat), ref["vhat"]) <= tol
    T = cfg.tokens_valid
    k, v = gpu_cache_layer(dc, 1, 0, T)
    assert rel_l2(k, ref["cache"][0][1][0].numpy()) <= (1e-5 if dtype == "f32" else 1e-2)


def test_codenoise_with_an_action_expert_of_its_own_width():
    cfg = configs.small("WJ", dtype="bf16", **dict(SMALL, Da=512, Fma=768, joint=True))
    print_case("co-denoising, action width 512")
    inp = inputs.generate(cfg)
    ref = O.run_codenoise(cfg, inp)
    dc = _run(cfg, inp)
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= 2e-2
    assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= 2e-2


# 128-wide heads: the attention tiles of both experts change shape
WIDE = dict(SMALL, D=256, Hh=2, dh=128)


@pytest.mark.parametrize("dtype,Da,Fma", [("f32", 0, 0), ("bf16", 0, 0), ("bf16", 512, 768)])
def test_chunk_with_128_wide_heads(dtype, Da, Fma):
    cfg = configs.small("H128", dtype=dtype, **dict(WIDE, Da=Da, Fma=Fma))
    print_case(f"dh 128, action width {Da or cfg.D}, {dtype}")
    inp = inputs.generate(cfg)
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    dc = _run(cfg, inp)
    tol, ktol = (1e-5, 1e-5) if dtype == "f32" else (2e-2, 1e-2)
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= tol
    assert rel_l2(to_np(dc.vhat), ref["vhat"]) <= tol
    assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= tol
    T = cfg.tokens_valid
    for l in range(cfg.L):
        k, v = gpu_cache_layer(dc, l, 0, T)
        assert rel_l2(k, ref["cache"][0][l][0].numpy()) <= ktol
        assert rel_l2(v, ref["cache"][0][l][1].numpy()) <= ktol


def test_codenoise_with_128_wide_heads():
    cfg = configs.small("H128J", dtype="bf16", **dict(WIDE, Hh=4, D=512, Da=256, Fma=512, joint=True))
    print_case("co-denoising, 4 x 128 heads, action width 256")
    inp = inputs.generate(cfg)
    ref = O.run_codenoise(cfg, inp)
    dc = _run(cfg, inp)
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= 2e-2
    assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= 2e-2


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_real_widths_full_size_against_oracle_values():
    """C6 (3072-wide video expert with 24 x 128 heads, 1024-wide action
    expert) against the oracle's stored values."""
    path = os.path.join(GOLDEN, "C6.json")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_golden.py C6)")
    g = json.load(open(path))
    cfg = configs.get("C6")
    print_case("full size C6 (real widths)")
    inp = inputs.generate(cfg)
    assert inputs.fingerprint(inp) == g["fingerprint"]
    dc = _run(cfg, inp)
    err = rel_l2(to_np(dc.actions), np.array(g["actions"]))
    print_case(f"C6 final actions rel-L2 {err:.3e}")
    assert err <= 2e-2
    rows, heads = np.array(g["sample_rows"]), np.array(g["sample_heads"])
    for l in g["sample_layers"]:
        ent = g["cache"][0][str(l)]
        k = to_np(dc.cache.k[l, 0])[heads, rows]
        v = to_np(dc.cache.v[l, 0]).transpose(0, 2, 1)[heads, rows]
        assert rel_l2(k, np.array(ent["k"])) <= 1e-2
        assert rel_l2(v, np.array(ent["v"])) <= 1e-2
