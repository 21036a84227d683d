"""Co-denoising (CoD) through the C-ABI against the oracle: the history
prefill, then N joint video + action Euler steps over [history ; future at
the step's video level]."""
import json
import os

import numpy as np
import pytest

from kv_cached_flow_amd import configs, inputs
from oracle import wam_oracle as O
from tests._util import gpu_cache_layer, print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu

SMALL = dict(L=2, D=256, Hh=4, Fm=512, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4),
             pad_frames=1, V=3, N=3, read_map=(0, 1), joint=True)


def _run_gpu(cfg, inp):
    import torch
    from kv_cached_flow_amd.runner import DeviceChunk
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


def _check_all(cfg, inp, dc, tol, ktol):
    ref = O.run_codenoise(cfg, inp, keep_cache=True)
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= tol
    assert rel_l2(to_np(dc.vhat), ref["vhat"]) <= tol
    assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= tol
    for b in range(cfg.B):
        T = int(dc.cache.len[b])
        assert T == ref["cache"][b][0][0].shape[0]
        for l in range(cfg.L):
            k, v = gpu_cache_layer(dc, l, b, T)
            assert rel_l2(k, ref["cache"][b][l][0].numpy()) <= ktol
            assert rel_l2(v, ref["cache"][b][l][1].numpy()) <= ktol


def test_codenoise_c0_fp32():
    cfg = configs.get("C0", joint=True)
    print_case("CoD C0 fp32")
    inp = inputs.generate(cfg)
    _check_all(cfg, inp, _run_gpu(cfg, inp), 1e-5, 1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_codenoise_small_ragged(dtype):
    # P = 100 (ragged tiles), one padded history frame, 3 joint steps
    cfg = configs.small("J", dtype=dtype, **SMALL)
    print_case(f"CoD small ragged {dtype}")
    inp = inputs.generate(cfg)
    tol = 1e-5 if dtype == "f32" else 2e-2
    _check_all(cfg, inp, _run_gpu(cfg, inp), tol, 1e-5 if dtype == "f32" else 1e-2)


def test_codenoise_video_end_and_batch():
    # two episodes with different padding, video stopping at 0.5
    cfg = configs.small("J2", dtype="bf16", **dict(SMALL, B=2, video_end=0.5))
    print_case("CoD B=2, video to 0.5")
    inp = inputs.generate(cfg)
    inp["hist_valid"] = inp["hist_valid"].copy()
    inp["hist_valid"][1, :] = 1
    _check_all(cfg, inp, _run_gpu(cfg, inp), 2e-2, 1e-2)


def test_codenoise_video_equals_imagine_bitwise():
    # video rows never read actions: CoD to 0.9 in V steps moves the future
    # latents exactly as the IDM imagine steps do (same kernels, same order)
    import torch
    cod = configs.small("JV", dtype="bf16", **dict(SMALL, video_end=0.9, V=3, N=3))
    idm = configs.small("IV", dtype="bf16", **dict(SMALL, joint=False, V=3, N=3))
    inp = inputs.generate(cod)
    a = _run_gpu(cod, inp)
    b = _run_gpu(idm, inp)
    assert torch.equal(a.z, b.z)


def test_codenoise_batch_independence_bitwise():
    import torch
    cfg2 = configs.small("JB2", dtype="bf16", **dict(SMALL, B=2))
    inp2 = inputs.generate(cfg2)
    both = _run_gpu(cfg2, inp2)
    for b in range(2):
        one = {k: (v[b:b + 1] if k in ("hist", "hist_valid", "eps_v", "eps_a") else v)
               for k, v in inp2.items()}
        single = _run_gpu(configs.small("JB1", dtype="bf16", **SMALL), one)
        assert torch.equal(both.actions[b], single.actions[0])
        assert torch.equal(both.z[b], single.z[0])


def test_codenoise_no_history():
    # every history frame padded: the joint steps see the future alone
    cfg = configs.small("JNH", dtype="f32", **dict(SMALL, pad_frames=3))
    inp = inputs.generate(cfg)
    _check_all(cfg, inp, _run_gpu(cfg, inp), 1e-5, 1e-5)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_codenoise_full_size_against_oracle_values():
    path = os.path.join(GOLDEN, "C5.json")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_golden.py C5)")
    g = json.load(open(path))
    cfg = configs.get("C5")
    print_case("full size C5 (CoD)")
    inp = inputs.generate(cfg)
    assert inputs.fingerprint(inp) == g["fingerprint"]
    dc = _run_gpu(cfg, inp)
    err = rel_l2(to_np(dc.actions), np.array(g["actions"]))
    print_case(f"C5 final actions rel-L2 {err:.3e}")
    assert err <= 2e-2
    rows, heads = np.array(g["sample_rows"]), np.array(g["sample_heads"])
    for l in g["sample_layers"]:
        ent = g["cache"][0][str(l)]
        k = to_np(dc.cache.k[l, 0])[heads, rows]
        v = to_np(dc.cache.v[l, 0]).transpose(0, 2, 1)[heads, rows]
        assert rel_l2(k, np.array(ent["k"])) <= 1e-2
        assert rel_l2(v, np.array(ent["v"])) <= 1e-2
    zr = np.array(g["z_rows"])
    z = to_np(dc.z).reshape(cfg.B, -1, cfg.Cv)[:, zr]
    assert rel_l2(z, np.array(g["z"])) <= 2e-2


def test_codenoise_reads_only_written_memory():
    """C5 shapes with 2 layers, cache and workspaces poisoned (NaN / 0xFF):
    every cache row below len, the latents and the actions come out finite."""
    import torch
    from kv_cached_flow_amd.runner import DeviceChunk
    cfg = configs.get("C5", L=2, read_map=(0, 1))
    print_case("C5 shapes, 2 layers, poisoned buffers")
    inp = inputs.generate(cfg)
    dc = DeviceChunk(cfg, inp)
    dc.cache.k.fill_(float("nan"))
    dc.cache.v.fill_(float("nan"))
    dc.ws_prefill.fill_(0xFF)
    dc.ws_denoise.fill_(0xFF)
    dc.run()
    torch.cuda.synchronize()
    n = int(dc.cache.len[0])
    assert n == cfg.tokens_valid
    assert torch.isfinite(dc.cache.k[:, :, :, :n].float()).all()
    assert torch.isfinite(dc.cache.v[:, :, :, :, :n].float()).all()
    assert torch.isfinite(dc.z).all()
    assert torch.isfinite(dc.actions).all()
