"""The text/state condition through the C-ABI: the condition K/V of both
experts, whole chunks (IDM, SparseMoT, co-denoising, rotary positions, two
episodes, 128-wide heads, a streamed history) and one action layer against
the oracle, and the full-size C6 chunk with the condition against the
oracle's stored values."""
import json
import os

import numpy as np
import pytest
import torch

from kv_cached_flow_amd import configs, inputs, wam
from kv_cached_flow_amd.runner import DeviceChunk, upload_expert
from oracle import wam_oracle as O
from tests._util import gpu_cache_layer, print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu

# 37 condition tokens (36 text + proprio) of width 128 from 14 state numbers
COND = dict(Tc=37, Ct=128, S=14)
SMALL = dict(L=2, D=256, Hh=4, Fm=512, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4),
             pad_frames=1, V=2, N=3, read_map=(0, 1), **COND)


def _run(cfg, inp):
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_condition_kv_vs_oracle(dtype):
    cfg = configs.small("CK", dtype=dtype, **dict(SMALL, B=2))
    print_case(f"condition K/V {dtype}")
    inp = inputs.generate(cfg)
    dc = DeviceChunk(cfg, inp)
    dc.condition()
    torch.cuda.synchronize()
    dt = O.oracle_dtype(cfg)
    tol = 1e-5 if dtype == "f32" else 1e-2
    for b in range(2):
        ctx = O.episode_condition(cfg, inp, b, dt)
        assert list(dc.cond_v.len) == [cfg.Tc] * 2 and list(dc.cond_a.len) == [cfg.Tc] * 2
        for kv, w in ((dc.cond_v, inp["video"]), (dc.cond_a, inp["action"])):
            ref = O.condition_cache(cfg, O.to_torch_expert(w, dt), ctx)
            for l in range(cfg.L):
                k, v = gpu_cache_layer(_View(kv), l, b, cfg.Tc)
                assert rel_l2(k, ref[l][0].numpy()) <= tol
                assert rel_l2(v, ref[l][1].numpy()) <= tol


class _View:
    """Lets gpu_cache_layer read a condition cache like a chunk's cache."""
    def __init__(self, kv):
        self.cache = kv


VARIANTS = {
    "idm": {},
    "sparse": dict(L=4, V=0, read_map=(-1, 0, -1, 1), fuse=((0, 2), (2, 2))),
    "two episodes": dict(B=2),
    "rope": dict(rope=True),
    "dh128": dict(Hh=2, dh=128),
    "wider action expert": dict(Da=384, Fma=768),
    "codenoise": dict(joint=True, V=2, N=2, video_end=0.0),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_with_condition_vs_oracle(variant, dtype):
    cfg = configs.small("CC", dtype=dtype, **dict(SMALL, **VARIANTS[variant]))
    print_case(f"chunk with condition {variant} {dtype}")
    inp = inputs.generate(cfg)
    ref = O.run_codenoise(cfg, inp) if cfg.joint else O.run_chunk(cfg, inp, keep_cache=True)
    dc = _run(cfg, inp)
    f32 = dtype == "f32"
    err = rel_l2(to_np(dc.actions), ref["actions"])
    print_case(f"  actions rel-L2 {err:.2e}")
    assert err <= (1e-5 if f32 else 2e-2)
    if not cfg.joint:
        T = cfg.tokens_valid
        for l in range(cfg.L):
            k, v = gpu_cache_layer(dc, l, 0, T)
            assert rel_l2(k, ref["cache"][0][l][0].numpy()) <= (1e-5 if f32 else 1e-2)
            assert rel_l2(v, ref["cache"][0][l][1].numpy()) <= (1e-5 if f32 else 1e-2)
    if cfg.V >= 1 or cfg.joint:
        assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= (1e-5 if f32 else 1e-2)


def test_condition_moves_the_chunk_and_the_state_reaches_it():
    """A different robot state changes the actions (the proprio token is
    read); the same inputs give bitwise the same chunk."""
    cfg = configs.small("CM", dtype="bf16", **SMALL)
    inp = inputs.generate(cfg)
    a = _run(cfg, inp)
    b = _run(cfg, inp)
    assert torch.equal(a.actions, b.actions)
    inp2 = dict(inp, state=inp["state"] + 1.0)
    c = _run(cfg, inp2)
    assert not torch.equal(a.actions, c.actions)
    ref2 = O.run_chunk(cfg, inp2)
    assert rel_l2(to_np(c.actions), ref2["actions"]) <= 2e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_action_layer_with_condition_vs_oracle(dtype):
    cfg = configs.small("AC", dtype=dtype, L=1, B=2, read_map=(0,), **COND)
    print_case(f"action layer with condition {dtype}")
    dt = wam.WAM_BF16 if dtype == "bf16" else wam.WAM_F32
    inp = inputs.generate(cfg)
    ex = upload_expert(inp["action"], cfg)
    rng = np.random.default_rng(41)
    lens = [300, 200]
    kv = wam.DeviceKV(1, 2, cfg.Hh, 64, 320, dt)
    rnd = lambda sh: (inputs.round_bf16(rng.standard_normal(sh).astype(np.float32)) if dtype == "bf16"
                      else rng.standard_normal(sh).astype(np.float32))
    Kc, Vc = rnd((2, cfg.Hh, 320, 64)), rnd((2, cfg.Hh, 320, 64))
    kv.k[0].copy_(torch.from_numpy(Kc))
    kv.v[0].copy_(torch.from_numpy(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2))))
    kv.len[:] = lens
    d = wam.dims(1, cfg.D, cfg.Hh, 64, cfg.Fm, cfg.Cv, cfg.A, 32, cfg.P, dt, Tc=cfg.Tc, Ct=cfg.Ct, S=cfg.S)
    cond = wam.DeviceKV(1, 2, cfg.Hh, 64, 64, dt)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(tdt).contiguous()
    wam.prefill_condition_kv(d, None, ex, dev(inp["proprio_w"]), dev(inp["text"]),
                             torch.from_numpy(inp["state"]).cuda(), 2, None, cond)
    x = rng.standard_normal((2, 32, cfg.D)).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    wam.action_layer(d, ex, 0, xd, kv, 0, 2, cond=cond, cond_layer=0)
    torch.cuda.synchronize()
    f64 = torch.float64
    lw = O.to_torch_expert(inp["action"], f64)["layers"][0]
    for b in range(2):
        ctx = O.episode_condition(cfg, inp, b, f64)
        ctxkv = (torch.tensor(Kc[b][:, : lens[b]], dtype=f64).permute(1, 0, 2),
                 torch.tensor(Vc[b][:, : lens[b]], dtype=f64).permute(1, 0, 2))
        ref, _, _ = O.layer(torch.tensor(x[b], dtype=f64), lw, cfg.Hh, ctxkv, None,
                            cond=O.condition_kv(ctx, lw, cfg.Hh))
        assert rel_l2(xd[b].cpu().numpy(), ref.numpy()) <= (1e-5 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_streamed_history_with_condition_vs_oracle(dtype):
    """Appending history frames under an unchanged condition, then the
    future: the cache equals the oracle's whole-window prefill."""
    cfg = configs.small("SC", dtype=dtype, **dict(SMALL, Fh=4, Ff=1, frame_block=(0, 1, 2, 3, 4),
                                                  pad_frames=0))
    print_case(f"streamed history with condition {dtype}")
    inp = inputs.generate(cfg)
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    dc = DeviceChunk(cfg, inp)
    dc.prepare_stream(2)
    dc.stream_decision(2)
    torch.cuda.synchronize()
    f32 = dtype == "f32"
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= (1e-5 if f32 else 2e-2)
    T = cfg.tokens_valid
    k, v = gpu_cache_layer(dc, cfg.L - 1, 0, T)
    assert rel_l2(k, ref["cache"][0][cfg.L - 1][0].numpy()) <= (1e-5 if f32 else 1e-2)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_full_size_c6_with_condition_against_oracle_values():
    path = os.path.join(GOLDEN, "C6_cond.json")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_golden.py C6+cond)")
    g = json.load(open(path))
    cfg = configs.get("C6", **configs.CONDITION)
    print_case("full size C6 with the text/state condition")
    inp = inputs.generate(cfg)
    assert inputs.fingerprint(inp) == g["fingerprint"]
    dc = _run(cfg, inp)
    err = rel_l2(to_np(dc.actions), np.array(g["actions"]))
    print_case(f"C6 with condition final actions rel-L2 {err:.3e}")
    assert err <= 2e-2
    rows, heads = np.array(g["sample_rows"]), np.array(g["sample_heads"])
    for l in g["sample_layers"]:
        ent = g["cache"][0][str(l)]
        k = to_np(dc.cache.k[l, 0])[heads, rows]
        assert rel_l2(k, np.array(ent["k"])) <= 1e-2
