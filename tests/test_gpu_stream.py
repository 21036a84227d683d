"""Streaming the history through the C-ABI: appending frames to a cached
history and then adding the future equals one prefill of the whole window,
decision after decision, and matches the oracle."""
import numpy as np
import pytest
import torch

from kv_cached_flow_amd import configs, inputs, wam
from kv_cached_flow_amd.runner import DeviceChunk
from oracle import wam_oracle as O
from tests._util import gpu_cache_layer, print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu

SMALL = dict(L=2, D=256, Hh=4, Fm=512, P=100, Fh=4, Ff=2, frame_block=(0, 1, 2, 3, 4, 5),
             pad_frames=1, V=2, N=3, read_map=(0, 1))


def _full(cfg, inp):
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


def _streamed(cfg, inp, arrivals):
    """The same chunk with the history arriving in groups of frames: each
    group is appended to the cached rows (from an empty cache), then the
    future and the action steps run."""
    dc = DeviceChunk(cfg, inp)
    d, B = dc.dims, cfg.B
    hv = dc.hist_valid
    dc.cache.len[:] = 0
    done = 0
    for n in arrivals:
        wam.extend_history_cache(d, dc.video, dc.hist[:, done:done + n].contiguous(),
                                 hv[:, :done + n], B, done, n, cfg.frame_block[:done + n], dc.cache)
        done += n
    assert done == cfg.Fh
    wam.prefill_future(d, dc.video, hv, B, cfg.Fh, dc.fut, cfg.Ff, cfg.frame_block, cfg.V,
                       cfg.sigma_star, cfg.shift, dc.cache, dc.z)
    dc.fuse()
    dc.denoise()
    torch.cuda.synchronize()
    return dc


@pytest.mark.parametrize("dtype,arrivals", [("f32", (1, 1, 2)), ("bf16", (2, 1, 1)), ("bf16", (1, 3))])
def test_streamed_history_equals_one_prefill(dtype, arrivals):
    cfg = configs.small("ST", dtype=dtype, **dict(SMALL, B=2))
    print_case(f"streamed history {dtype} {arrivals}")
    inp = inputs.generate(cfg)
    inp["hist_valid"] = inp["hist_valid"].copy()
    inp["hist_valid"][1, :] = 1                 # episode 1 without padding
    full = _full(cfg, inp)
    st = _streamed(cfg, inp, arrivals)
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    tol, ktol = (1e-5, 1e-5) if dtype == "f32" else (2e-2, 1e-2)
    for b in range(cfg.B):
        assert int(st.cache.len[b]) == int(full.cache.len[b])
        T = int(st.cache.len[b])
        for l in range(cfg.L):
            k, v = gpu_cache_layer(st, l, b, T)
            assert rel_l2(k, ref["cache"][b][l][0].numpy()) <= ktol
            assert rel_l2(v, ref["cache"][b][l][1].numpy()) <= ktol
            kf, vf = gpu_cache_layer(full, l, b, T)
            assert rel_l2(k, kf) <= ktol
    assert rel_l2(to_np(st.actions), ref["actions"]) <= tol
    assert rel_l2(to_np(st.z).reshape(ref["z"].shape), ref["z"]) <= tol


def test_decisions_over_a_growing_window():
    """Three decisions: each drops the future rows, appends the frame that
    arrived, adds the future and denoises; the last decision's actions and
    cache match one prefill of the final window (C3's frame shape, 2 layers)
    on the GPU and the oracle's chunk over that window."""
    cfg = configs.get("C3", L=2, read_map=(0, 1), Fh=6, Ff=2, frame_block=tuple(range(8)), N=2, V=2)
    print_case("three streamed decisions, 880-token frames")
    inp = inputs.generate(cfg)
    dc = DeviceChunk(cfg, inp)
    d, P = dc.dims, cfg.P
    hv = dc.hist_valid
    wam.prefill_video_cache(d, dc.video, dc.hist[:, :3].contiguous(), hv[:, :3], 1, 3, None, 0,
                            cfg.frame_block[:3], 0, cfg.sigma_star, cfg.shift, dc.cache)
    for done in (3, 4, 5):
        dc.cache.len[:] = int(hv[0, :done].sum()) * P       # drop the previous decision's future
        wam.extend_history_cache(d, dc.video, dc.hist[:, done:done + 1].contiguous(), hv[:, :done + 1],
                                 1, done, 1, cfg.frame_block[:done + 1], dc.cache)
        fut_blocks = cfg.frame_block[:done + 1] + cfg.frame_block[6:8]
        wam.prefill_future(d, dc.video, hv[:, :done + 1], 1, done + 1, dc.fut, 2, fut_blocks, cfg.V,
                           cfg.sigma_star, cfg.shift, dc.cache, dc.z)
        dc.denoise()
    torch.cuda.synchronize()
    full = _full(cfg, inp)
    assert torch.equal(dc.z, full.z) or rel_l2(to_np(dc.z), to_np(full.z)) <= 1e-2
    assert rel_l2(to_np(dc.actions), to_np(full.actions)) <= 2e-2
    T = int(full.cache.len[0])
    assert int(dc.cache.len[0]) == T
    for l in range(cfg.L):
        k, _ = gpu_cache_layer(dc, l, 0, T)
        kf, _ = gpu_cache_layer(full, l, 0, T)
        assert rel_l2(k, kf) <= 1e-2
    # and against the oracle: its streamed history is pinned to one prefill of
    # the final window, so the last decision must land on the oracle's chunk
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    err = rel_l2(to_np(dc.actions), ref["actions"])
    zerr = rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"])
    print(f"three decisions against the oracle: rel L2 actions {err:.2e}, future latents {zerr:.2e}")
    assert err <= 2e-2 and zerr <= 1e-2
    for l in range(cfg.L):
        k, v = gpu_cache_layer(dc, l, 0, T)
        assert rel_l2(k, ref["cache"][0][l][0].numpy()) <= 1e-2
        assert rel_l2(v, ref["cache"][0][l][1].numpy()) <= 1e-2
