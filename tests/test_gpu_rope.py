"""The rotary position option through the C-ABI against the oracle: Q and K
of both experts rotated by their token's index in the episode's joint
sequence, the cached K rotated, for the IDM chunk (dense and SparseMoT),
co-denoising, two episodes of different lengths and a streamed history."""
import pytest
import torch

from kv_cached_flow_amd import configs, inputs, wam
from kv_cached_flow_amd.runner import DeviceChunk
from oracle import wam_oracle as O
from tests._util import gpu_cache_layer, print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu

SMALL = dict(L=2, D=256, Hh=4, Fm=512, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4),
             pad_frames=1, V=2, N=3, read_map=(0, 1), rope=True)


def _run(cfg, inp):
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


def _check_chunk(cfg, inp, dc, ref, tol, ktol):
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


@pytest.mark.parametrize("dtype,dh", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_chunk_with_rotary_positions(dtype, dh):
    kw = dict(SMALL, Hh=256 // dh, dh=dh)
    cfg = configs.small("R", dtype=dtype, **kw)
    print_case(f"rotary option, {dtype}, dh {dh}")
    inp = inputs.generate(cfg)
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    tol, ktol = (1e-5, 1e-5) if dtype == "f32" else (2e-2, 1e-2)
    _check_chunk(cfg, inp, _run(cfg, inp), ref, tol, ktol)
    # the option changes the result (not a no-op on either side)
    base = O.run_chunk(configs.small("R0", dtype=dtype, **dict(kw, rope=False)), inp)
    assert rel_l2(base["actions"], ref["actions"]) > 1e-3


def test_rotary_two_episodes_of_different_lengths():
    # episode 1 has no padded frame: its future rows and action tokens sit
    # 100 positions later than episode 0's
    cfg = configs.small("RB", dtype="bf16", **dict(SMALL, B=2))
    print_case("rotary option, B=2 of different lengths")
    inp = inputs.generate(cfg)
    inp["hist_valid"] = inp["hist_valid"].copy()
    inp["hist_valid"][1, :] = 1
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    _check_chunk(cfg, inp, _run(cfg, inp), ref, 2e-2, 1e-2)


def test_rotary_sparse_mot():
    cfg = configs.small("RS", dtype="bf16", **dict(SMALL, L=4, V=0, read_map=(-1, 0, -1, 1),
                                                    fuse=((0, 2), (2, 2))))
    print_case("rotary option, SparseMoT")
    inp = inputs.generate(cfg)
    ref = O.run_chunk(cfg, inp)
    dc = _run(cfg, inp)
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= 2e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rotary_codenoise(dtype):
    cfg = configs.small("RJ", dtype=dtype, **dict(SMALL, V=3, joint=True))
    print_case(f"rotary option, co-denoising, {dtype}")
    inp = inputs.generate(cfg)
    ref = O.run_codenoise(cfg, inp)
    dc = _run(cfg, inp)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= tol
    assert rel_l2(to_np(dc.z).reshape(ref["z"].shape), ref["z"]) <= tol


@pytest.mark.parametrize("dh", [64, 128])
def test_rotary_streamed_history(dh):
    # frames appended one block at a time keep their positions: the streamed
    # chunk equals the oracle's one-prefill chunk
    cfg = configs.small("RST", dtype="f32", **dict(SMALL, Fh=4, frame_block=(0, 1, 2, 3, 4, 5),
                                                    Hh=256 // dh, dh=dh))
    print_case(f"rotary option, streamed history (1, 1, 2 frames), dh {dh}")
    inp = inputs.generate(cfg)
    dc = DeviceChunk(cfg, inp)
    d, B = dc.dims, cfg.B
    hv = dc.hist_valid
    dc.cache.len[:] = 0
    done = 0
    for n in (1, 1, 2):
        wam.extend_history_cache(d, dc.video, dc.hist[:, done:done + n].contiguous(), hv[:, :done + n], B,
                                 done, n, cfg.frame_block[:done + n], dc.cache)
        done += n
    wam.prefill_future(d, dc.video, hv, B, cfg.Fh, dc.fut, cfg.Ff, cfg.frame_block, cfg.V,
                       cfg.sigma_star, cfg.shift, dc.cache, dc.z)
    dc.fuse()
    dc.denoise()
    torch.cuda.synchronize()
    ref = O.run_chunk(cfg, inp, keep_cache=True)
    _check_chunk(cfg, inp, dc, ref, 1e-5, 1e-5)
