"""The allocation-free denoise entry (wam_denoise_chunk_noalloc) against
wam_denoise_chunk with a caller workspace, through the C-ABI: two calls in a
row on the library's static scratch, the second with a smaller input, each
bitwise equal to the workspace entry (same kernels, same split plan)."""
import pytest
import torch

from kv_cached_flow_amd import configs, inputs, wam
from kv_cached_flow_amd.runner import DeviceChunk
from tests._util import print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu


def _denoise_both(cfg):
    inp = inputs.generate(cfg)
    dc = DeviceChunk(cfg, inp)
    dc.prefill()
    dc.fuse()
    ref_a, ref_v = torch.empty_like(dc.actions), torch.empty_like(dc.vhat)
    got_a, got_v = torch.full_like(dc.actions, float("nan")), torch.full_like(dc.vhat, float("nan"))
    wam.denoise_chunk(dc.dims, dc.action, dc.read_kv, cfg.read_map, dc.eps_a, cfg.B, cfg.N, cfg.shift,
                      ref_a, ref_v, dc.ws_denoise)
    wam.denoise_chunk_noalloc(dc.dims, dc.action, dc.read_kv, cfg.read_map, dc.eps_a, cfg.B, cfg.N,
                              cfg.shift, got_a, got_v)
    torch.cuda.synchronize()
    return ref_a, ref_v, got_a, got_v


def test_noalloc_denoise_equals_the_workspace_entry_on_two_calls():
    first = configs.small("NA", dtype="bf16", L=2, D=256, Hh=4, Fm=512, P=100, Fh=3, Ff=2,
                          frame_block=(0, 1, 2, 3, 4), pad_frames=1, V=2, N=4, B=2, read_map=(0, 1))
    # the second call is smaller: one episode, fewer cached tokens and steps
    second = configs.small("NB", dtype="bf16", L=2, D=256, Hh=4, Fm=512, P=60, Fh=2, Ff=1,
                           frame_block=(0, 1, 2), pad_frames=0, V=1, N=2, B=1, read_map=(0, 1))
    for cfg in (first, second):
        print_case(f"no-allocation denoise, B={cfg.B}, N={cfg.N}")
        ra, rv, ga, gv = _denoise_both(cfg)
        assert torch.isfinite(ra).all()
        assert torch.equal(ra, ga) and torch.equal(rv, gv)


def test_noalloc_denoise_fp32_with_condition():
    cfg = configs.small("NC", dtype="f32", L=2, D=128, Hh=2, Fm=256, P=40, Fh=2, Ff=1,
                        frame_block=(0, 1, 2), pad_frames=0, V=1, N=3, B=1, read_map=(0, 1),
                        Tc=9, Ct=64, S=14)
    print_case("no-allocation denoise, fp32 with a condition")
    ra, rv, ga, gv = _denoise_both(cfg)
    assert torch.equal(ra, ga) and torch.equal(rv, gv)
    assert rel_l2(to_np(ga), to_np(ra)) == 0.0
