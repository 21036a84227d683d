"""The E4M3 cache option through the C-ABI: quantisation bit-exact against
the oracle's codec, the attention over an E4M3 cache bitwise equal to the
bf16 attention over the same dequantised values, and whole chunks against
the oracle with the option on."""
import json
import os

import numpy as np
import pytest
import torch

from kv_cached_flow_amd import configs, inputs, wam
from oracle import wam_oracle as O
from tests._util import print_case, rel_l2, to_np

pytestmark = pytest.mark.gpu

# byte p of a V^T tile row holds key LANE[p]; byte p of a K row holds dim lane_k(dh)[p]
LANE = np.array([32 * ss + 8 * g + j for g in range(4) for ss in range(2) for j in range(8)])


def lane_k(dh):
    return np.array([64 * u + 32 * ss + 8 * g + j for g in range(4) for u in range(dh // 64)
                     for ss in range(2) for j in range(8)])


def _bf16(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).float().numpy()


def _case(rng, B, Hh, lens, cap, dh=64):
    K = _bf16(rng.standard_normal((B, Hh, cap, dh)))
    V = _bf16(rng.standard_normal((B, Hh, cap, dh)))
    K[0, 0, 64:128] *= 1e-3          # a tile with its own small scale
    V[0, 1, :64] = 0.0               # an all-zero tile
    K[-1, -1, :64] *= 4.0            # and a large one
    # tiles whose largest value is about 1e-37 (below 448 * 2^-127, so the
    # scale exponent stays at -126); every value a normal number
    tiny = lambda a: np.sign(a) * np.maximum(np.abs(a), 0.25) * 1e-37
    K[0, 1 % Hh, :64] = tiny(K[0, 1 % Hh, :64])
    V[0, 2 % Hh, :64] = tiny(V[0, 2 % Hh, :64])
    K, V = _bf16(K), _bf16(V)        # the values the bf16 cache holds
    for b, n in enumerate(lens):
        K[b, :, n:] = np.nan         # rows past len must never be read
        V[b, :, n:] = np.nan
    return K, V


def _device_caches(K, V, lens, cap):
    B, Hh, _, dh = K.shape
    src = wam.DeviceKV(1, B, Hh, dh, cap, wam.WAM_BF16)
    src.k.copy_(torch.tensor(K[None]).to(torch.bfloat16))
    src.v.copy_(torch.tensor(np.ascontiguousarray(V.transpose(0, 1, 3, 2))[None]).to(torch.bfloat16))
    src.len[:] = lens
    dst = wam.DeviceKV(1, B, Hh, dh, cap, wam.WAM_FP8)
    dst.k.fill_(0x7F)                 # NaN codes: every byte read must have been written
    dst.v.fill_(0x7F)
    wam.quantize_kv_fp8(src, dst)
    torch.cuda.synchronize()
    return src, dst


def _codes_in_order(dst, b, n):
    """(codes_K [n, Hh, dh], codes_V [n, Hh, dh]) of episode b in dim/key order."""
    k8 = dst.k[0, b, :, :n].cpu().numpy()                       # [Hh, n, dh bytes]
    ck = np.empty_like(k8)
    ck[:, :, lane_k(k8.shape[2])] = k8
    v8 = dst.v[0, b].cpu().numpy()                             # [Hh, dh dims, cap bytes]
    nt = (n + 63) // 64
    cv = np.empty((v8.shape[0], v8.shape[1], nt * 64), dtype=np.uint8)
    for t in range(nt):
        cv[:, :, 64 * t + LANE] = v8[:, :, 64 * t:64 * t + 64]
    return ck.transpose(1, 0, 2), cv[:, :, :n].transpose(2, 0, 1)


@pytest.mark.parametrize("dh", [64, 128])
def test_quantize_bit_exact_against_oracle(dh):
    rng = np.random.default_rng(11)
    lens, cap = [150, 64, 1], 192
    print_case(f"E4M3 quantisation vs the oracle codec, dh {dh}")
    K, V = _case(rng, 3, 3, lens, cap, dh)
    _, dst = _device_caches(K, V, lens, cap)
    assert list(dst.len) == lens
    for b, n in enumerate(lens):
        Kt = torch.tensor(K[b, :, :n].transpose(1, 0, 2), dtype=torch.float64)
        Vt = torch.tensor(V[b, :, :n].transpose(1, 0, 2), dtype=torch.float64)
        _, _, (ck, ek, cv, ev) = O.quantize_kv_fp8(Kt, Vt)
        gk, gv = _codes_in_order(dst, b, n)
        assert np.array_equal(gk, ck)
        assert np.array_equal(gv, cv)
        nt = (n + 63) // 64
        assert np.array_equal(dst.k_scale[0, b, :, :nt].cpu().numpy(), 2.0 ** ek)
        assert np.array_equal(dst.v_scale[0, b, :, :nt].cpu().numpy(), 2.0 ** ev)
        # rows past len in the last tile hold code 0
        if n % 64:
            t0 = n // 64 * 64
            assert not dst.k[0, b, :, n:t0 + 64].any()
            vt = dst.v[0, b, :, :, t0:t0 + 64].cpu().numpy()
            keys = t0 + LANE
            assert not vt[:, :, keys >= n].any()


def _dequant_bf16_cache(dst, lens, cap):
    """A bf16 cache holding exactly the values the E4M3 cache stands for."""
    B, Hh, dh = dst.k.shape[1], dst.k.shape[2], dst.k.shape[4]
    K = np.zeros((B, Hh, cap, dh), np.float32)
    V = np.zeros((B, Hh, cap, dh), np.float32)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        ck, cv = _codes_in_order(dst, b, n)
        nt = (n + 63) // 64
        sk = np.repeat(dst.k_scale[0, b, :, :nt].cpu().numpy(), 64, axis=1)[:, :n]   # [Hh, n]
        sv = np.repeat(dst.v_scale[0, b, :, :nt].cpu().numpy(), 64, axis=1)[:, :n]
        K[b, :, :n] = O.e4m3_decode(ck.transpose(1, 0, 2)) * sk[:, :, None]
        V[b, :, :n] = O.e4m3_decode(cv.transpose(1, 0, 2)) * sv[:, :, None]
    return K, V


@pytest.mark.parametrize("shape", [
    ("C1-like", 1, 16, [9216], 32, 64, 1.0),
    ("ragged", 3, 4, [100, 3000, 777], 32, 64, 1.0),
    ("partial-own", 2, 4, [300, 129], 20, 64, 1.0),
    ("peaked scores", 2, 4, [3000, 700], 32, 64, 3.0),
    ("C6-like", 1, 24, [9216], 32, 128, 1.0),
    ("ragged dh=128", 3, 4, [100, 3000, 777], 32, 128, 1.0),
    ("partial-own dh=128", 2, 4, [300, 129], 20, 128, 1.0),
    ("peaked scores dh=128", 2, 4, [3000, 700], 32, 128, 3.0),
])
def test_attention_fp8_equals_bf16_on_dequantised_values(shape):
    """q_std 3 gives score std 3 (12 on the tile whose keys are 4x larger)."""
    name, B, Hh, lens, n_act, dh, q_std = shape
    print_case(f"E4M3 action attention {name}")
    rng = np.random.default_rng(17)
    cap = (max(lens) + 63) // 64 * 64
    K, V = _case(rng, B, Hh, lens, cap, dh)
    _, dst = _device_caches(K, V, lens, cap)
    Kd, Vd = _dequant_bf16_cache(dst, lens, cap)
    # the bf16 kernels take q as Q log2(e) / sqrt(dh), rounded once
    qs = np.log2(np.e) / np.sqrt(dh)
    q = torch.tensor(_bf16(rng.standard_normal((B, Hh, 32, dh)) * q_std * qs)).to(torch.bfloat16).cuda()
    ka = torch.tensor(_bf16(rng.standard_normal((B, Hh, 32, dh)))).to(torch.bfloat16).cuda()
    va = torch.tensor(_bf16(rng.standard_normal((B, Hh, dh, 32)))).to(torch.bfloat16).cuda()
    o8 = torch.empty((B, 32, Hh * dh), dtype=torch.bfloat16, device="cuda")
    o16 = torch.empty_like(o8)
    lens_a = np.asarray(lens, np.int32)
    wam.attention_action_fp8(q, ka, va, n_act, dst.k[0], dst.v[0], dst.k_scale[0], dst.v_scale[0],
                             cap, lens_a, o8)
    kd = torch.tensor(Kd).to(torch.bfloat16).cuda()
    vd = torch.tensor(np.ascontiguousarray(Vd.transpose(0, 1, 3, 2))).to(torch.bfloat16).cuda()
    wam.attention_action(wam.WAM_BF16, q, ka, va, n_act, kd, vd, cap, lens_a, o16)
    torch.cuda.synchronize()
    assert torch.equal(o8, o16)
    # and against the oracle's attention over the dequantised keys and values
    ref = []
    for b in range(B):
        kk = np.concatenate([Kd[b][:, :lens[b]], ka[b, :, :n_act].float().cpu().numpy()], axis=1)
        vv = np.concatenate([Vd[b][:, :lens[b]], va[b, :, :, :n_act].float().cpu().numpy().transpose(0, 2, 1)],
                            axis=1)
        qq = q[b].double().cpu().numpy() / qs
        ref.append(O.attention(torch.tensor(qq, dtype=torch.float64).permute(1, 0, 2),
                               torch.tensor(kk, dtype=torch.float64).permute(1, 0, 2),
                               torch.tensor(vv, dtype=torch.float64).permute(1, 0, 2)).numpy())
    got = to_np(o8).reshape(B, 32, Hh, dh)
    assert rel_l2(got, np.stack(ref)) <= 5e-3


SMALL = dict(L=2, D=256, Hh=4, Fm=512, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4),
             pad_frames=1, V=2, N=3, read_map=(0, 1), kv_fp8=True)


def _run_gpu(cfg, inp):
    from kv_cached_flow_amd.runner import DeviceChunk
    dc = DeviceChunk(cfg, inp)
    dc.run()
    torch.cuda.synchronize()
    return dc


@pytest.mark.parametrize("variant", ["dense", "sparse", "dh128"])
def test_chunk_with_fp8_cache_vs_oracle(variant):
    kw = dict(SMALL)
    if variant == "sparse":
        kw.update(L=4, V=0, read_map=(-1, 0, -1, 1), fuse=((0, 2), (2, 2)))
    if variant == "dh128":
        kw.update(Hh=2, dh=128)
    cfg = configs.small("Q", dtype="bf16", **kw)
    print_case(f"chunk with E4M3 cache, {variant}")
    inp = inputs.generate(cfg)
    ref = O.run_chunk(cfg, inp, kv_fp8=True)
    dc = _run_gpu(cfg, inp)
    assert rel_l2(to_np(dc.actions), ref["actions"]) <= 2e-2
    # the option moves the actions, by about the E4M3 step
    base = O.run_chunk(cfg, inp)
    d = rel_l2(ref["actions"], base["actions"])
    assert 0 < d < 0.1


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name", ["C1", "C6"])
def test_fp8_full_size_against_oracle_values(name):
    """Full size with the E4M3 cache: C1 (16 x 64 heads) and C6 (the real
    widths, 24 x 128 heads) against the oracle with the same quantisation."""
    path = os.path.join(GOLDEN, f"{name}_fp8.json")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_golden.py {name}+fp8)")
    g = json.load(open(path))
    cfg = configs.get(name, kv_fp8=True)
    print_case(f"full size {name} with the E4M3 cache")
    inp = inputs.generate(cfg)
    assert inputs.fingerprint(inp) == g["fingerprint"]
    dc = _run_gpu(cfg, inp)
    err = rel_l2(to_np(dc.actions), np.array(g["actions"]))
    print_case(f"{name} E4M3 final actions rel-L2 {err:.3e}")
    assert err <= 2e-2
