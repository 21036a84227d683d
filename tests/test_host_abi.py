"""Host-side tests of libwam (no GPU): exports, schedules, frame tables and
argument validation.  Every call here returns before any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

from kv_cached_flow_amd import wam
from oracle import wam_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wam.h")


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(wam_\w+)\s*\(", txt, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = wam.lib()
    names = header_functions()
    assert len(names) == 29
    for n in names:
        assert hasattr(L, n), n
    assert sorted(wam.exported_names()) == names
    assert wam.abi_version() == 4


def test_status_strings():
    L = wam.lib()
    for code in range(0, -7, -1):
        assert L.wam_status_str(code).decode()
    assert L.wam_status_str(-99).decode() == "unknown status"


@pytest.mark.parametrize("steps", [1, 2, 3, 4, 7, 10, 32])
@pytest.mark.parametrize("sigma_end", [0.0, 0.9, 0.5, 0.123])
@pytest.mark.parametrize("shift", [1.0, 3.0, 0.7])
def test_schedule_bit_exact_with_oracle(steps, sigma_end, shift):
    got = wam.schedule(steps, sigma_end, shift)
    ref = O.schedule(steps, sigma_end, shift)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _brute(frames, block, valid, P):
    fr = torch.tensor(frames).repeat_interleave(P)
    return O.video_visible(fr, fr, torch.tensor(block), torch.tensor(valid)).numpy()


@pytest.mark.parametrize("seed", range(12))
def test_frame_table_matches_oracle_mask(seed):
    r = np.random.default_rng(seed)
    Fh, Ff, P = int(r.integers(0, 6)), int(r.integers(0, 3)), int(r.integers(1, 5))
    if Fh + Ff == 0:
        Fh = 1
    F = Fh + Ff
    block = np.sort(r.integers(0, F + 1, F)).astype(np.int32)
    valid = (r.uniform(size=Fh) < 0.7).astype(np.uint8)
    src, kend = wam.frame_table(block, valid, Fh, Ff, P)
    keep = [f for f in range(Fh) if valid[f]] + list(range(Fh, F))
    assert list(src) == keep
    # visibility implied by the table (row i sees rows < kend[i // P]) == oracle on kept frames
    n = len(keep) * P
    vis = np.zeros((n, n), dtype=bool)
    for i in range(n):
        vis[i, : kend[i // P]] = True
    fvalid = np.concatenate([valid, np.ones(Ff, np.uint8)]).astype(np.int64)
    assert np.array_equal(vis, _brute(keep, block, fvalid, P))


def test_frame_table_rejects_non_monotone_blocks():
    with pytest.raises(wam.WamError, match="non-decreasing"):
        wam.frame_table([0, 2, 1], None, 3, 0, 4)


# ---------------------------------------------------------------- validation
FAKE = 0x100000  # aligned, never dereferenced: validation returns first


def good_dims(**kw):
    d = dict(L=2, D=256, Hh=4, dh=64, Fm=512, Cv=64, A=14, H=32, P=100, dtype=wam.WAM_BF16)
    d.update(kw)
    return wam.dims(**d)


class FakeExpert:
    def __init__(self, L, ptr=FAKE, cross=False, cond=None):
        n = 10 if cross else 6   # with the condition's cross-attention weights
        self.larr = (wam.WamLayerW * L)(*[wam.WamLayerW(*([ptr] * n)) for _ in range(L)])
        self.c = wam.WamExpertW(ptr, ptr, ptr, C.cast(self.larr, C.POINTER(wam.WamLayerW)), L,
                                C.pointer(cond) if cond is not None else None)


def fake_kv(n_layers=2, B=1, Hh=4, cap=512, dtype=wam.WAM_BF16, lens=None, dh=64):
    ln = np.asarray(lens if lens is not None else [cap] * B, dtype=np.int32)
    kv = wam.WamKV(FAKE, FAKE, n_layers, B, Hh, dh, cap, dtype, ln.ctypes.data_as(C.POINTER(C.c_int32)))
    return kv, ln


def call_prefill(d=None, expert=None, hist=FAKE, valid=None, B=1, Fh=3, fut=FAKE, Ff=2,
                 blocks=(0, 1, 2, 3, 4), V=2, sigma=0.9, shift=1.0, kv=None, ws=FAKE, ws_bytes=1 << 40):
    L = wam.lib()
    d = d or good_dims()
    ex = expert or FakeExpert(d.L)
    if kv is None:
        kv, _keep = fake_kv(cap=512)
    fb = np.asarray(blocks, dtype=np.int32)
    va = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    st = L.wam_prefill_video_cache(C.byref(d), C.byref(ex.c), hist, None if va is None else va.ctypes.data,
                                   B, Fh, fut, Ff, fb.ctypes.data, V, sigma, shift, C.byref(kv), None,
                                   ws, ws_bytes, None)
    return st, L.wam_last_error().decode()


def test_prefill_validation_errors():
    assert call_prefill(d=good_dims(dh=32))[0] == -2
    assert call_prefill(d=good_dims(D=512))[0] == -2          # D != Hh*dh
    assert call_prefill(d=good_dims(H=16))[0] == -2
    assert call_prefill(d=good_dims(dtype=7))[0] == -1
    assert call_prefill(d=good_dims(Cv=65))[0] == -2
    assert call_prefill(d=good_dims(Da=100))[0] == -2         # action width not a multiple of 64
    assert call_prefill(d=good_dims(Fma=-64))[0] == -2
    assert call_prefill(d=good_dims(Hh=80, D=5120))[0] == -2  # widths above 4096
    assert call_prefill(d=good_dims(Hh=2, dh=96, D=192))[0] == -2  # heads of 64 or 128 only
    assert call_prefill(d=good_dims(rope=2))[0] == -1              # rope is 0 or 1
    assert call_prefill(d=good_dims(rope=1), ws_bytes=4096)[0] == -5  # accepted up to the workspace
    kv128, _k = fake_kv(Hh=2, dh=128)
    assert call_prefill(d=good_dims(Hh=2, dh=128), kv=kv128, ws_bytes=4096)[0] == -5  # 128 accepted
    assert call_prefill(d=good_dims(Hh=2, dh=128), kv=fake_kv(Hh=2)[0])[0] == -2     # cache dh differs
    assert call_prefill(blocks=(0, 2, 1, 3, 4))[0] == -2      # non-monotone
    assert call_prefill(V=2, sigma=1.0)[0] == -1              # sigma* must be < 1
    assert call_prefill(V=-1)[0] == -1
    assert call_prefill(hist=FAKE + 4)[0] == -4               # misaligned
    assert call_prefill(ws=None)[0] == -5
    assert call_prefill(ws_bytes=1024)[0] == -5
    st, msg = call_prefill(expert=FakeExpert(1))
    assert st == -2 and "layers" in msg
    kv, _k = fake_kv(cap=500)
    assert call_prefill(kv=kv)[0] == -2                       # cap not a multiple of 64
    kv, _k = fake_kv(cap=256)
    st, msg = call_prefill(kv=kv)                             # needs 4 frames x 100 rows
    assert st == -2 and "cap" in msg
    kv, _k = fake_kv(cap=512)
    st, msg = call_prefill(Ff=0, blocks=(0, 1, 2), valid=np.zeros((1, 3)), kv=kv)
    assert st == -2 and "no valid frame" in msg


def test_prefill_limits():
    # the documented maxima pass validation, one past them is rejected
    kv, _k = fake_kv(cap=512)
    kv65, _k65 = fake_kv(B=wam.WAM_MAX_BATCH + 1, cap=512)
    st, msg = call_prefill(B=wam.WAM_MAX_BATCH + 1, kv=kv65)
    assert st == -2 and "B must be" in msg
    F = wam.WAM_MAX_FRAMES + 1
    st, msg = call_prefill(Fh=F - 2, Ff=2, blocks=tuple(range(F)), kv=kv)
    assert st == -2 and "frame counts" in msg
    st, msg = call_prefill(V=wam.WAM_MAX_STEPS + 1)
    assert st == -1 and "video_steps" in msg


def call_denoise(d=None, expert=None, kv=None, read_map=(0, 1), eps=FAKE, B=1, N=4, shift=1.0,
                 out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    L = wam.lib()
    d = d or good_dims()
    ex = expert or FakeExpert(d.L)
    rm = np.asarray(read_map, dtype=np.int32)
    kvp = C.byref(kv) if kv is not None else None
    return L.wam_denoise_chunk(C.byref(d), C.byref(ex.c), kvp, rm.ctypes.data, eps, B, N, shift, out,
                               None, ws, ws_bytes, None)


def test_denoise_validation_errors():
    kv, _k = fake_kv()
    assert call_denoise(kv=kv, N=0) == -1
    assert call_denoise(kv=kv, N=65) == -1
    assert call_denoise(kv=kv, B=0) == -2
    assert call_denoise(kv=kv, eps=FAKE + 8) == -4
    assert call_denoise(kv=None) == -1                        # reads a cache, none given
    assert call_denoise(kv=kv, read_map=(0, 5)) == -1          # layer 5 does not exist
    kv2, _k2 = fake_kv(dtype=wam.WAM_F32)
    assert call_denoise(kv=kv2) == -3                          # dtype mismatch
    kv3, _k3 = fake_kv(lens=[600], cap=512)
    assert call_denoise(kv=kv3) == -2                          # len > cap
    assert call_denoise(kv=kv, ws_bytes=4096) == -5
    assert call_denoise(kv=kv, shift=0.0) == -1


def call_codenoise(d=None, video=None, action=None, valid=None, B=1, Fh=3, fut=FAKE, Ff=2,
                   blocks=(0, 1, 2, 3, 4), eps=FAKE, N=4, end=0.0, shift=1.0, kv=None, out=FAKE,
                   z=FAKE, ws=FAKE, ws_bytes=1 << 40):
    L = wam.lib()
    d = d or good_dims()
    vx = video or FakeExpert(d.L)
    ax = action or FakeExpert(d.L)
    if kv is None:
        kv, _keep = fake_kv(cap=512, lens=[300])
    fb = np.asarray(blocks, dtype=np.int32)
    va = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    st = L.wam_codenoise_chunk(C.byref(d), C.byref(vx.c), C.byref(ax.c),
                               None if va is None else va.ctypes.data, B, Fh, fut, Ff, fb.ctypes.data,
                               eps, N, end, shift, C.byref(kv), out, z, None, ws, ws_bytes, None)
    return st, L.wam_last_error().decode()


def test_codenoise_validation_errors():
    st, msg = call_codenoise(Ff=0, blocks=(0, 1, 2))
    assert st == -2 and "Ff >= 1" in msg
    assert call_codenoise(N=0)[0] == -1
    assert call_codenoise(N=wam.WAM_MAX_STEPS + 1)[0] == -1
    assert call_codenoise(end=1.0)[0] == -1
    assert call_codenoise(end=-0.25)[0] == -1
    assert call_codenoise(shift=0.0)[0] == -1
    assert call_codenoise(z=None)[0] == -1                     # the video latents are required
    assert call_codenoise(eps=FAKE + 8)[0] == -4
    assert call_codenoise(blocks=(0, 2, 1, 3, 4))[0] == -2      # non-monotone
    assert call_codenoise(action=FakeExpert(1))[0] == -2        # layer count
    assert call_codenoise(ws_bytes=4096)[0] == -5
    kv, _k = fake_kv(cap=512, lens=[512])
    st, msg = call_codenoise(kv=kv)                              # not a history-only cache
    assert st == -2 and "valid history" in msg
    kv, _k = fake_kv(cap=256, lens=[300])
    st, msg = call_codenoise(kv=kv)                              # 5 frames x 100 rows > cap
    assert st == -2 and "cap" in msg
    kv, _k = fake_kv(n_layers=1, cap=512, lens=[300])
    assert call_codenoise(kv=kv)[0] == -2                       # cache must hold L layers
    # one padded history frame: the cache must then hold 2 frames of rows
    kv, _k = fake_kv(cap=512, lens=[300])
    st, msg = call_codenoise(kv=kv, valid=np.array([[0, 1, 1]]))
    assert st == -2 and "valid history" in msg


def test_codenoise_workspace_covers_both_experts():
    d = good_dims()
    kv, _k = fake_kv(cap=512, lens=[300])
    L = wam.lib()
    w = L.wam_codenoise_workspace_bytes(C.byref(d), 1, 2, C.byref(kv))
    assert w >= L.wam_prefill_workspace_bytes(C.byref(d), 1, 0, 2)
    assert w >= L.wam_denoise_workspace_bytes(C.byref(d), 1, C.byref(kv))
    assert L.wam_codenoise_workspace_bytes(C.byref(d), 1, 0, C.byref(kv)) == 0


def test_fp8_cache_validation_errors():
    L = wam.lib()
    src, _a = fake_kv(n_layers=2, cap=512, lens=[300])
    dst, _b = fake_kv(n_layers=2, cap=512, lens=[0], dtype=wam.WAM_FP8)
    dst.k_scale = dst.v_scale = FAKE

    def q(a, b):
        return L.wam_quantize_kv_fp8(C.byref(a), C.byref(b), None), L.wam_last_error().decode()

    src32, _c = fake_kv(n_layers=2, cap=512, lens=[300], dtype=wam.WAM_F32)
    assert q(src32, dst)[0] == -3                      # source must be bf16
    dstb, _d = fake_kv(n_layers=2, cap=512, lens=[0])
    dstb.k_scale = dstb.v_scale = FAKE
    assert q(src, dstb)[0] == -3                       # destination must be E4M3
    dst3, _e = fake_kv(n_layers=3, cap=512, lens=[0], dtype=wam.WAM_FP8)
    dst3.k_scale = dst3.v_scale = FAKE
    assert q(src, dst3)[0] == -2                       # layer counts differ
    dstn, _f = fake_kv(n_layers=2, cap=512, lens=[0], dtype=wam.WAM_FP8)
    assert q(src, dstn)[0] == -1                       # no tile scales
    big, _g = fake_kv(n_layers=2, cap=512, lens=[600])
    assert q(big, dst)[0] == -2                        # len > cap
    # an E4M3 cache is read by the action layers of a bf16 model only
    kv8, _h = fake_kv(dtype=wam.WAM_FP8)
    kv8.k_scale = kv8.v_scale = FAKE
    assert call_denoise(kv=kv8, ws_bytes=4096) == -5   # accepted up to the workspace check
    assert call_denoise(d=good_dims(dtype=wam.WAM_F32), kv=kv8) == -3
    kv8n, _i = fake_kv(dtype=wam.WAM_FP8)
    assert call_denoise(kv=kv8n) == -1                 # no scales
    assert call_prefill(kv=kv8)[0] == -3               # the prefill writes bf16 only
    kv8c, _j = fake_kv(cap=512, lens=[300], dtype=wam.WAM_FP8)
    kv8c.k_scale = kv8c.v_scale = FAKE
    assert call_codenoise(kv=kv8c)[0] == -3
    # E4M3 caches of 64- and 128-wide heads (nothing is launched: every call
    # below stops at a check)
    s96, _l = fake_kv(n_layers=2, cap=512, lens=[300], dh=96)
    d96, _m = fake_kv(n_layers=2, cap=512, lens=[0], dtype=wam.WAM_FP8, dh=96)
    d96.k_scale = d96.v_scale = FAKE
    assert q(s96, d96)[0] == -2                        # heads of 64 or 128 only
    k128, _n = fake_kv(Hh=2, dtype=wam.WAM_FP8, dh=128)
    k128.k_scale = k128.v_scale = FAKE
    assert call_denoise(d=good_dims(Hh=2, dh=128), kv=k128, ws_bytes=4096) == -5   # accepted
    ln = np.array([100], np.int32)
    st = L.wam_attention_action_fp8(1, 4, 96, 32, FAKE, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, 128,
                                    ln.ctypes.data, FAKE, 0, FAKE, 1 << 30, None)
    assert st == -2


def test_async_schedule_rule_by_brute_force():
    # R/2 <= S < R <= H with S > 0 (Long-WAM Summary section 4.1), over every small triple
    for H in range(0, 12):
        for R in range(-1, 13):
            for S in range(-1, 13):
                want = 0 < S < R <= H and 2 * S >= R
                assert wam.async_check(H, R, S) == want, (H, R, S)
    # the deployed settings: R = 24 with strides 12, 16, 20; the default stride (R+1)//2
    for S in (12, 16, 20, (24 + 1) // 2):
        assert wam.async_check(32, 24, S)


def test_async_handoff():
    assert wam.async_handoff(32, 24, 16, 0) == (0, 24)
    assert wam.async_handoff(32, 24, 16, 5) == (5, 19)
    assert wam.async_handoff(32, 24, 16, 8) == (8, 16)       # exactly at the deadline O = 8
    with pytest.raises(wam.WamError, match="overlap"):
        wam.async_handoff(32, 24, 16, 9)                       # missed: the robot waited
    with pytest.raises(wam.WamError):
        wam.async_handoff(32, 24, 16, -1)
    with pytest.raises(wam.WamError):
        wam.async_handoff(32, 24, 11, 0)                       # S < R/2


def call_extend(d=None, hist=FAKE, valid=None, B=1, Fh_old=3, Fn=2, blocks=(0, 1, 2, 3, 4), kv=None,
                ws=FAKE, ws_bytes=1 << 40):
    L = wam.lib()
    d = d or good_dims()
    ex = FakeExpert(d.L)
    if kv is None:
        kv, _keep = fake_kv(cap=512, lens=[300])
    fb = np.asarray(blocks, dtype=np.int32)
    va = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    st = L.wam_extend_history_cache(C.byref(d), C.byref(ex.c), hist, None if va is None else va.ctypes.data,
                                    B, Fh_old, Fn, fb.ctypes.data, C.byref(kv), ws, ws_bytes, None)
    return st, L.wam_last_error().decode()


def call_future(d=None, valid=None, B=1, Fh=3, fut=FAKE, Ff=2, blocks=(0, 1, 2, 3, 4), V=2, kv=None,
                ws=FAKE, ws_bytes=1 << 40):
    L = wam.lib()
    d = d or good_dims()
    ex = FakeExpert(d.L)
    if kv is None:
        kv, _keep = fake_kv(cap=512, lens=[300])
    fb = np.asarray(blocks, dtype=np.int32)
    va = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    st = L.wam_prefill_future(C.byref(d), C.byref(ex.c), None if va is None else va.ctypes.data, B, Fh,
                              fut, Ff, fb.ctypes.data, V, 0.9, 1.0, C.byref(kv), None, ws, ws_bytes, None)
    return st, L.wam_last_error().decode()


def test_streaming_validation_errors():
    assert call_extend(Fn=0)[0] == -2
    assert call_extend(hist=None)[0] == -1
    assert call_extend(hist=FAKE + 2)[0] == -4
    assert call_extend(ws_bytes=1024)[0] == -5
    kv, _k = fake_kv(cap=512, lens=[200])
    st, msg = call_extend(kv=kv)                               # len must be the old frames' rows
    assert st == -2 and "cache holds" in msg
    st, msg = call_extend(blocks=(0, 1, 1, 1, 2))              # new frame 3 shares block 1 with frame 2
    assert st == -2 and "shares temporal block" in msg
    kv, _k = fake_kv(cap=256, lens=[300])
    st, msg = call_extend(kv=kv)
    assert st == -2
    # one padded old frame: the cache must hold 2 frames of rows
    kv, _k = fake_kv(cap=512, lens=[200])
    st, msg = call_extend(kv=kv, valid=np.array([[0, 1, 1, 1, 1]]), ws_bytes=16)
    assert st == -5                                            # validation passed up to the workspace
    assert call_future(Ff=0, blocks=(0, 1, 2))[0] == -2
    assert call_future(fut=None)[0] == -1
    assert call_future(V=-1)[0] == -1
    kv, _k = fake_kv(cap=512, lens=[500])
    st, msg = call_future(kv=kv)
    assert st == -2 and "valid history" in msg
    assert call_future(ws_bytes=1024)[0] == -5


def test_fuse_validation_errors():
    L = wam.lib()
    src, _a = fake_kv(n_layers=8)
    dst, _b = fake_kv(n_layers=2)

    def fuse(start, count, logits, M=None):
        s = np.asarray(start, np.int32)
        c = np.asarray(count, np.int32)
        lg = np.ascontiguousarray(logits, np.float32)
        return L.wam_fuse_interval_kv(C.byref(src), M or len(s), s.ctypes.data, c.ctypes.data,
                                      lg.ctypes.data, lg.shape[1], C.byref(dst), None)

    assert fuse([0, 4], [4, 4], np.full((2, 4), -np.inf)) == -1       # all -inf
    assert fuse([0, 6], [4, 4], np.zeros((2, 4))) == -2               # past the last layer
    assert fuse([0], [9], np.zeros((1, 9))) == -2                     # interval too long
    assert fuse([0, 4, 0], [4, 4, 1], np.zeros((3, 4))) == -2         # dst too small


def test_attention_entry_validation():
    L = wam.lib()
    ln = np.array([100], np.int32)
    st = L.wam_attention_action(wam.WAM_BF16, 1, 4, 64, 16, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 128,
                                ln.ctypes.data, FAKE, 0, FAKE, 1 << 30, None)
    assert st == -2                                            # H must be 32
    st = L.wam_attention_action(wam.WAM_BF16, 1, 4, 64, 32, FAKE, None, None, 0, None, None, 0,
                                None, FAKE, 0, FAKE, 1 << 30, None)
    assert st == -2                                            # no key at all
    ke = np.array([100, 200], np.int32)
    st = L.wam_attention_prefill(wam.WAM_BF16, 4, 64, 300, 0, 100, ke.ctypes.data, 2, FAKE, FAKE,
                                 FAKE, 256, FAKE, None)
    assert st == -2                                            # rows beyond the table
    ke = np.array([200, 100], np.int32)
    st = L.wam_attention_prefill(wam.WAM_BF16, 4, 64, 150, 0, 100, ke.ctypes.data, 2, FAKE, FAKE,
                                 FAKE, 256, FAKE, None)
    assert st == -2                                            # kend not monotone


def test_workspace_sizes_grow_with_shapes():
    d = good_dims()
    small = wam.prefill_workspace_bytes(d, 1, 3, 2)
    big = wam.prefill_workspace_bytes(good_dims(P=1000), 1, 3, 2)
    assert 0 < small < big
    kv, _k = fake_kv(cap=512)
    kvb, _kb = fake_kv(cap=8192, lens=[8192])
    a = wam.lib().wam_denoise_workspace_bytes(C.byref(d), 1, C.byref(kv))
    b = wam.lib().wam_denoise_workspace_bytes(C.byref(d), 1, C.byref(kvb))
    assert 0 < a <= b


def test_euler_rejects_negative_count():
    assert wam.lib().wam_flow_euler_step(FAKE, FAKE, -1, 1.0, 0.5, None) == -1
    assert wam.lib().wam_flow_euler_step(FAKE, FAKE, 0, 1.0, 0.5, None) == 0


def test_python_limits_match_header():
    hdr = open(os.path.join(os.path.dirname(wam.__file__), os.pardir, "include", "wam.h")).read()
    for name in ("WAM_MAX_FRAMES", "WAM_MAX_BATCH", "WAM_MAX_FUSE", "WAM_MAX_INTERVAL", "WAM_MAX_STEPS"):
        m = re.search(r"#define %s (\d+)" % name, hdr)
        assert m and int(m.group(1)) == getattr(wam, name)


# ---------------------------------------------------------------- text/state condition
def test_condition_validation_errors():
    L = wam.lib()
    d = good_dims(Tc=37, Ct=128, S=14)
    # the condition needs the cross-attention weights and the expert's cache
    st, msg = call_prefill(d=d, expert=FakeExpert(d.L))
    assert st == -1 and "cross-attention" in msg
    st, msg = call_prefill(d=d, expert=FakeExpert(d.L, cross=True))
    assert st == -1 and "condition cache" in msg
    bad, _k2 = fake_kv(cap=64, lens=[36])                   # len must be Tc
    st, msg = call_prefill(d=d, expert=FakeExpert(d.L, cross=True, cond=bad))
    assert st == -2 and "len" in msg
    small, _k3 = fake_kv(cap=0, lens=[37])                  # cap below Tc
    st, msg = call_prefill(d=d, expert=FakeExpert(d.L, cross=True, cond=small))
    assert st == -2
    # dims
    assert L.wam_prefill_condition_kv(C.byref(good_dims(Tc=5, Ct=100)), None, None, FAKE, FAKE,
                                      FAKE, 1, None, None, FAKE, 1 << 30, None) == -2  # Ct % 64
    assert L.wam_prefill_condition_kv(C.byref(good_dims()), None, None, FAKE, FAKE, FAKE, 1, None,
                                      None, FAKE, 1 << 30, None) == -2                  # Tc == 0
    ex = FakeExpert(d.L, cross=True)
    assert L.wam_prefill_condition_kv(C.byref(d), None, None, FAKE, FAKE, FAKE, 1, None, None, FAKE,
                                      1 << 30, None) == -1                              # no expert
    assert L.wam_prefill_condition_kv(C.byref(d), C.byref(ex.c), None, FAKE, FAKE, FAKE, 1, None,
                                      None, FAKE, 1 << 30, None) == -1                  # no cache
    cc, _k4 = fake_kv(cap=64, lens=[0])
    assert L.wam_prefill_condition_kv(C.byref(d), C.byref(ex.c), None, FAKE, FAKE, FAKE, 1,
                                      C.byref(cc), None, FAKE, 16, None) == -5          # workspace
    assert L.wam_condition_workspace_bytes(C.byref(d), 2) >= 2 * 37 * 128 * 2
    assert L.wam_condition_workspace_bytes(C.byref(good_dims()), 1) == 0


def test_noalloc_denoise_rejects_chunks_beyond_its_scratch():
    # 64 episodes of 16 heads x 128 need far more than the 64 MiB static
    # scratch: refused on the host, before anything is enqueued
    L = wam.lib()
    d = good_dims(D=2048, Hh=16, dh=128)
    ex = FakeExpert(d.L)
    kv, _k = fake_kv(B=64, Hh=16, dh=128, cap=4096, lens=[4096] * 64)
    rm = np.asarray([0, 1], dtype=np.int32)
    need = L.wam_denoise_workspace_bytes(C.byref(d), 64, C.byref(kv))
    assert need > wam.WAM_NOALLOC_SCRATCH_BYTES
    st = L.wam_denoise_chunk_noalloc(C.byref(d), C.byref(ex.c), C.byref(kv), rm.ctypes.data, FAKE, 64,
                                     4, 1.0, FAKE, None, None)
    assert st == -5 and "scratch" in L.wam_last_error().decode()
