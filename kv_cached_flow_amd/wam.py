"""Python binding of libwam (ctypes).  Argument marshalling only: every step
of the hot path runs in the library's HIP kernels.  Tensors are PyTorch
device tensors (memory and streams only).  The names follow the C calls in
``include/wam.h``.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwam.so")

WAM_F32, WAM_BF16, WAM_FP8 = 0, 1, 2
WAM_MAX_FRAMES = 256   # limits of the C-ABI (include/wam.h)
WAM_MAX_BATCH = 64
WAM_MAX_FUSE = 32
WAM_MAX_INTERVAL = 8
WAM_MAX_STEPS = 64

_lib = None


class WamError(RuntimeError):
    pass


class WamDims(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("L", "D", "Hh", "dh", "Fm", "Cv", "A", "H", "P", "dtype", "Da",
                                        "Fma", "rope", "Tc", "Ct", "S")]


LAYER_FIELDS = ("g1", "wqkv", "wo", "g2", "w1", "w2", "gx", "wqx", "wkvx", "wox")


class WamLayerW(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_FIELDS]


class WamKV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n_layers", C.c_int), ("B", C.c_int),
                ("Hh", C.c_int), ("dh", C.c_int), ("cap", C.c_int), ("dtype", C.c_int),
                ("len", C.POINTER(C.c_int32)), ("k_scale", C.c_void_p), ("v_scale", C.c_void_p)]


class WamExpertW(C.Structure):
    _fields_ = [("w_in", C.c_void_p), ("g_out", C.c_void_p), ("w_out", C.c_void_p),
                ("layers", C.POINTER(WamLayerW)), ("n_layers", C.c_int),
                ("cond", C.POINTER(WamKV))]


class WamKernelStat(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int), ("ms", C.c_double),
                ("bytes", C.c_double), ("flops", C.c_double)]


_EXPORTS = {
    "wam_abi_version": (C.c_int, []),
    "wam_status_str": (C.c_char_p, [C.c_int]),
    "wam_last_error": (C.c_char_p, []),
    "wam_schedule": (C.c_int, [C.c_int, C.c_double, C.c_double, C.c_void_p]),
    "wam_frame_table": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "wam_prefill_workspace_bytes": (C.c_size_t, [C.POINTER(WamDims), C.c_int, C.c_int, C.c_int]),
    "wam_prefill_video_cache": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW), C.c_void_p, C.c_void_p,
                                          C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_int,
                                          C.c_double, C.c_double, C.POINTER(WamKV), C.c_void_p,
                                          C.c_void_p, C.c_size_t, C.c_void_p]),
    "wam_extend_history_cache": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW), C.c_void_p,
                                           C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                           C.POINTER(WamKV), C.c_void_p, C.c_size_t, C.c_void_p]),
    "wam_prefill_future": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW), C.c_void_p, C.c_int,
                                     C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_double,
                                     C.c_double, C.POINTER(WamKV), C.c_void_p, C.c_void_p,
                                     C.c_size_t, C.c_void_p]),
    "wam_async_check": (C.c_int, [C.c_int, C.c_int, C.c_int]),
    "wam_async_handoff": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_int),
                                    C.POINTER(C.c_int)]),
    "wam_fuse_interval_kv": (C.c_int, [C.POINTER(WamKV), C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_int, C.POINTER(WamKV), C.c_void_p]),
    "wam_action_workspace_bytes": (C.c_size_t, [C.POINTER(WamDims), C.c_int, C.POINTER(WamKV)]),
    "wam_action_layer": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamLayerW), C.c_void_p,
                                   C.POINTER(WamKV), C.c_int, C.POINTER(WamKV), C.c_int, C.c_int,
                                   C.c_void_p, C.c_size_t, C.c_void_p]),
    "wam_condition_workspace_bytes": (C.c_size_t, [C.POINTER(WamDims), C.c_int]),
    "wam_prefill_condition_kv": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW),
                                           C.POINTER(WamExpertW), C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_int, C.POINTER(WamKV), C.POINTER(WamKV), C.c_void_p,
                                           C.c_size_t, C.c_void_p]),
    "wam_flow_euler_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_float, C.c_float,
                                      C.c_void_p]),
    "wam_denoise_workspace_bytes": (C.c_size_t, [C.POINTER(WamDims), C.c_int, C.POINTER(WamKV)]),
    "wam_denoise_chunk": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW), C.POINTER(WamKV),
                                    C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_double, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "wam_denoise_chunk_noalloc": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW), C.POINTER(WamKV),
                                            C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_double,
                                            C.c_void_p, C.c_void_p, C.c_void_p]),
    "wam_codenoise_workspace_bytes": (C.c_size_t, [C.POINTER(WamDims), C.c_int, C.c_int, C.POINTER(WamKV)]),
    "wam_codenoise_chunk": (C.c_int, [C.POINTER(WamDims), C.POINTER(WamExpertW), C.POINTER(WamExpertW),
                                      C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                      C.c_void_p, C.c_int, C.c_double, C.c_double, C.POINTER(WamKV),
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                      C.c_void_p]),
    "wam_debug_visibility": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                       C.c_void_p]),
    "wam_attention_action": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                                       C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p,
                                       C.c_size_t, C.c_void_p]),
    "wam_attention_action_fp8": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_int,
                                           C.c_void_p, C.c_size_t, C.c_void_p]),
    "wam_quantize_kv_fp8": (C.c_int, [C.POINTER(WamKV), C.POINTER(WamKV), C.c_void_p]),
    "wam_attention_prefill": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                        C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_int, C.c_void_p, C.c_void_p]),
    "wam_timing": (C.c_int, [C.c_int]),
    "wam_timing_report": (C.c_int, [C.POINTER(WamKernelStat), C.c_int]),
}


def lib():
    """Load libwam.so (fails loudly when it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise WamError(f"{LIB_PATH} is missing: build it with `python -m kv_cached_flow_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_names() -> List[str]:
    return list(_EXPORTS)


def _check(st: int, what: str):
    if st < 0:
        L = lib()
        raise WamError(f"{what}: {L.wam_status_str(st).decode()} ({st}): {L.wam_last_error().decode()}")
    return st


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ------------------------------------------------------------------ host-side calls
def abi_version() -> int:
    return lib().wam_abi_version()


def schedule(steps: int, sigma_end: float, shift: float = 1.0) -> np.ndarray:
    out = np.zeros(steps + 1, dtype=np.float32)
    _check(lib().wam_schedule(steps, sigma_end, shift, out.ctypes.data), "wam_schedule")
    return out


def frame_table(frame_block: Sequence[int], valid: Optional[Sequence[int]], Fh: int, Ff: int, P: int):
    fb = np.ascontiguousarray(frame_block, dtype=np.int32)
    va = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    src = np.zeros(WAM_MAX_FRAMES, dtype=np.int32)
    kend = np.zeros(WAM_MAX_FRAMES, dtype=np.int32)
    n = _check(lib().wam_frame_table(fb.ctypes.data, None if va is None else va.ctypes.data,
                                     Fh, Ff, P, src.ctypes.data, kend.ctypes.data), "wam_frame_table")
    return src[:n].copy(), kend[:n].copy()


# ------------------------------------------------------------------ device structs
def dims(L, D, Hh, dh, Fm, Cv, A, H, P, dtype, Da=0, Fma=0, rope=0, Tc=0, Ct=0, S=0) -> WamDims:
    """Shapes of a call; Da / Fma: the action expert's width and MLP width (0: D / Fm);
    rope: 1 for the rotary position option; Tc / Ct / S: the text/state condition
    (tokens, width, robot-state dims; Tc = 0: none)."""
    return WamDims(L, D, Hh, dh, Fm, Cv, A, H, P, dtype, Da, Fma, rope, Tc, Ct, S)


class DeviceExpert:
    """An expert's weights as device tensors plus the C struct pointing at them.
    ``set_cond`` points the struct at the expert's condition cache of a call."""

    def __init__(self, w_in, g_out, w_out, layers: List[dict]):
        self.w_in, self.g_out, self.w_out, self.layers = w_in, g_out, w_out, layers
        n = len(layers)
        self._larr = (WamLayerW * n)()
        for i, lw in enumerate(layers):
            self._larr[i] = WamLayerW(*[lw[k].data_ptr() if k in lw else None for k in LAYER_FIELDS])
        self.c = WamExpertW(w_in.data_ptr(), g_out.data_ptr(), w_out.data_ptr(),
                            C.cast(self._larr, C.POINTER(WamLayerW)), n, None)
        self.cond = None

    def set_cond(self, kv: Optional["DeviceKV"]):
        self.cond = kv
        self.c.cond = C.pointer(kv.c) if kv is not None else None

    def layer_struct(self, l: int) -> WamLayerW:
        return self._larr[l]


class DeviceKV:
    """Per-layer K/V cache of B episodes: k [n][B][Hh][cap][dh], v [n][B][Hh][dh][cap];
    WAM_FP8: uint8 codes in the lane order of the header, plus tile scales
    k_scale / v_scale [n][B][Hh][cap/64] fp32."""

    def __init__(self, n_layers: int, B: int, Hh: int, dh: int, cap: int, dtype: int, device="cuda"):
        import torch
        if cap % 64:
            raise WamError("cap must be a multiple of 64")
        tdt = {WAM_BF16: torch.bfloat16, WAM_F32: torch.float32, WAM_FP8: torch.uint8}[dtype]
        self.k = torch.empty((n_layers, B, Hh, cap, dh), dtype=tdt, device=device)
        self.v = torch.empty((n_layers, B, Hh, dh, cap), dtype=tdt, device=device)
        self.k_scale = self.v_scale = None
        if dtype == WAM_FP8:
            self.k_scale = torch.empty((n_layers, B, Hh, cap // 64), dtype=torch.float32, device=device)
            self.v_scale = torch.empty((n_layers, B, Hh, cap // 64), dtype=torch.float32, device=device)
        self.len = np.zeros(B, dtype=np.int32)
        self.c = WamKV(self.k.data_ptr(), self.v.data_ptr(), n_layers, B, Hh, dh, cap, dtype,
                       self.len.ctypes.data_as(C.POINTER(C.c_int32)), _ptr(self.k_scale),
                       _ptr(self.v_scale))

    @property
    def cap(self):
        return self.c.cap


def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ the C calls
def prefill_workspace_bytes(d: WamDims, B: int, Fh: int, Ff: int) -> int:
    return lib().wam_prefill_workspace_bytes(C.byref(d), B, Fh, Ff)


def prefill_video_cache(d: WamDims, video: DeviceExpert, hist, hist_valid, B: int, Fh: int,
                        fut_noise, Ff: int, frame_block, video_steps: int, sigma_star: float,
                        shift: float, cache: DeviceKV, fut_latents_out=None, ws=None, stream=None):
    hv = None if hist_valid is None else np.ascontiguousarray(hist_valid, dtype=np.uint8)
    fb = np.ascontiguousarray(frame_block, dtype=np.int32)
    if ws is None:
        ws = workspace(prefill_workspace_bytes(d, B, Fh, Ff))
    _check(lib().wam_prefill_video_cache(
        C.byref(d), C.byref(video.c), _ptr(hist), None if hv is None else hv.ctypes.data, B, Fh,
        _ptr(fut_noise), Ff, fb.ctypes.data, video_steps, sigma_star, shift, C.byref(cache.c),
        _ptr(fut_latents_out), _ptr(ws), ws.numel(), _stream(stream)), "wam_prefill_video_cache")


def extend_history_cache(d: WamDims, video: DeviceExpert, hist_new, hist_valid, B: int, Fh_old: int,
                         Fn: int, frame_block, cache: DeviceKV, ws=None, stream=None):
    hv = None if hist_valid is None else np.ascontiguousarray(hist_valid, dtype=np.uint8)
    fb = np.ascontiguousarray(frame_block, dtype=np.int32)
    if ws is None:
        ws = workspace(prefill_workspace_bytes(d, B, Fn, 0))
    _check(lib().wam_extend_history_cache(
        C.byref(d), C.byref(video.c), _ptr(hist_new), None if hv is None else hv.ctypes.data, B,
        Fh_old, Fn, fb.ctypes.data, C.byref(cache.c), _ptr(ws), ws.numel(), _stream(stream)),
        "wam_extend_history_cache")


def prefill_future(d: WamDims, video: DeviceExpert, hist_valid, B: int, Fh: int, fut_noise, Ff: int,
                   frame_block, video_steps: int, sigma_star: float, shift: float, cache: DeviceKV,
                   fut_latents_out=None, ws=None, stream=None):
    hv = None if hist_valid is None else np.ascontiguousarray(hist_valid, dtype=np.uint8)
    fb = np.ascontiguousarray(frame_block, dtype=np.int32)
    if ws is None:
        ws = workspace(prefill_workspace_bytes(d, B, 0, Ff))
    _check(lib().wam_prefill_future(
        C.byref(d), C.byref(video.c), None if hv is None else hv.ctypes.data, B, Fh, _ptr(fut_noise),
        Ff, fb.ctypes.data, video_steps, sigma_star, shift, C.byref(cache.c),
        _ptr(fut_latents_out), _ptr(ws), ws.numel(), _stream(stream)), "wam_prefill_future")


def async_check(H: int, R: int, S: int) -> bool:
    """True iff (H, R, S) satisfies R/2 <= S < R <= H."""
    return lib().wam_async_check(H, R, S) == 0


def async_handoff(H: int, R: int, S: int, elapsed: int):
    """(first, count): the aligned suffix of a chunk ready `elapsed` steps after its trigger."""
    f, c = C.c_int(), C.c_int()
    _check(lib().wam_async_handoff(H, R, S, elapsed, C.byref(f), C.byref(c)), "wam_async_handoff")
    return f.value, c.value


def fuse_interval_kv(src: DeviceKV, start, count, logits, dst: DeviceKV, stream=None):
    st = np.ascontiguousarray(start, dtype=np.int32)
    cn = np.ascontiguousarray(count, dtype=np.int32)
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    _check(lib().wam_fuse_interval_kv(C.byref(src.c), len(st), st.ctypes.data, cn.ctypes.data,
                                      lg.ctypes.data, lg.shape[1], C.byref(dst.c), _stream(stream)),
           "wam_fuse_interval_kv")


def action_workspace_bytes(d: WamDims, B: int, kv: Optional[DeviceKV]) -> int:
    return lib().wam_action_workspace_bytes(C.byref(d), B, C.byref(kv.c) if kv is not None else None)


def action_layer(d: WamDims, expert: DeviceExpert, l: int, x, kv: Optional[DeviceKV], kv_layer: int,
                 B: int, ws=None, stream=None, cond: Optional[DeviceKV] = None, cond_layer: int = 0):
    if ws is None:
        ws = workspace(action_workspace_bytes(d, B, kv))
    lw = expert.layer_struct(l)
    _check(lib().wam_action_layer(C.byref(d), C.byref(lw), _ptr(x),
                                  C.byref(kv.c) if kv is not None else None, kv_layer,
                                  C.byref(cond.c) if cond is not None else None, cond_layer, B,
                                  _ptr(ws), ws.numel(), _stream(stream)), "wam_action_layer")


def condition_workspace_bytes(d: WamDims, B: int) -> int:
    return lib().wam_condition_workspace_bytes(C.byref(d), B)


def prefill_condition_kv(d: WamDims, video: Optional[DeviceExpert], action: Optional[DeviceExpert],
                         proprio_w, text, state, B: int, cond_video: Optional[DeviceKV],
                         cond_action: Optional[DeviceKV], ws=None, stream=None):
    if ws is None:
        ws = workspace(condition_workspace_bytes(d, B))
    _check(lib().wam_prefill_condition_kv(
        C.byref(d), C.byref(video.c) if video is not None else None,
        C.byref(action.c) if action is not None else None, _ptr(proprio_w), _ptr(text), _ptr(state), B,
        C.byref(cond_video.c) if cond_video is not None else None,
        C.byref(cond_action.c) if cond_action is not None else None, _ptr(ws), ws.numel(),
        _stream(stream)), "wam_prefill_condition_kv")


def flow_euler_step(x, v, sigma: float, sigma_next: float, stream=None):
    _check(lib().wam_flow_euler_step(_ptr(x), _ptr(v), x.numel(), sigma, sigma_next, _stream(stream)),
           "wam_flow_euler_step")


def denoise_workspace_bytes(d: WamDims, B: int, kv: Optional[DeviceKV]) -> int:
    return lib().wam_denoise_workspace_bytes(C.byref(d), B, C.byref(kv.c) if kv is not None else None)


def denoise_chunk(d: WamDims, action: DeviceExpert, kv: Optional[DeviceKV], read_map, eps, B: int,
                  N: int, shift: float, actions_out, vhat_out=None, ws=None, stream=None):
    rm = np.ascontiguousarray(read_map, dtype=np.int32)
    if ws is None:
        ws = workspace(denoise_workspace_bytes(d, B, kv))
    _check(lib().wam_denoise_chunk(C.byref(d), C.byref(action.c), C.byref(kv.c) if kv is not None else None,
                                   rm.ctypes.data, _ptr(eps), B, N, shift, _ptr(actions_out),
                                   _ptr(vhat_out), _ptr(ws), ws.numel(), _stream(stream)),
           "wam_denoise_chunk")


WAM_NOALLOC_SCRATCH_BYTES = 64 << 20


def denoise_chunk_noalloc(d: WamDims, action: DeviceExpert, kv: Optional[DeviceKV], read_map, eps,
                          B: int, N: int, shift: float, actions_out, vhat_out=None, stream=None):
    """wam_denoise_chunk on the library's static scratch (no workspace, no allocation)."""
    rm = np.ascontiguousarray(read_map, dtype=np.int32)
    _check(lib().wam_denoise_chunk_noalloc(C.byref(d), C.byref(action.c),
                                           C.byref(kv.c) if kv is not None else None, rm.ctypes.data,
                                           _ptr(eps), B, N, shift, _ptr(actions_out), _ptr(vhat_out),
                                           _stream(stream)), "wam_denoise_chunk_noalloc")


def codenoise_workspace_bytes(d: WamDims, B: int, Ff: int, cache: DeviceKV) -> int:
    return lib().wam_codenoise_workspace_bytes(C.byref(d), B, Ff, C.byref(cache.c))


def codenoise_chunk(d: WamDims, video: DeviceExpert, action: DeviceExpert, hist_valid, B: int,
                    Fh: int, fut_noise, Ff: int, frame_block, eps, N: int, sigma_video_end: float,
                    shift: float, cache: DeviceKV, actions_out, fut_latents_out, vhat_out=None,
                    ws=None, stream=None):
    hv = None if hist_valid is None else np.ascontiguousarray(hist_valid, dtype=np.uint8)
    fb = np.ascontiguousarray(frame_block, dtype=np.int32)
    if ws is None:
        ws = workspace(codenoise_workspace_bytes(d, B, Ff, cache))
    _check(lib().wam_codenoise_chunk(
        C.byref(d), C.byref(video.c), C.byref(action.c), None if hv is None else hv.ctypes.data, B,
        Fh, _ptr(fut_noise), Ff, fb.ctypes.data, _ptr(eps), N, sigma_video_end, shift,
        C.byref(cache.c), _ptr(actions_out), _ptr(fut_latents_out), _ptr(vhat_out), _ptr(ws),
        ws.numel(), _stream(stream)), "wam_codenoise_chunk")


def debug_visibility(frame_block, valid, Fh: int, Ff: int, P: int, stream=None):
    import torch
    fb = np.ascontiguousarray(frame_block, dtype=np.int32)
    va = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    n = (Fh + Ff) * P
    vis = torch.empty((n, n), dtype=torch.uint8, device="cuda")
    _check(lib().wam_debug_visibility(fb.ctypes.data, None if va is None else va.ctypes.data, Fh, Ff,
                                      P, _ptr(vis), _stream(stream)), "wam_debug_visibility")
    return vis


def attention_action(dtype: int, q, ka, va, n_act: int, kc, vc, cap: int, lens, out,
                     splits_hint: int = 0, ws=None, stream=None):
    B, Hh, H, dh = q.shape
    ln = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    if ws is None:
        ws = workspace(64 << 20)
    _check(lib().wam_attention_action(dtype, B, Hh, dh, H, _ptr(q), _ptr(ka), _ptr(va), n_act,
                                      _ptr(kc), _ptr(vc), cap, None if ln is None else ln.ctypes.data,
                                      _ptr(out), splits_hint, _ptr(ws), ws.numel(), _stream(stream)),
           "wam_attention_action")


def attention_action_fp8(q, ka, va, n_act: int, kc8, vc8, k_scale, v_scale, cap: int, lens, out,
                         splits_hint: int = 0, ws=None, stream=None):
    B, Hh, H, dh = q.shape
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    if ws is None:
        ws = workspace(64 << 20)
    _check(lib().wam_attention_action_fp8(B, Hh, dh, H, _ptr(q), _ptr(ka), _ptr(va), n_act, _ptr(kc8),
                                          _ptr(vc8), _ptr(k_scale), _ptr(v_scale), cap,
                                          ln.ctypes.data, _ptr(out), splits_hint, _ptr(ws),
                                          ws.numel(), _stream(stream)), "wam_attention_action_fp8")


def quantize_kv_fp8(src: "DeviceKV", dst: "DeviceKV", stream=None):
    _check(lib().wam_quantize_kv_fp8(C.byref(src.c), C.byref(dst.c), _stream(stream)),
           "wam_quantize_kv_fp8")


def attention_prefill(dtype: int, q, row0: int, P: int, kend, kc, vc, cap: int, out, stream=None):
    Hh, nq, dh = q.shape
    ke = np.ascontiguousarray(kend, dtype=np.int32)
    _check(lib().wam_attention_prefill(dtype, Hh, dh, nq, row0, P, ke.ctypes.data, len(ke), _ptr(q),
                                       _ptr(kc), _ptr(vc), cap, _ptr(out), _stream(stream)),
           "wam_attention_prefill")


def timing(enable: bool):
    """Turn per-kernel-class event timing on (clearing old records) or off."""
    _check(lib().wam_timing(1 if enable else 0), "wam_timing")


def timing_report() -> dict:
    """{class: {launches, ms, bytes, flops}} of the launches recorded so far."""
    arr = (WamKernelStat * 32)()
    n = _check(lib().wam_timing_report(arr, 32), "wam_timing_report")
    return {arr[i].name.decode(): {"launches": arr[i].launches, "ms": arr[i].ms,
                                   "bytes": arr[i].bytes, "flops": arr[i].flops} for i in range(n)}
