"""One action chunk on the GPU: upload the seeded inputs once, then sequence
the C calls (prefill -> optional interval fusion -> N-step denoise).  No
arithmetic of the method here: every step runs in libwam's kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import wam
from .configs import WamConfig


def _tdt(cfg: WamConfig):
    import torch
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def upload_expert(w: dict, cfg: WamConfig, device="cuda") -> wam.DeviceExpert:
    import torch
    mat = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device).to(_tdt(cfg)).contiguous()
    vec = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    gains = ("g1", "g2", "gx")
    layers = [{k: (vec(a) if k in gains else mat(a)) for k, a in l.items()} for l in w["layers"]]
    return wam.DeviceExpert(mat(w["w_in"]), vec(w["g_out"]), mat(w["w_out"]), layers)


def cache_rows(cfg: WamConfig, hist_valid: np.ndarray) -> int:
    """Cache capacity (multiple of 64) for the valid frames of every episode."""
    n = int(hist_valid.sum(axis=1).max()) + cfg.Ff
    return ((n * cfg.P + 63) // 64) * 64


class DeviceChunk:
    """Device-resident inputs, outputs and workspaces of one chunk."""

    def __init__(self, cfg: WamConfig, inp: dict, device="cuda"):
        import torch
        self.cfg = cfg
        self.dt = wam.WAM_BF16 if cfg.dtype == "bf16" else wam.WAM_F32
        self.dims = wam.dims(cfg.L, cfg.D, cfg.Hh, cfg.dh, cfg.Fm, cfg.Cv, cfg.A, cfg.H, cfg.P, self.dt,
                             cfg.Da, cfg.Fma, int(cfg.rope), cfg.Tc, cfg.Ct, cfg.S)
        tdt = _tdt(cfg)
        self.video = upload_expert(inp["video"], cfg, device)
        self.action = upload_expert(inp["action"], cfg, device)
        self.hist = torch.from_numpy(inp["hist"]).to(device).to(tdt).contiguous()
        self.fut = torch.from_numpy(inp["eps_v"]).to(device).to(tdt).contiguous()
        self.eps_a = torch.from_numpy(inp["eps_a"]).to(device).contiguous()
        self.hist_valid = np.ascontiguousarray(inp["hist_valid"], dtype=np.uint8)
        self.logits = inp["fuse_logits"]
        cap = cache_rows(cfg, self.hist_valid)
        self.cache = wam.DeviceKV(cfg.L, cfg.B, cfg.Hh, cfg.dh, cap, self.dt, device)
        self.fused = (wam.DeviceKV(len(cfg.fuse), cfg.B, cfg.Hh, cfg.dh, cap, self.dt, device)
                      if cfg.fuse else None)
        self.kv8 = None
        if cfg.kv_fp8:
            if cfg.dtype != "bf16" or cfg.joint:
                raise wam.WamError("the E4M3 cache option is for bf16 IDM / Faster-WAM chunks")
            self.kv8 = wam.DeviceKV(cfg.n_kv, cfg.B, cfg.Hh, cfg.dh, cap, wam.WAM_FP8, device)
        self.cond_v = self.cond_a = None
        if cfg.Tc > 0:
            # the text/state condition: inputs, and one K/V cache per expert
            self.text = torch.from_numpy(inp["text"]).to(device).to(tdt).contiguous()
            self.state = torch.from_numpy(inp["state"]).to(device).contiguous()
            self.proprio_w = torch.from_numpy(inp["proprio_w"]).to(device).to(tdt).contiguous()
            ccap = (cfg.Tc + 63) // 64 * 64
            self.cond_v = wam.DeviceKV(cfg.L, cfg.B, cfg.Hh, cfg.dh, ccap, self.dt, device)
            self.cond_a = wam.DeviceKV(cfg.L, cfg.B, cfg.Hh, cfg.dh, ccap, self.dt, device)
            self.video.set_cond(self.cond_v)
            self.action.set_cond(self.cond_a)
            self.ws_cond = wam.workspace(wam.condition_workspace_bytes(self.dims, cfg.B), device)
        self.z = torch.zeros((cfg.B, cfg.Ff, cfg.P, cfg.Cv), dtype=torch.float32, device=device)
        self.actions = torch.zeros((cfg.B, cfg.H, cfg.A), dtype=torch.float32, device=device)
        self.vhat = torch.zeros((cfg.N, cfg.B, cfg.H, cfg.A), dtype=torch.float32, device=device)
        if cfg.joint:
            # co-denoising: the prefill covers the history only; the future is
            # denoised together with the actions
            self.ws_prefill = wam.workspace(wam.prefill_workspace_bytes(self.dims, cfg.B, cfg.Fh, 0),
                                            device)
            self.ws_denoise = wam.workspace(
                wam.codenoise_workspace_bytes(self.dims, cfg.B, cfg.Ff, self.cache), device)
            return
        self.ws_prefill = wam.workspace(wam.prefill_workspace_bytes(self.dims, cfg.B, cfg.Fh, cfg.Ff), device)
        kv = self.fused if self.fused is not None else self.cache
        kv.len[:] = cap  # size the workspace for a full cache
        self.ws_denoise = wam.workspace(wam.denoise_workspace_bytes(self.dims, cfg.B, kv), device)

    @property
    def read_kv(self) -> wam.DeviceKV:
        if self.kv8 is not None:
            return self.kv8
        return self.fused if self.fused is not None else self.cache

    def condition(self, stream=None):
        """The condition K/V of both experts, once per call (no-op without one)."""
        c = self.cfg
        if c.Tc > 0:
            wam.prefill_condition_kv(self.dims, self.video, self.action, self.proprio_w, self.text,
                                     self.state, c.B, self.cond_v, self.cond_a, self.ws_cond, stream)

    def prefill(self, stream=None):
        c = self.cfg
        self.condition(stream)
        if c.joint:
            if c.Fh == 0 or not self.hist_valid.any():
                self.cache.len[:] = 0   # no observed history: the joint steps see the future alone
                return
            wam.prefill_video_cache(self.dims, self.video, self.hist, self.hist_valid, c.B, c.Fh, None,
                                    0, c.frame_block[:c.Fh], 0, c.sigma_star, c.shift, self.cache,
                                    None, self.ws_prefill, stream)
            return
        wam.prefill_video_cache(self.dims, self.video, self.hist, self.hist_valid, c.B, c.Fh, self.fut,
                                c.Ff, c.frame_block, c.V, c.sigma_star, c.shift, self.cache, self.z,
                                self.ws_prefill, stream)

    def fuse(self, stream=None):
        """Cache transforms between the prefill and the action steps: the
        interval fusion (SparseMoT) and, with the E4M3 option, quantising what
        the action layers read."""
        c = self.cfg
        if c.fuse:
            wam.fuse_interval_kv(self.cache, [s for s, _ in c.fuse], [n for _, n in c.fuse],
                                 self.logits, self.fused, stream)
        if self.kv8 is not None:
            wam.quantize_kv_fp8(self.fused if self.fused is not None else self.cache, self.kv8, stream)

    def denoise(self, stream=None):
        c = self.cfg
        if c.joint:
            wam.codenoise_chunk(self.dims, self.video, self.action, self.hist_valid, c.B, c.Fh,
                                self.fut, c.Ff, c.frame_block, self.eps_a, c.N, c.video_end,
                                c.shift, self.cache, self.actions, self.z, self.vhat,
                                self.ws_denoise, stream)
            return
        wam.denoise_chunk(self.dims, self.action, self.read_kv, c.read_map, self.eps_a, c.B, c.N,
                          c.shift, self.actions, self.vhat, self.ws_denoise, stream)

    def stream_decision(self, new_frames: int, stream=None):
        """One decision of a streamed history whose last ``new_frames`` history
        frames just arrived: drop the previous future rows, append the new
        frames to the cached history, add the future, then fuse and denoise.
        The first Fh - new_frames frames must already be cached (one
        ``prefill`` of them, or earlier decisions)."""
        c = self.cfg
        old = c.Fh - new_frames
        self.condition(stream)   # the state changes at every decision
        self.cache.len[:] = self.hist_valid[:, :old].sum(axis=1) * c.P
        wam.extend_history_cache(self.dims, self.video, self.hist[:, old:].contiguous(), self.hist_valid,
                                 c.B, old, new_frames, c.frame_block[:c.Fh], self.cache, self.ws_extend,
                                 stream)
        wam.prefill_future(self.dims, self.video, self.hist_valid, c.B, c.Fh, self.fut, c.Ff,
                           c.frame_block, c.V, c.sigma_star, c.shift, self.cache, self.z,
                           self.ws_future, stream)
        self.fuse(stream)
        self.denoise(stream)
        return self.actions

    def prepare_stream(self, new_frames: int, stream=None):
        """Cache the first Fh - new_frames history frames (workspaces for
        ``stream_decision``)."""
        c = self.cfg
        old = c.Fh - new_frames
        self.ws_extend = wam.workspace(wam.prefill_workspace_bytes(self.dims, c.B, new_frames, 0))
        self.ws_future = wam.workspace(wam.prefill_workspace_bytes(self.dims, c.B, 0, c.Ff))
        self.condition(stream)
        wam.prefill_video_cache(self.dims, self.video, self.hist[:, :old].contiguous(),
                                self.hist_valid[:, :old], c.B, old, None, 0, c.frame_block[:old], 0,
                                c.sigma_star, c.shift, self.cache, None, self.ws_prefill, stream)

    def run(self, stream=None):
        """One whole chunk: prefill, fuse (SparseMoT), N action steps (with
        co-denoising: the history prefill, then N joint video + action steps)."""
        self.prefill(stream)
        self.fuse(stream)
        self.denoise(stream)
        return self.actions
