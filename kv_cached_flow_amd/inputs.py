"""Seeded synthetic inputs shared by the oracle and the GPU path.

The only module both sides import.  It draws numbers and rounds them to the
storage type; it holds none of the method's arithmetic.

Recipe (stated once, used everywhere):

* every tensor has its own PCG64 stream, seeded by
  ``SeedSequence([cfg.seed, group, layer, slot])``, so tensors can be drawn
  in any order and in parallel with identical bytes;
* weight matrices ~ N(0, w_std^2) (Wq/Wk rows of the fused QKV matrix use
  ``qk_std``); RMSNorm gains ~ 1 + N(0, w_std^2);
* history/anchor latent tokens, future noise eps_v and action noise eps_a
  ~ N(0, 1); padded history frames are exact zeros; fusion logits ~ N(0, 1);
* with a text/state condition: text tokens (standing in for the text
  encoder's output) and robot state ~ N(0, 1), the proprio encoder and the
  cross-attention matrices ~ N(0, w_std^2), their RMSNorm gains
  ~ 1 + N(0, w_std^2);
* in bf16 workloads every device array is rounded to bf16
  (round-to-nearest-even) and kept as float32 holding bf16 values, so both
  paths consume identical numbers.

Matrices use the out-major layout ``[out_features][in_features]``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import hashlib

import numpy as np

from .configs import WamConfig

_G_VIDEO, _G_ACTION, _G_LOGITS, _G_HIST, _G_EPSV, _G_EPSA = 1, 2, 3, 4, 5, 6
_G_TEXT, _G_STATE, _G_PROPRIO = 7, 8, 9
_S_WIN, _S_G1, _S_QKV, _S_WO, _S_G2, _S_W1, _S_W2, _S_GOUT, _S_WOUT = range(9)
_S_GX, _S_WQX, _S_WKVX, _S_WOX = 9, 10, 11, 12


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    nan = np.isnan(x)
    out = r.view(np.float32)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _normal(cfg: WamConfig, key, shape, std=1.0, mean=0.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, *key])))
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return round_bf16(a) if cfg.dtype == "bf16" else a


LAYER_NAMES = ("g1", "wqkv", "wo", "g2", "w1", "w2")
COND_NAMES = ("gx", "wqx", "wkvx", "wox")


def expert_weights(cfg: WamConfig, which: str, n_layers: int | None = None,
                   pool: _cf.Executor | None = None) -> dict:
    """Weights of one expert.  ``which`` is "video" (in/out width Cv) or
    "action" (in/out width A).  ``n_layers`` truncates the stack (the drawn
    layers are identical to the first layers of the full stack)."""
    g = _G_VIDEO if which == "video" else _G_ACTION
    cio = cfg.Cv if which == "video" else cfg.A
    # hidden width D and MLP width Fm of this expert; Q/K/V use the shared
    # attention interface Dq = Hh * dh
    D, Fm = (cfg.D, cfg.Fm) if which == "video" else (cfg.Dact, cfg.Fact)
    Dq = cfg.Dq
    L = cfg.L if n_layers is None else n_layers

    def qkv(l):
        w = _normal(cfg, (g, l, _S_QKV), (3 * Dq, D), cfg.w_std)
        if cfg.qk_std != cfg.w_std:
            qk = _normal(cfg, (g, l, _S_QKV, 1), (2 * Dq, D), cfg.qk_std)
            w[: 2 * Dq] = qk
        return w

    jobs = {"w_in": lambda: _normal(cfg, (g, 0, _S_WIN), (D, cio), cfg.w_std),
            "g_out": lambda: _normal(cfg, (g, 0, _S_GOUT), (D,), cfg.w_std, 1.0),
            "w_out": lambda: _normal(cfg, (g, 0, _S_WOUT), (cio, D), cfg.w_std)}
    for l in range(L):
        jobs[("g1", l)] = (lambda l=l: _normal(cfg, (g, l, _S_G1), (D,), cfg.w_std, 1.0))
        jobs[("wqkv", l)] = (lambda l=l: qkv(l))
        jobs[("wo", l)] = (lambda l=l: _normal(cfg, (g, l, _S_WO), (D, Dq), cfg.w_std))
        jobs[("g2", l)] = (lambda l=l: _normal(cfg, (g, l, _S_G2), (D,), cfg.w_std, 1.0))
        jobs[("w1", l)] = (lambda l=l: _normal(cfg, (g, l, _S_W1), (Fm, D), cfg.w_std))
        jobs[("w2", l)] = (lambda l=l: _normal(cfg, (g, l, _S_W2), (D, Fm), cfg.w_std))
        if cfg.Tc > 0:
            # cross-attention to the condition: RMSNorm gain, Q from the
            # expert's width, K and V from the condition width, output
            jobs[("gx", l)] = (lambda l=l: _normal(cfg, (g, l, _S_GX), (D,), cfg.w_std, 1.0))
            jobs[("wqx", l)] = (lambda l=l: _normal(cfg, (g, l, _S_WQX), (Dq, D), cfg.w_std))
            jobs[("wkvx", l)] = (lambda l=l: _normal(cfg, (g, l, _S_WKVX), (2 * Dq, cfg.Ct), cfg.w_std))
            jobs[("wox", l)] = (lambda l=l: _normal(cfg, (g, l, _S_WOX), (D, Dq), cfg.w_std))
    if pool is not None:
        futs = {k: pool.submit(f) for k, f in jobs.items()}
        res = {k: f.result() for k, f in futs.items()}
    else:
        res = {k: f() for k, f in jobs.items()}
    names = LAYER_NAMES + (COND_NAMES if cfg.Tc > 0 else ())
    layers = [{n: res[(n, l)] for n in names} for l in range(L)]
    return {"w_in": res["w_in"], "layers": layers, "g_out": res["g_out"],
            "w_out": res["w_out"]}


def history_valid(cfg: WamConfig) -> np.ndarray:
    """Valid flag per (episode, history frame): the earliest ``pad_frames``
    frames of every episode are padding."""
    v = np.ones((cfg.B, cfg.Fh), dtype=np.uint8)
    v[:, : cfg.pad_frames] = 0
    return v


def generate(cfg: WamConfig, n_layers: int | None = None, threads: int = 8) -> dict:
    """All inputs of one chunk.  Arrays are float32 (bf16 values in bf16 workloads)."""
    with _cf.ThreadPoolExecutor(max_workers=threads) as pool:
        video = expert_weights(cfg, "video", n_layers, pool)
        action = expert_weights(cfg, "action", n_layers, pool)
    logits = None
    if cfg.fuse:
        width = max(c for _, c in cfg.fuse)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, _G_LOGITS])))
        logits = rng.standard_normal((len(cfg.fuse), width), dtype=np.float32)
    valid = history_valid(cfg)
    hist = _normal(cfg, (_G_HIST,), (cfg.B, cfg.Fh, cfg.P, cfg.Cv))
    hist[valid == 0] = 0.0
    eps_v = _normal(cfg, (_G_EPSV,), (cfg.B, cfg.Ff, cfg.P, cfg.Cv))
    eps_a = _normal(cfg, (_G_EPSA,), (cfg.B, cfg.H, cfg.A))
    out = {"video": video, "action": action, "fuse_logits": logits,
           "hist": hist, "hist_valid": valid, "eps_v": eps_v, "eps_a": eps_a}
    if cfg.Tc > 0:
        out["text"] = _normal(cfg, (_G_TEXT,), (cfg.B, cfg.Tc - 1, cfg.Ct))
        out["state"] = _normal(cfg, (_G_STATE,), (cfg.B, cfg.Sdim))
        out["proprio_w"] = _normal(cfg, (_G_PROPRIO,), (cfg.Ct, cfg.Sdim), cfg.w_std)
    return out


def fingerprint(inp: dict) -> str:
    """Short SHA-256 over a fixed sample of every array (shape + head + tail),
    so a stored expected value can assert it was computed on these inputs."""
    h = hashlib.sha256()

    def add(a):
        a = np.ascontiguousarray(a)
        h.update(str(a.shape).encode())
        flat = a.reshape(-1)
        h.update(flat[:4096].tobytes())
        h.update(flat[-4096:].tobytes())

    for ex in ("video", "action"):
        w = inp[ex]
        add(w["w_in"]); add(w["g_out"]); add(w["w_out"])
        for lw in w["layers"]:
            for n in LAYER_NAMES + COND_NAMES:
                if n in lw:
                    add(lw[n])
    if inp["fuse_logits"] is not None:
        add(inp["fuse_logits"])
    for n in ("hist", "hist_valid", "eps_v", "eps_a", "text", "state", "proprio_w"):
        if n in inp:
            add(inp[n])
    return h.hexdigest()[:16]
