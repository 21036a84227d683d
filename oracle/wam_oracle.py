"""Oracle for KV-cached action denoising: plain, slow, CPU-only.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the C-ABI library and its Python binding) never calls it, and this module
imports nothing from that path: it shares only the seeded input generator
(``kv_cached_flow_amd.inputs``/``configs``), which holds no arithmetic of the
method.

Written in plain PyTorch CPU ops (a matmul, a softmax, ``erf`` serve as
library steps), float64 for the fp32 workload C0 and float32 for the bf16
workloads, on the same (bf16-rounded) inputs the GPU path consumes; nothing is
rounded here.  Every function states the passage of the pages it follows.  The
pages are:

* "Long-WAM 源码精读" (yeyulingfeng.com), sections 03-04;
* "Fast-WAM 精读" (alicepotter4869.xyz), sections 四 (the text/state
  condition, 四.5), 五 (both experts read the condition through
  cross-attention, step 3) and 七;
* "Long-WAM: Scaling the Context of World-Action Models | Summary"
  (greeksharifa.github.io), sections 3.1, 3.2, 4.2 (text/state KV reused
  across denoising steps) and appendix B.2;
* "世界模型之Faster-WAM详解" (171host.com), sections 3.1-3.4.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
closed forms, library routines, special cases or brute force.  The composite
network output (``run_chunk``) has no numeric example on the pages: it is
pinned through its parts and through the structural identities (joint
sequence == cached path, cached history == recompute, padding invariance),
not against printed values.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np
import torch

RMS_EPS = 1e-6

# --------------------------------------------------------------------------
# Schedules and the flow path
# --------------------------------------------------------------------------


def phi(u: float, shift: float) -> float:
    """Time-shift map applied to the uniform grid u in [0, 1].

    The Long-WAM code close-reading (section 04, 对照一) names ``_phi(u, shift)``
    without defining it.  Reading adopted: the usual flow-matching shift
    s*u / (1 + (s-1)*u), which is the identity for s = 1 (every workload here);
    the endpoints are pinned to 0 and 1 exactly.
    """
    if u == 0.0:
        return 0.0
    if u == 1.0:
        return 1.0
    if shift == 1.0:
        return u
    return shift * u / (1.0 + (shift - 1.0) * u)


def schedule(steps: int, sigma_end: float, shift: float = 1.0) -> np.ndarray:
    """Noise levels sigma_0 .. sigma_steps, computed in float64, stored float32.

    Long-WAM code close-reading, section 04 (对照一): a uniform grid from 1 to 0
    with steps+1 points, mapped through ``_phi``, re-calibrated so that the
    first level is pure noise and the last is exactly sigma* (0.9 for the IDM
    video steps).  Reading: sigma_k = sigma_end + (1 - sigma_end) * phi(1 - k/steps).
    Action steps use sigma_end = 0 (1 -> 0, "Fast-WAM" page section 七).
    sigma_end is taken as a float64 number (0.9, not its float32 rounding).
    """
    if steps < 1:
        raise ValueError("steps must be >= 1")
    se = float(sigma_end)
    out = []
    for k in range(steps + 1):
        u = 1.0 - k / steps
        out.append(se + (1.0 - se) * phi(u, shift))
    return np.asarray(out, dtype=np.float64).astype(np.float32)


def flow_point(x0, eps, sigma):
    """Point on the flow path x_sigma = (1 - sigma) x + sigma eps (Long-WAM
    close-reading section 03; Fast-WAM page section 五 step 5)."""
    return (1.0 - sigma) * x0 + sigma * eps


def flow_velocity(x0, eps):
    """Velocity target u = eps - x (Long-WAM close-reading section 03)."""
    return eps - x0


def euler_step(x, v, sigma, sigma_next):
    """One Euler step of dx/dsigma = u from sigma to sigma_next.

    The pages only say the scheduler "updates the latent" after each pass
    (Fast-WAM page section 七.2).  Since d x_sigma / d sigma = eps - x = u on the
    linear path, the step is x + (sigma_next - sigma) * v.
    """
    return x + (float(sigma_next) - float(sigma)) * v


def integrate(x_init, sigmas: Sequence[float], velocity: Callable):
    """Run Euler over a schedule; ``velocity(x, k, sigma_k)`` returns v-hat.
    Returns the final state and the list of v-hat per step."""
    x = x_init
    vs = []
    for k in range(len(sigmas) - 1):
        v = velocity(x, k, float(sigmas[k]))
        vs.append(v)
        x = euler_step(x, v, sigmas[k], sigmas[k + 1])
    return x, vs


# --------------------------------------------------------------------------
# Layer pieces
# --------------------------------------------------------------------------


def time_embedding(sigma: float, D: int, dtype=torch.float64) -> torch.Tensor:
    """Sinusoidal embedding of the flow time, added to every token.

    The pages do not give the conditioning form (they speak of per-token noise
    levels, "Faster-WAM" page section 3.4).  Reading: t = 1000*sigma,
    w_i = 10000^(-i/(D/2)), emb = [cos(t w_0..), sin(t w_0..)], in float64.
    """
    t = 1000.0 * float(sigma)
    half = D // 2
    i = torch.arange(half, dtype=torch.float64)
    w = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -i / half)
    a = t * w
    return torch.cat([torch.cos(a), torch.sin(a)]).to(dtype)


def rmsnorm(x: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """RMSNorm(x; g) = x * (mean(x^2) + eps)^(-1/2) * g, eps = 1e-6 (the
    pages give no normalisation details; a pre-norm block is the reading)."""
    return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + RMS_EPS) * g


def gelu(x: torch.Tensor) -> torch.Tensor:
    """Exact GELU, 0.5 x (1 + erf(x / sqrt 2)) (the workload's "GELU MLP")."""
    return 0.5 * x * (1.0 + torch.erf(x / math.sqrt(2.0)))


MaskFn = Callable[[int, int], torch.Tensor]


def attention(q, k, v, allow: Optional[MaskFn] = None, q_chunk: int = 1024):
    """Scaled dot-product attention, one head at a time in a batch.

    q [nq, Hh, dh], k/v [nk, Hh, dh]; ``allow(q0, q1)`` returns the boolean
    visibility of keys for query rows q0..q1 (None: every key visible).
    s_ij = q_i.k_j / sqrt(dh) over visible keys, p = softmax_j(s),
    o_i = sum_j p_ij v_j.  A row with no visible key returns zeros (only
    padding rows, whose outputs nobody reads, can be in that case).
    Query rows are processed in chunks only to bound memory.
    """
    nq, Hh, dh = q.shape
    scale = 1.0 / math.sqrt(dh)
    kh = k.permute(1, 2, 0)          # [Hh, dh, nk]
    vh = v.permute(1, 0, 2)          # [Hh, nk, dh]
    out = torch.empty_like(q)
    for q0 in range(0, nq, q_chunk):
        q1 = min(nq, q0 + q_chunk)
        qh = q[q0:q1].permute(1, 0, 2)                    # [Hh, qc, dh]
        s = torch.matmul(qh, kh) * scale                  # [Hh, qc, nk]
        if allow is not None:
            m = allow(q0, q1)                             # [qc, nk]
            s = s.masked_fill(~m.unsqueeze(0), float("-inf"))
            empty = ~m.any(dim=1)
            if bool(empty.any()):
                s[:, empty, :] = 0.0
            p = torch.softmax(s, dim=-1)
            if bool(empty.any()):
                p[:, empty, :] = 0.0
        else:
            p = torch.softmax(s, dim=-1)
        out[q0:q1] = torch.matmul(p, vh).permute(1, 0, 2)
    return out


ROPE_BASE = 10000.0


def rope(x, pos):
    """Rotary position embedding of x [n, Hh, dh] at token positions pos [n].

    The pages only say that the rotary position tables, which encode token
    positions, are computed once per inference call and reused across the
    denoising steps (Long-WAM Summary section 4.2).  Reading adopted (an
    option; the workloads C1-C6 run without it): the rotation of the usual
    rotary embedding, pair j = (x[2j], x[2j+1]) of every head taken as the
    complex number x[2j] + i x[2j+1] and multiplied by exp(i p w_j) with
    w_j = 10000^(-2j/dh), p the token's position.  Angles in float64.
    """
    n, Hh, dh = x.shape
    j = torch.arange(dh // 2, dtype=torch.float64)
    w = ROPE_BASE ** (-2.0 * j / dh)
    ang = pos.to(torch.float64)[:, None] * w[None, :]            # [n, dh/2]
    c = torch.cos(ang).to(x.dtype)[:, None, :]
    sn = torch.sin(ang).to(x.dtype)[:, None, :]
    a, b = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = a * c - b * sn
    out[..., 1::2] = a * sn + b * c
    return out


def token_positions(cfg, first: int, n: int) -> Optional[torch.Tensor]:
    """Positions first .. first + n - 1 with the rotary option on, else None.

    Reading adopted for the position of a token: its index in the episode's
    joint sequence as the attention sees it, [valid history rows in frame
    order ; future rows ; the action chunk] (padded frames are not in it), so
    that appending frames leaves every cached row's position unchanged."""
    if not getattr(cfg, "rope", False):
        return None
    return torch.arange(first, first + n, dtype=torch.int64)


def layer(X, w: dict, Hh: int, ctx: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
          allow: Optional[MaskFn] = None, kv_only: bool = False, pos=None,
          cond: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """One expert layer on token states X [n, D] with attention context ctx.

    Keys and values are [ctx ; this layer's own K, V] ("Fast-WAM" page
    section 七.2: K = [K_video ; K_action], V likewise).  Block:
      Y = RMSNorm(X; g1); Q, K, V = Y Wq^T, Y Wk^T, Y Wv^T (split into heads);
      X += concat(attn) Wo^T;  X += GELU(RMSNorm(X; g2) W1^T) W2^T.
    No biases.  Returns (X_out, K, V); K, V are this layer's cache rows.
    With ``kv_only`` only K, V are produced (X_out is None).
    Q, K and V have the width Dq = Hh * dh of the attention interface the two
    experts share (24 heads x 128 on the "Fast-WAM 精读" page, section 四.4),
    which may differ from the expert's own width D (Wqkv [3 Dq][D], Wo [D][Dq]).
    With ``pos`` (token positions [n]) Q and K are rotated by ``rope`` before
    the attention, so the K rows returned for the cache are rotated too.
    With ``cond`` (this layer's condition K, V [Tc, Hh, dh], ``condition_kv``)
    a cross-attention sub-layer follows the self-attention:
      X += Attn(RMSNorm(X; gx) Wqx^T ; K_c, V_c) Wox^T
    (the tokens read the text/state condition through cross-attention,
    "Fast-WAM 精读" section 五, step 3; no rotary positions there).
    """
    n, D = X.shape
    Dq = w["wqkv"].shape[0] // 3
    dh = Dq // Hh
    Y = rmsnorm(X, w["g1"])
    qkv = Y @ w["wqkv"].T
    Q = qkv[:, :Dq].reshape(n, Hh, dh)
    K = qkv[:, Dq:2 * Dq].reshape(n, Hh, dh)
    V = qkv[:, 2 * Dq:].reshape(n, Hh, dh)
    if pos is not None:
        Q, K = rope(Q, pos), rope(K, pos)
    if kv_only:
        return None, K, V
    if ctx is not None:
        Kall = torch.cat([ctx[0], K], dim=0)
        Vall = torch.cat([ctx[1], V], dim=0)
    else:
        Kall, Vall = K, V
    O = attention(Q, Kall, Vall, allow)
    X = X + O.reshape(n, Dq) @ w["wo"].T
    if cond is not None:
        Qx = (rmsnorm(X, w["gx"]) @ w["wqx"].T).reshape(n, Hh, dh)
        X = X + attention(Qx, cond[0], cond[1]).reshape(n, Dq) @ w["wox"].T
    X = X + gelu(rmsnorm(X, w["g2"]) @ w["w1"].T) @ w["w2"].T
    return X, K, V


def condition(text_b, state_b, proprio_w):
    """The condition sequence of one episode [Tc, Ct]: the text tokens (the
    text encoder's output, "Fast-WAM 精读" section 四.5), then one proprio token
    that a linear layer makes from the robot state, of the text tokens' width,
    appended after them (same section)."""
    return torch.cat([text_b, (state_b @ proprio_w.T).unsqueeze(0)])


def condition_kv(ctx, lw: dict, Hh: int):
    """K, V [Tc, Hh, dh] of the condition for one expert layer: ctx Wk_x^T and
    ctx Wv_x^T with wkvx = [Wk_x ; Wv_x].  They do not depend on the flow time
    or on any latent, so they are computed once per inference call and reused
    at every denoising step (text/state KV, Long-WAM Summary section 4.2)."""
    Dq = lw["wkvx"].shape[0] // 2
    kv = ctx @ lw["wkvx"].T
    n = ctx.shape[0]
    return kv[:, :Dq].reshape(n, Hh, -1), kv[:, Dq:].reshape(n, Hh, -1)


def condition_cache(cfg, w: dict, ctx):
    """Per-layer condition K, V of one expert (None without a condition)."""
    if ctx is None:
        return None
    return [condition_kv(ctx, lw, cfg.Hh) for lw in w["layers"]]


def _cl(cond, l):
    return None if cond is None else cond[l]


def head(X, g_out, w_out):
    """Velocity head v-hat = RMSNorm(X_L; g_out) W_out^T."""
    return rmsnorm(X, g_out) @ w_out.T


def embed(x, w_in, sigma: float, D: int):
    """Token embedding X = x W_in^T + emb(sigma) (the action expert maps each
    action step to the hidden width with one linear layer, "Fast-WAM" page
    section 四.3; the video side is the same form on latent channels)."""
    return x @ w_in.T + time_embedding(sigma, D, x.dtype)


# --------------------------------------------------------------------------
# Masks
# --------------------------------------------------------------------------


def video_visible(frame_q: torch.Tensor, frame_k: torch.Tensor,
                  block: torch.Tensor, valid: torch.Tensor) -> torch.Tensor:
    """Visibility of video key tokens for video query tokens.

    A video query reads its own and earlier temporal blocks ("Long-WAM ...
    Summary" page, section 3.2; Faster-WAM page section 3.1: future slots read
    the anchor and each other, the anchor does not read future slots), and
    never a padded frame (appendix B.2: padding is masked).  Video rows never
    see action tokens: no action column exists in any video pass.
    allow(q, k) = valid(f(k)) and block(f(k)) <= block(f(q)).
    """
    bq = block[frame_q].unsqueeze(1)
    bk = block[frame_k].unsqueeze(0)
    return (bk <= bq) & valid[frame_k].unsqueeze(0).bool()


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------


def to_torch_expert(w: dict, dtype) -> dict:
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dtype)
    return {"w_in": t(w["w_in"]), "g_out": t(w["g_out"]), "w_out": t(w["w_out"]),
            "layers": [{k: t(v) for k, v in lw.items()} for lw in w["layers"]]}


def oracle_dtype(cfg) -> torch.dtype:
    return torch.float64 if cfg.dtype == "f32" else torch.float32


def history_cache(cfg, vw: dict, hist_b, valid_b, drop_padded: bool = True, cond=None):
    """History/anchor prefill of one episode: the history tokens at sigma = 0
    run through the L layers with block-causal attention and each layer's
    K, V are kept (Fast-WAM page section 七.1, ``prefill_video_cache``;
    Long-WAM Summary section 3.2).  The last layer only needs K, V.

    Returns (cache_h: list of (K, V) [Th, Hh, dh] per layer, fall: frame index
    of every [history ; future] token, valid: frame validity [Fh + Ff],
    mask_f: visibility of [history ; future] keys for the future queries).
    """
    dt = vw["w_in"].dtype
    P, Fh, Ff, D, Hh, L = cfg.P, cfg.Fh, cfg.Ff, cfg.D, cfg.Hh, len(vw["layers"])
    hist_frames = [f for f in range(Fh) if (valid_b[f] or not drop_padded)]
    fut_frames = [Fh + j for j in range(Ff)]
    block = torch.tensor(cfg.frame_block, dtype=torch.int64)
    valid = torch.tensor(list(valid_b) + [1] * Ff, dtype=torch.int64)
    fh = torch.tensor(hist_frames, dtype=torch.int64).repeat_interleave(P)
    ff = torch.tensor(fut_frames, dtype=torch.int64).repeat_interleave(P)
    fall = torch.cat([fh, ff])

    hist_tok = torch.from_numpy(np.ascontiguousarray(hist_b[hist_frames])).to(dt).reshape(-1, cfg.Cv)
    mask_h = lambda q0, q1: video_visible(fh[q0:q1], fh, block, valid)
    mask_f = lambda q0, q1: video_visible(ff[q0:q1], fall, block, valid)

    cache_h = []
    if len(hist_frames):
        X = embed(hist_tok, vw["w_in"], 0.0, D)
        pos = None
        if getattr(cfg, "rope", False):
            # a token's position counts the valid tokens before it (padded
            # tokens, kept only with drop_padded=False, are masked keys)
            vt = valid[fh]
            pos = torch.cumsum(vt, 0) - vt
        for l, lw in enumerate(vw["layers"]):
            X, K, V = layer(X, lw, Hh, None, mask_h, kv_only=(l == L - 1), pos=pos,
                            cond=_cl(cond, l))
            cache_h.append((K, V))
    else:
        empty = torch.zeros((0, Hh, cfg.dh), dtype=dt)
        cache_h = [(empty, empty)] * L
    return cache_h, fall, valid, mask_f


def extend_history(cfg, vw: dict, cache_old, n_old: int, hist_b, valid_b, cond=None):
    """Append history frames n_old..Fh-1 of one episode to the cache of its
    first n_old frames (their valid rows, in order): the new frames' tokens at
    sigma = 0 run through the L layers with keys [cached rows ; new rows]
    under the block rule, and their K, V are appended.

    Streaming observation encoding: frames are encoded as they arrive, not
    when the whole window is complete (the Long-WAM tutorial, section 三;
    Long-WAM Summary section 4.1).  Old rows are not recomputed: under the
    block rule a frame reads no later block, so appending is exact when the
    new frames start a new temporal block (frames of one block read each
    other) and no frame leaves the window; eviction, or a change of the
    temporal positions, invalidates the cache (Long-WAM Summary appendix
    B.2) and needs a new prefill.
    """
    dt = vw["w_in"].dtype
    P, Fh, Ff, D, Hh, L = cfg.P, cfg.Fh, cfg.Ff, cfg.D, cfg.Hh, len(vw["layers"])
    old = [f for f in range(n_old) if valid_b[f]]
    new = [f for f in range(n_old, Fh) if valid_b[f]]
    if not new:
        return cache_old
    block = torch.tensor(cfg.frame_block, dtype=torch.int64)
    valid = torch.tensor(list(valid_b) + [1] * Ff, dtype=torch.int64)
    fo = torch.tensor(old, dtype=torch.int64).repeat_interleave(P)
    fn = torch.tensor(new, dtype=torch.int64).repeat_interleave(P)
    fall = torch.cat([fo, fn])
    mask = lambda q0, q1: video_visible(fn[q0:q1], fall, block, valid)
    tok = torch.from_numpy(np.ascontiguousarray(hist_b[new])).to(dt).reshape(-1, cfg.Cv)
    X = embed(tok, vw["w_in"], 0.0, D)
    pos = token_positions(cfg, int(cache_old[0][0].shape[0]), X.shape[0])
    cache = []
    for l, lw in enumerate(vw["layers"]):
        X, K, V = layer(X, lw, Hh, cache_old[l], mask, kv_only=(l == L - 1), pos=pos,
                        cond=_cl(cond, l))
        cache.append((torch.cat([cache_old[l][0], K]), torch.cat([cache_old[l][1], V])))
    return cache


def video_prefill(cfg, vw: dict, hist_b, valid_b, eps_v_b, drop_padded: bool = True, cond=None):
    """Video expert for one episode: history prefill, imagine, cache pass.

    * History/anchor tokens at sigma = 0 run through the L layers with
      block-causal attention; each layer's K, V are kept (Fast-WAM page
      section 七.1, ``prefill_video_cache``; Long-WAM Summary section 3.2).
    * Imagine (V >= 1): future latents start from noise and take V Euler steps
      to sigma* = 0.9, keys = [history cache ; future] under the same block
      rule; they are never decoded (Long-WAM close-reading sections 03-04;
      Summary section 3.2).
    * Cache pass: the future latents at sigma* (or, with V = 0, the noise at
      video time 1, Faster-WAM page section 3.1) run once more and their
      per-layer K, V are appended to the cache.  The last layer only needs K, V.

    ``drop_padded`` leaves padded history frames out of the token list; with
    False they are kept as tokens and masked as keys (the result on valid
    rows is the same, a pinned identity).
    Returns (cache: list of (K, V) [T, Hh, dh] per layer over the valid rows
             in frame order, z: [Ff*P, Cv], frames: frame index per cache row).
    """
    dt = vw["w_in"].dtype
    D, Hh, L = cfg.D, cfg.Hh, len(vw["layers"])
    cache_h, fall, valid, mask_f = history_cache(cfg, vw, hist_b, valid_b, drop_padded, cond)

    z = torch.from_numpy(np.ascontiguousarray(eps_v_b)).to(dt).reshape(-1, cfg.Cv)
    pos_f = token_positions(cfg, int(sum(valid_b[:cfg.Fh])) * cfg.P, z.shape[0])
    if cfg.V >= 1:
        sig = schedule(cfg.V, cfg.sigma_star, cfg.shift)

        def vel(zc, k, s):
            X = embed(zc, vw["w_in"], s, D)
            for l, lw in enumerate(vw["layers"]):
                X, _, _ = layer(X, lw, Hh, cache_h[l], mask_f, pos=pos_f, cond=_cl(cond, l))
            return head(X, vw["g_out"], vw["w_out"])

        z, _ = integrate(z, sig, vel)
        sigma_f = float(sig[-1])
    else:
        sigma_f = 1.0

    cache = []
    keep = valid[fall].bool()          # the cache holds valid rows only
    X = embed(z, vw["w_in"], sigma_f, D)
    for l, lw in enumerate(vw["layers"]):
        X, K, V = layer(X, lw, Hh, cache_h[l], mask_f, kv_only=(l == L - 1), pos=pos_f,
                        cond=_cl(cond, l))
        cache.append((torch.cat([cache_h[l][0], K])[keep], torch.cat([cache_h[l][1], V])[keep]))
    return cache, z, fall[keep]


def fusion_weights(logits_row, count: int) -> np.ndarray:
    """Softmax-normalised fusion weights of one interval, in float64
    (Faster-WAM page section 3.3: W^fuse is softmax-normalised)."""
    x = np.asarray(logits_row[:count], dtype=np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / e.sum()


def fuse_interval(cache: List[Tuple[torch.Tensor, torch.Tensor]], fuse, logits):
    """Interval KV-Fusion: (K_bar, V_bar)_m = sum_{j in I_m} W_{m,j} (K_j, V_j).

    Faster-WAM page section 3.3.  One scalar weight per (m, j), shared by K
    and V, all heads and all tokens; the fused pair has one layer's length.
    """
    out = []
    for m, (s, c) in enumerate(fuse):
        w = fusion_weights(logits[m], c)
        Kb = sum(float(w[j]) * cache[s + j][0] for j in range(c))
        Vb = sum(float(w[j]) * cache[s + j][1] for j in range(c))
        out.append((Kb, Vb))
    return out


def action_velocity(cfg, aw: dict, kv_read: List[Optional[Tuple]], a, sigma: float,
                    pos0: int = 0, cond=None):
    """One pass of the action expert at flow time sigma: v-hat for the chunk.

    Per layer the 32 action queries attend over [video K/V read by this layer ;
    the chunk's own K/V], or over the chunk alone where the layer reads
    nothing (SparseMoT, Faster-WAM page section 3.2); no mask among action
    tokens (Long-WAM Summary section 3.2: the entire noisy chunk is visible).
    ``pos0``: position of the first action token (the episode's cached rows
    come first) for the rotary option.  ``cond``: the action expert's
    per-layer condition K, V (``condition_cache``), or None.
    """
    X = embed(a, aw["w_in"], sigma, cfg.Dact)
    pos = token_positions(cfg, pos0, X.shape[0])
    for l, lw in enumerate(aw["layers"]):
        X, _, _ = layer(X, lw, cfg.Hh, kv_read[l], None, pos=pos, cond=_cl(cond, l))
    return head(X, aw["g_out"], aw["w_out"])


def denoise(cfg, aw: dict, kv_read, eps_a_b, pos0: int = 0, cond=None):
    """N Euler steps of the action flow from noise at t=1 to t=0, re-reading
    the same video K/V (and condition K/V) at every step (Fast-WAM page
    section 七.2-七.3)."""
    t = schedule(cfg.N, 0.0, cfg.shift)
    a = torch.from_numpy(np.ascontiguousarray(eps_a_b)).to(aw["w_in"].dtype)
    return integrate(a, t, lambda x, k, s: action_velocity(cfg, aw, kv_read, x, s, pos0, cond))


def read_layers(cfg, cache, fused):
    """The K/V each action layer reads: cache[l] (dense MoT pairing, Fast-WAM
    page section 四.4), fused pair m at interaction layers, nothing elsewhere."""
    src = fused if cfg.fuse else cache
    return [None if r < 0 else src[r] for r in cfg.read_map]


def episode_condition(cfg, inp: dict, b: int, dt):
    """Condition sequence of episode b (None without one)."""
    if cfg.Tc <= 0:
        return None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt)
    return condition(t(inp["text"][b]), t(inp["state"][b]), t(inp["proprio_w"]))


def run_chunk(cfg, inp: dict, dtype=None, drop_padded: bool = True,
              cache_sampler: Optional[Callable] = None, keep_cache: bool = False,
              kv_fp8: bool = False):
    """Whole chunk per episode: prefill -> (fuse) -> N action steps.

    Returns actions [B, H, A] (numpy float64), z [B, Ff*P, Cv], v-hat per
    step [N, B, H, A]; with ``keep_cache`` also the cache per episode (valid
    rows, in frame order) and the fused pairs.  ``kv_fp8``: the action layers
    read the E4M3 form of their K/V (``quantize_kv_fp8``).  ``cache_sampler(b, cache,
    fused)`` is called per episode before the cache is dropped.
    """
    dt = dtype or oracle_dtype(cfg)
    vw = to_torch_expert(inp["video"], dt)
    aw = to_torch_expert(inp["action"], dt)
    acts, zs, vhs, caches, fuseds = [], [], [], [], []
    for b in range(cfg.B):
        ctx = episode_condition(cfg, inp, b, dt)
        condv, conda = condition_cache(cfg, vw, ctx), condition_cache(cfg, aw, ctx)
        cache, z, _ = video_prefill(cfg, vw, inp["hist"][b], inp["hist_valid"][b],
                                    inp["eps_v"][b], drop_padded, condv)
        fused = fuse_interval(cache, cfg.fuse, inp["fuse_logits"]) if cfg.fuse else None
        kv_read = read_layers(cfg, cache, fused)
        if kv_fp8:
            kv_read = quantize_read(kv_read)
        a, vh = denoise(cfg, aw, kv_read, inp["eps_a"][b], int(cache[0][0].shape[0]), conda)
        if cache_sampler is not None:
            cache_sampler(b, cache, fused)
        acts.append(a.double().numpy())
        zs.append(z.double().numpy())
        vhs.append(np.stack([v.double().numpy() for v in vh]))
        if keep_cache:
            caches.append(cache)
            fuseds.append(fused)
    out = {"actions": np.stack(acts), "z": np.stack(zs),
           "vhat": np.stack(vhs, axis=1)}
    if keep_cache:
        out["cache"] = caches
        out["fused"] = fuseds
    return out


# --------------------------------------------------------------------------
# Co-denoising (CoD)
# --------------------------------------------------------------------------


def codenoise(cfg, vw: dict, aw: dict, hist_b, valid_b, eps_v_b, eps_a_b, steps: int,
              sigma_video_end: float = 0.0, condv=None, conda=None):
    """Co-denoising of one episode: the future video latents and the action
    chunk take the same number of Euler steps together.

    The pages set CoD beside IDM: video and actions are updated jointly
    (Long-WAM Summary section 3.2, Figure 2; the page "Long-WAM：机器人操作模型
    的长历史..." section 三, the four-strategy figure), and the joint inference
    call creates both latents and returns both after its iterations ("Fast-WAM
    精读" page, section 03).  In every pass video queries never read action
    tokens, and action queries read the observed history, the partially
    denoised future and the whole noisy chunk (same two places).

    Reading adopted (the pages give no step-level listing): one shared step
    count (the pages time CoD as V4/A4 and V2/A2, Long-WAM Summary appendix F);
    video levels sigma_v = schedule(steps, sigma_video_end) (0: the returned
    video is fully denoised), action levels t = schedule(steps, 0).  Step k:
      1. the future at sigma_v[k] runs through the video layers with keys
         [history cache ; future] under the block rule -> v-hat_video and the
         future K, V of every layer;
      2. the action expert at t[k] reads [history ; future at sigma_v[k]] at
         every layer it pairs with -> v-hat_action;
      3. z += (sigma_v[k+1] - sigma_v[k]) v-hat_video, a += (t[k+1] - t[k])
         v-hat_action.
    Since video rows never read actions, computing step 1 before step 2 is
    the same as one joint pass over [history ; future ; actions].

    Returns (a, z, per-step list of (z_k, a_k, vhat_video_k, vhat_action_k),
    cache: per layer (K, V) over [history ; future at the last video level]).
    """
    dt = vw["w_in"].dtype
    D, Hh = cfg.D, cfg.Hh
    if cfg.fuse:
        raise ValueError("co-denoising reads the per-layer cache (no interval fusion)")
    cache_h, fall, valid, mask_f = history_cache(cfg, vw, hist_b, valid_b, cond=condv)
    sv = schedule(steps, sigma_video_end, cfg.shift)
    ta = schedule(steps, 0.0, cfg.shift)
    z = torch.from_numpy(np.ascontiguousarray(eps_v_b)).to(dt).reshape(-1, cfg.Cv)
    a = torch.from_numpy(np.ascontiguousarray(eps_a_b)).to(dt)
    Th = int(cache_h[0][0].shape[0])
    pos_f = token_positions(cfg, Th, z.shape[0])
    traj = []
    cache = None
    for k in range(steps):
        X = embed(z, vw["w_in"], float(sv[k]), D)
        cache = []
        for l, lw in enumerate(vw["layers"]):
            X, K, V = layer(X, lw, Hh, cache_h[l], mask_f, pos=pos_f, cond=_cl(condv, l))
            cache.append((torch.cat([cache_h[l][0], K]), torch.cat([cache_h[l][1], V])))
        v_v = head(X, vw["g_out"], vw["w_out"])
        v_a = action_velocity(cfg, aw, [None if r < 0 else cache[r] for r in cfg.read_map],
                              a, float(ta[k]), Th + z.shape[0], conda)
        traj.append((z, a, v_v, v_a))
        z = euler_step(z, v_v, sv[k], sv[k + 1])
        a = euler_step(a, v_a, ta[k], ta[k + 1])
    return a, z, traj, cache


def run_codenoise(cfg, inp: dict, dtype=None, steps: Optional[int] = None,
                  sigma_video_end: Optional[float] = None, keep_cache: bool = False,
                  cache_sampler: Optional[Callable] = None):
    """CoD for every episode (``codenoise``); ``steps`` = cfg.N and
    ``sigma_video_end`` = cfg.video_end by default.  Returns actions
    [B, H, A], z [B, Ff*P, Cv] (float64 numpy) and the action v-hat per step
    [steps, B, H, A]; with ``keep_cache`` also the cache per episode
    (history ; future at the last video level).  ``cache_sampler(b, cache,
    None)`` is called per episode before the cache is dropped."""
    dt = dtype or oracle_dtype(cfg)
    n = steps or cfg.N
    end = cfg.video_end if sigma_video_end is None else sigma_video_end
    vw = to_torch_expert(inp["video"], dt)
    aw = to_torch_expert(inp["action"], dt)
    acts, zs, vhs, caches = [], [], [], []
    for b in range(cfg.B):
        ctx = episode_condition(cfg, inp, b, dt)
        a, z, traj, cache = codenoise(cfg, vw, aw, inp["hist"][b], inp["hist_valid"][b],
                                      inp["eps_v"][b], inp["eps_a"][b], n, end,
                                      condition_cache(cfg, vw, ctx), condition_cache(cfg, aw, ctx))
        if cache_sampler is not None:
            cache_sampler(b, cache, None)
        acts.append(a.double().numpy())
        zs.append(z.double().numpy())
        vhs.append(np.stack([t[3].double().numpy() for t in traj]))
        if keep_cache:
            caches.append(cache)
    out = {"actions": np.stack(acts), "z": np.stack(zs), "vhat": np.stack(vhs, axis=1)}
    if keep_cache:
        out["cache"] = caches
    return out


# --------------------------------------------------------------------------
# FP8 (E4M3) key/value cache: an option that departs from the pages' bf16 cache
# --------------------------------------------------------------------------
#
# Long-WAM keeps its KV storage in bf16 (Long-WAM Summary section 4.2), while
# the LongLive-2.0 stack it builds on quantises its KV cache block by block
# (the Long-WAM tutorial, section 三).  The option here stores the cache the
# action expert reads as OCP E4M3 codes with one power-of-two scale per
# (head, 64-key tile) for K and one for V.  A power of two makes code * scale
# exact in bf16 and fp32, so the GPU's dequantised operands are exactly the
# values below.

E4M3_MAX = 448.0
KV_TILE = 64


def e4m3_value(code: int) -> float:
    """Value of one OCP 8-bit E4M3 code: sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 is subnormal, (m/8) 2^-6; S.1111.111 is
    NaN and there is no infinity (OCP 8-bit floating-point specification)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)])
_E4M3_POS = _E4M3_TABLE[:0x7F]        # codes 0..126: the finite non-negative values, increasing


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes, dtype=np.int64)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code, ties to the even code (|x| <= 448, no NaN); the sign
    bit follows the sign of x (negative values that round to 0 give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.isnan(a).any() or (a > E4M3_MAX).any():
        raise ValueError("E4M3 encoding needs finite |x| <= 448")
    hi = np.minimum(np.searchsorted(_E4M3_POS, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


KV_MIN_EXP = -126   # 2^-126: the smallest normal float32 number


def kv_tile_exponent(amax: float) -> int:
    """Smallest integer e >= -126 with amax <= 448 * 2^e (0 for an all-zero
    tile).  The pages fix no scale format (the LongLive-2.0 stack quantises its
    KV cache block by block, the Long-WAM tutorial section 三); reading adopted:
    the scale 2^e is a normal float32 number, so tiles whose largest value is
    below 448 * 2^-127 keep e = -126 (their codes are then smaller than 224)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    if amax <= E4M3_MAX * 2.0 ** (KV_MIN_EXP - 1):
        return KV_MIN_EXP
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_kv_fp8(K, V):
    """E4M3 cache of one layer (K, V [T, Hh, dh], the valid rows from row 0).

    Per head and 64-row tile (the last one ragged) of K, and likewise of V:
    e = kv_tile_exponent(max |x| over the tile), code = E4M3(x / 2^e) and the
    value read back is value(code) 2^e.  Returns (K', V') dequantised in the
    input dtype and, for the bit-exact tests, (codes_K, exps_K, codes_V,
    exps_V) with exps [Hh, tiles].
    """
    res = []
    for X in (K, V):
        Xn = X.double().numpy()
        T, Hh, dh = Xn.shape
        nt = (T + KV_TILE - 1) // KV_TILE
        exps = np.zeros((Hh, nt), dtype=np.int64)
        codes = np.zeros(Xn.shape, dtype=np.uint8)
        deq = np.zeros(Xn.shape)
        for h in range(Hh):
            for t in range(nt):
                r0, r1 = t * KV_TILE, min(T, (t + 1) * KV_TILE)
                blk = Xn[r0:r1, h, :]
                e = kv_tile_exponent(np.max(np.abs(blk)))
                c = e4m3_encode(blk / 2.0 ** e)
                exps[h, t] = e
                codes[r0:r1, h, :] = c
                deq[r0:r1, h, :] = e4m3_decode(c) * 2.0 ** e
        res.append((torch.from_numpy(deq).to(X.dtype), codes, exps))
    (Kq, ck, ek), (Vq, cv, ev) = res
    return Kq, Vq, (ck, ek, cv, ev)


def quantize_read(kv_read):
    """The FP8 option applied to what the action layers read (None stays)."""
    return [None if kv is None else quantize_kv_fp8(kv[0], kv[1])[:2] for kv in kv_read]


# --------------------------------------------------------------------------
# Uncached references used by the structural pins
# --------------------------------------------------------------------------


def joint_mot_step(cfg, vw: dict, aw: dict, video_tok, video_sigma, video_frames,
                   frame_valid, a, t: float, video_head: bool = False, ctx=None):
    """One pass of the two experts over ONE joint sequence [video ; action],
    with no cache: each row uses its expert's weights, one attention over the
    union with an explicit mask where video rows see video columns by the
    block rule and never action columns, and action rows see every valid
    video column and every action column (Long-WAM Summary section 3.2's
    asymmetric interface; Fast-WAM page section 四.4 layer pairing).

    video_tok [Nv, Cv] at per-row levels video_sigma [Nv]; a [H, A] at t.
    Returns (v-hat of the action rows, per-layer video (K, V)), and with
    ``video_head`` also the video expert's v-hat of every video row.
    With a condition sequence ``ctx`` [Tc, Ct], every row then reads it
    through its own expert's cross-attention, its K, V projected from ctx
    inside this pass (nothing cached).
    """
    D, Hh, dh, Dq = cfg.D, cfg.Hh, cfg.dh, cfg.Dq
    dt = vw["w_in"].dtype
    Nv, H = video_tok.shape[0], a.shape[0]
    Xv = video_tok @ vw["w_in"].T + torch.stack(
        [time_embedding(float(s), D, dt) for s in video_sigma])
    Xa = embed(a, aw["w_in"], t, cfg.Dact)
    block = torch.tensor(cfg.frame_block, dtype=torch.int64)
    valid = torch.as_tensor(frame_valid, dtype=torch.int64)
    vv = video_visible(video_frames, video_frames, block, valid)
    full = torch.zeros((Nv + H, Nv + H), dtype=torch.bool)
    full[:Nv, :Nv] = vv
    full[Nv:, :Nv] = valid[video_frames].bool().unsqueeze(0)
    full[Nv:, Nv:] = True
    kv = []
    for lv, la in zip(vw["layers"], aw["layers"]):
        Yv, Ya = rmsnorm(Xv, lv["g1"]), rmsnorm(Xa, la["g1"])
        qv, qa = Yv @ lv["wqkv"].T, Ya @ la["wqkv"].T
        Q = torch.cat([qv[:, :Dq], qa[:, :Dq]]).reshape(-1, Hh, dh)
        K = torch.cat([qv[:, Dq:2 * Dq], qa[:, Dq:2 * Dq]]).reshape(-1, Hh, dh)
        V = torch.cat([qv[:, 2 * Dq:], qa[:, 2 * Dq:]]).reshape(-1, Hh, dh)
        pos = token_positions(cfg, 0, Nv + H)   # the joint sequence's own order
        if pos is not None:
            Q, K = rope(Q, pos), rope(K, pos)
        kv.append((K[:Nv], V[:Nv]))
        O = attention(Q, K, V, lambda q0, q1: full[q0:q1]).reshape(-1, Dq)
        Xv = Xv + O[:Nv] @ lv["wo"].T
        Xa = Xa + O[Nv:] @ la["wo"].T
        if ctx is not None:
            for lw, rows in ((lv, "v"), (la, "a")):
                Xr = Xv if rows == "v" else Xa
                kvc = ctx @ lw["wkvx"].T
                Kc = kvc[:, :Dq].reshape(-1, Hh, dh)
                Vc = kvc[:, Dq:].reshape(-1, Hh, dh)
                Qx = (rmsnorm(Xr, lw["gx"]) @ lw["wqx"].T).reshape(-1, Hh, dh)
                Xr = Xr + attention(Qx, Kc, Vc).reshape(-1, Dq) @ lw["wox"].T
                if rows == "v":
                    Xv = Xr
                else:
                    Xa = Xr
        Xv = Xv + gelu(rmsnorm(Xv, lv["g2"]) @ lv["w1"].T) @ lv["w2"].T
        Xa = Xa + gelu(rmsnorm(Xa, la["g2"]) @ la["w1"].T) @ la["w2"].T
    if video_head:
        return head(Xa, aw["g_out"], aw["w_out"]), kv, head(Xv, vw["g_out"], vw["w_out"])
    return head(Xa, aw["g_out"], aw["w_out"]), kv


def imagine_recompute(cfg, vw: dict, hist_b, valid_b, eps_v_b, cond=None):
    """Imagine without a history cache: at every video step the whole
    [history ; future] sequence runs through the layers (history at sigma=0).
    Returns z after V steps.  Equal to ``video_prefill``'s z because history
    rows never see future columns (block causality)."""
    dt = vw["w_in"].dtype
    P, Fh, Ff, D, Hh = cfg.P, cfg.Fh, cfg.Ff, cfg.D, cfg.Hh
    hist_frames = [f for f in range(Fh) if valid_b[f]]
    frames = torch.tensor(hist_frames + [Fh + j for j in range(Ff)]).repeat_interleave(P)
    block = torch.tensor(cfg.frame_block, dtype=torch.int64)
    valid = torch.tensor(list(valid_b) + [1] * Ff, dtype=torch.int64)
    nh = len(hist_frames) * P
    hist_tok = torch.from_numpy(np.ascontiguousarray(hist_b[hist_frames])).to(dt).reshape(-1, cfg.Cv)
    sig = schedule(cfg.V, cfg.sigma_star, cfg.shift)
    mask = lambda q0, q1: video_visible(frames[q0:q1], frames, block, valid)

    def vel(zc, k, s):
        X = torch.cat([embed(hist_tok, vw["w_in"], 0.0, D), embed(zc, vw["w_in"], s, D)])
        for l, lw in enumerate(vw["layers"]):
            X, _, _ = layer(X, lw, Hh, None, mask, cond=_cl(cond, l))
        return head(X[nh:], vw["g_out"], vw["w_out"])

    z0 = torch.from_numpy(np.ascontiguousarray(eps_v_b)).to(dt).reshape(-1, cfg.Cv)
    z, _ = integrate(z0, sig, vel)
    return z
