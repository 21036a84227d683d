"""Workload registry for KV-cached action denoising.

Five synthetic workloads span the three systems the pages describe:

* ``C0`` tiny fp32 IDM case: one history frame, one future frame, V=4 video
  steps to sigma*=0.9, N=4 action steps.
* ``C1`` Fast-WAM-shaped: a 9-frame one-shot video pass (Faster-WAM's anchor
  plus 8 future slots at video flow time 1, "Faster-WAM" page, section 3.1),
  30 paired layers, dense interaction, 10 action steps ("Fast-WAM" page,
  section 7: ten denoising steps over a 32-step chunk).
* ``C2`` Faster-WAM SparseMoT: the C1 shape with every 4th action layer
  reading one interval-fused K/V pair ("Faster-WAM" page, sections 3.2-3.3).
* ``C3`` Long-WAM IDM: 24 history frames + 2 future frames of 880 tokens,
  4 video steps to sigma*=0.9, 4 action steps ("Long-WAM ... Summary" page,
  section 3.2 and section 6.2, V4/A4).
* ``C4`` long-context stress: 48 history frames (the earliest 19 zero-padded
  and masked), 10 action steps, 4 independent episodes.
* ``C5`` Long-WAM co-denoising (CoD): the C3 shape with the two future frames
  and the action chunk denoised together, 4 joint steps (V4/A4), the video to
  flow time 0 ("Long-WAM ... Summary" page, section 3.2 and appendix F).
* ``C6`` C1's chunk at the experts' own widths (see below).

Options (``get(name, ...)``): ``kv_fp8`` (E4M3 cache read by the action
layers), ``rope`` (rotary positions), ``qk_std=0.06`` (the sharp variant) and
the text/state condition ``Tc``/``Ct``/``S``: ``Tc - 1`` text tokens of width
``Ct`` (standing in for the text encoder's output) and one proprio token that a
linear layer makes from the ``S`` robot-state numbers, read by every layer of
both experts through cross-attention ("Fast-WAM 精读" section 四.5 and
section 五, step 3); ``CONDITION`` holds the setting used with C6.

This module holds shapes and tables only; no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class WamConfig:
    name: str
    dtype: str            # "f32" or "bf16": storage/compute type of the GPU path
    L: int                # layers per expert (video layer i pairs with action layer i)
    D: int                # hidden width of both experts
    Hh: int               # attention heads
    dh: int               # head dim
    Fm: int               # MLP inner width
    Cv: int               # channels per video latent token
    A: int                # action dims per action token
    H: int                # action tokens per chunk
    B: int                # independent episodes
    P: int                # tokens per latent frame
    Fh: int               # history (or anchor) frames
    Ff: int               # future frames
    frame_block: Tuple[int, ...]   # temporal block id per frame (Fh + Ff), non-decreasing
    pad_frames: int       # earliest history frames that are zero padding (masked)
    V: int                # video steps (0: one-shot future at sigma=1)
    sigma_star: float     # video stop level
    N: int                # action Euler steps
    shift: float          # time-shift of the schedules (1.0 = identity)
    read_map: Tuple[int, ...]      # per action layer: -1 (action-only) or KV layer read
    fuse: Optional[Tuple[Tuple[int, int], ...]] = None  # (start, count) per fused pair
    seed: int = 0
    qk_std: float = 0.02  # std of the Wq/Wk rows (0.06 gives the "sharp" variant)
    w_std: float = 0.02   # std of every other matrix
    joint: bool = False   # co-denoising: video and actions take the N steps together
    video_end: float = 0.0  # co-denoising: flow time the video reaches after N steps
    kv_fp8: bool = False  # the action layers read an E4M3 copy of their K/V (not the pages' bf16)
    Da: int = 0           # action expert width (0: D); the attention interface is Hh x dh for both
    Fma: int = 0          # action expert MLP width (0: Fm)
    rope: bool = False    # rotary position embedding on Q and K of both experts (an option)
    Tc: int = 0           # condition tokens per episode: Tc - 1 text tokens + 1 proprio token (0: none)
    Ct: int = 0           # width of a condition token (the text encoder's output width)
    S: int = 0            # proprio (robot state) dims (0: A)

    @property
    def F(self) -> int:
        return self.Fh + self.Ff

    @property
    def Dq(self) -> int:
        """Attention interface width Hh * dh, shared by both experts."""
        return self.Hh * self.dh

    @property
    def Dact(self) -> int:
        """Hidden width of the action expert."""
        return self.Da or self.D

    @property
    def Fact(self) -> int:
        """MLP width of the action expert."""
        return self.Fma or self.Fm

    @property
    def Sdim(self) -> int:
        """Robot state dims the proprio encoder reads."""
        return self.S or self.A

    @property
    def n_valid_hist(self) -> int:
        return self.Fh - self.pad_frames

    @property
    def tokens_valid(self) -> int:
        """Valid cache tokens per layer per episode."""
        return (self.n_valid_hist + self.Ff) * self.P

    @property
    def n_kv(self) -> int:
        """Number of K/V layers the action expert reads from (fused or not)."""
        return len(self.fuse) if self.fuse else self.L


def _dense(L: int) -> Tuple[int, ...]:
    return tuple(range(L))


def sparse_mot_tables(L: int, stride: int):
    """SparseMoT interaction set and the depth interval fused into each member.

    The interval partition is [stride*m, min(stride*m + stride, L)); the
    interaction layer j_m is the last layer of its interval, so that each
    interaction layer reads the interval that precedes it in depth
    ("Faster-WAM" page, sections 3.2-3.3).  Returns (read_map, fuse).
    """
    fuse = []
    read_map = [-1] * L
    m = 0
    for s in range(0, L, stride):
        cnt = min(stride, L - s)
        fuse.append((s, cnt))
        read_map[s + cnt - 1] = m
        m += 1
    return tuple(read_map), tuple(fuse)


_C2_READ, _C2_FUSE = sparse_mot_tables(30, 4)

CONFIGS = {
    "C0": WamConfig(
        name="C0", dtype="f32", L=1, D=128, Hh=2, dh=64, Fm=512, Cv=64, A=8, H=32,
        B=1, P=128, Fh=1, Ff=1, frame_block=(0, 1), pad_frames=0, V=4,
        sigma_star=0.9, N=4, shift=1.0, read_map=(0,), seed=1000),
    "C1": WamConfig(
        name="C1", dtype="bf16", L=30, D=1024, Hh=16, dh=64, Fm=4096, Cv=64, A=14,
        H=32, B=1, P=1024, Fh=1, Ff=8, frame_block=(0,) + (1,) * 8, pad_frames=0,
        V=0, sigma_star=0.9, N=10, shift=1.0, read_map=_dense(30), seed=1001),
    "C2": WamConfig(
        name="C2", dtype="bf16", L=30, D=1024, Hh=16, dh=64, Fm=4096, Cv=64, A=14,
        H=32, B=1, P=1024, Fh=1, Ff=8, frame_block=(0,) + (1,) * 8, pad_frames=0,
        V=0, sigma_star=0.9, N=10, shift=1.0, read_map=_C2_READ, fuse=_C2_FUSE,
        seed=1002),
    "C3": WamConfig(
        name="C3", dtype="bf16", L=30, D=1024, Hh=16, dh=64, Fm=4096, Cv=64, A=14,
        H=32, B=1, P=880, Fh=24, Ff=2, frame_block=tuple(range(26)), pad_frames=0,
        V=4, sigma_star=0.9, N=4, shift=1.0, read_map=_dense(30), seed=1003),
    "C4": WamConfig(
        name="C4", dtype="bf16", L=30, D=1024, Hh=16, dh=64, Fm=4096, Cv=64, A=14,
        H=32, B=4, P=880, Fh=48, Ff=2, frame_block=tuple(range(50)), pad_frames=19,
        V=4, sigma_star=0.9, N=10, shift=1.0, read_map=_dense(30), seed=1004),
    "C5": WamConfig(
        name="C5", dtype="bf16", L=30, D=1024, Hh=16, dh=64, Fm=4096, Cv=64, A=14,
        H=32, B=1, P=880, Fh=24, Ff=2, frame_block=tuple(range(26)), pad_frames=0,
        V=4, sigma_star=0.9, N=4, shift=1.0, read_map=_dense(30), seed=1005,
        joint=True, video_end=0.0),
    # C1's chunk at the experts' own widths: video expert 3072 wide with
    # 24 x 128 heads (MLP 4 x 3072: the width is not given, the usual ratio is
    # taken), action expert 1024 wide (MLP 4096) over the same 24 x 128
    # attention interface
    "C6": WamConfig(
        name="C6", dtype="bf16", L=30, D=3072, Hh=24, dh=128, Fm=12288, Cv=64, A=14,
        H=32, B=1, P=1024, Fh=1, Ff=8, frame_block=(0,) + (1,) * 8, pad_frames=0,
        V=0, sigma_star=0.9, N=10, shift=1.0, read_map=_dense(30), seed=1006,
        Da=1024, Fma=4096),
}


# 100 text tokens of the text encoder's width 4096 plus one proprio token made
# from 14 state numbers (RoboTwin's actions and states are both 14-dim,
# "Fast-WAM 精读" section 四.3)
CONDITION = dict(Tc=101, Ct=4096, S=14)


def get(name: str, **overrides) -> WamConfig:
    """Look up a workload, optionally overriding fields (diagnostic variants)."""
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def small(name: str = "S", **kw) -> WamConfig:
    """A small bf16-or-f32 workload for unit and parity tests: several tiles
    along every axis plus ragged tails (P not a multiple of 64)."""
    base = dict(
        name=name, dtype="bf16", L=2, D=256, Hh=4, dh=64, Fm=512, Cv=64, A=14, H=32,
        B=1, P=100, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4), pad_frames=1, V=2,
        sigma_star=0.9, N=3, shift=1.0, read_map=(0, 1), seed=7)
    base.update(kw)
    return WamConfig(**base)
