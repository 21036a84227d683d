"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types an oracle formula: each compares against a
closed form, a library routine, a special case, an identity that a mistake
(dropped term, wrong sign or index, transposed operand) would break, or brute
force on tiny inputs.
"""
import math
import struct

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from kv_cached_flow_amd import configs, inputs
from oracle import wam_oracle as O

f64 = torch.float64


def bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


# ---------------------------------------------------------------- schedules
@pytest.mark.parametrize("V", [1, 2, 4, 7])
def test_video_schedule_endpoints(V):
    # Long-WAM close-reading section 04: start is pure noise, end exactly sigma*=0.9
    s = O.schedule(V, 0.9)
    assert s.dtype == np.float32 and len(s) == V + 1
    assert bits(s[0]) == bits(1.0)
    assert bits(s[-1]) == 0x3F666666
    assert np.all(np.diff(s.astype(np.float64)) < 0)


def test_video_schedule_v4_values():
    s = O.schedule(4, 0.9)
    want = np.array([1.0, 0.975, 0.95, 0.925, 0.9], dtype=np.float32)
    assert np.array_equal(s.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("N", [1, 2, 4, 10])
@pytest.mark.parametrize("shift", [1.0, 3.0, 0.5])
def test_action_schedule(N, shift):
    t = O.schedule(N, 0.0, shift)
    assert t[0] == 1.0 and t[-1] == 0.0
    assert np.all(np.diff(t.astype(np.float64)) < 0)
    if shift == 1.0:
        assert np.allclose(t, np.linspace(1, 0, N + 1), atol=1e-7)


def test_shift_map_closed_form():
    # shift s maps u=1/2 to s/(1+s): a textbook value of the shift map
    for s in (0.5, 2.0, 3.0, 5.0):
        assert abs(O.phi(0.5, s) - s / (1 + s)) < 1e-15


# ---------------------------------------------------------------- flow / Euler
def _sched(n, seed):
    r = np.random.default_rng(seed)
    x = np.sort(r.uniform(0, 1, n - 1))[::-1]
    return np.concatenate([[1.0], x, [0.0]])


@pytest.mark.parametrize("seed", range(5))
def test_euler_exact_velocity_lands_on_data(seed):
    # The path is linear in sigma, so Euler with the exact velocity eps - x0 is
    # exact at every node: x_k = (1 - t_k) x0 + t_k eps for ANY schedule.
    r = np.random.default_rng(100 + seed)
    x0 = torch.tensor(r.standard_normal((32, 14)), dtype=f64)
    eps = torch.tensor(r.standard_normal((32, 14)), dtype=f64)
    ts = _sched(2 + seed * 3, seed)
    states = []

    def vel(x, k, s):
        states.append((x.clone(), ts[k]))
        return eps - x0

    xN, vs = O.integrate(eps, ts, vel)
    assert torch.max(torch.abs(xN - x0)) < 1e-13
    for x, t in states:
        assert torch.max(torch.abs(x - ((1 - t) * x0 + t * eps))) < 1e-13
    assert len(vs) == len(ts) - 1


def test_euler_constant_velocity():
    # x_N = x_0 + (t_N - t_0) v = eps - v for the action schedule 1 -> 0
    r = np.random.default_rng(3)
    eps = torch.tensor(r.standard_normal((8, 3)), dtype=f64)
    v = torch.tensor(r.standard_normal((8, 3)), dtype=f64)
    xN, _ = O.integrate(eps, O.schedule(10, 0.0), lambda x, k, s: v)
    assert torch.max(torch.abs(xN - (eps - v))) < 1e-13


def test_flow_velocity_is_path_derivative():
    r = np.random.default_rng(4)
    x0 = torch.tensor(r.standard_normal(50), dtype=f64)
    eps = torch.tensor(r.standard_normal(50), dtype=f64)
    s, h = 0.37, 1e-6
    fd = (O.flow_point(x0, eps, s + h) - O.flow_point(x0, eps, s - h)) / (2 * h)
    assert torch.max(torch.abs(fd - O.flow_velocity(x0, eps))) < 1e-8
    assert torch.equal(O.flow_point(x0, eps, 0.0), x0)
    assert torch.equal(O.flow_point(x0, eps, 1.0), eps)


# ---------------------------------------------------------------- layer pieces
def test_time_embedding_structure():
    D = 64
    e0 = O.time_embedding(0.0, D)
    assert torch.equal(e0, torch.cat([torch.ones(32, dtype=f64), torch.zeros(32, dtype=f64)]))
    e = O.time_embedding(0.731, D)
    # each frequency is a point on the unit circle; lowest frequency is 1 rad per unit t
    assert torch.max(torch.abs(e[:32] ** 2 + e[32:] ** 2 - 1)) < 1e-14
    assert abs(e[0].item() - math.cos(731.0)) < 1e-12
    assert abs(e[32].item() - math.sin(731.0)) < 1e-12
    # frequencies decrease geometrically by 10000^(1/32) per index
    tt = 1000 * 0.731
    w1 = math.atan2(e[33].item(), e[1].item())
    assert abs(math.remainder(w1 - tt * 10000 ** (-1 / 32), 2 * math.pi)) < 1e-9


def test_rmsnorm_vs_library():
    r = np.random.default_rng(5)
    x = torch.tensor(r.standard_normal((7, 96)), dtype=f64)
    g = torch.tensor(1 + 0.1 * r.standard_normal(96), dtype=f64)
    ref = F.rms_norm(x, (96,), g, eps=1e-6)
    assert torch.max(torch.abs(O.rmsnorm(x, g) - ref)) < 1e-14
    y = O.rmsnorm(x, torch.ones(96, dtype=f64))
    assert torch.max(torch.abs((y * y).mean(-1) - 1)) < 1e-5


def test_head_vs_library():
    # the velocity head: the expert's final RMSNorm with its own gain, then the
    # output projection [C][D] (non-square, so a transposed W fails), on rows
    # whose RMS is far from 1 (so a dropped RMSNorm fails)
    r = np.random.default_rng(6)
    X = torch.tensor(r.standard_normal((7, 96)) * 5.0, dtype=f64)
    g = torch.tensor(1 + 0.3 * r.standard_normal(96), dtype=f64)
    W = torch.tensor(r.standard_normal((5, 96)), dtype=f64)
    got = O.head(X, g, W)
    assert tuple(got.shape) == (7, 5)
    ref = F.linear(F.rms_norm(X, (96,), g, eps=1e-6), W)
    assert torch.max(torch.abs(got - ref)) < 1e-12
    assert torch.max(torch.abs(got - F.linear(X, W))) > 1.0


def test_heads_read_their_own_expert_gain():
    # Doubling an expert's g_out doubles exactly its velocity (the head is
    # linear in the gain, and 2 is exact): a head that dropped the gain or
    # took another weight's fails.
    cfg = configs.small("HG", dtype="f32", L=1, D=128, Hh=2, Fm=256, P=16, Fh=2, Ff=1,
                        frame_block=(0, 1, 2), pad_frames=0, V=1, N=1, read_map=(0,))
    inp = inputs.generate(cfg)
    vw = O.to_torch_expert(inp["video"], f64)
    aw = O.to_torch_expert(inp["action"], f64)
    cache, z, _ = O.video_prefill(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    a = torch.tensor(inp["eps_a"][0], dtype=f64)
    v1 = O.action_velocity(cfg, aw, O.read_layers(cfg, cache, None), a, 0.7)
    aw2 = dict(aw, g_out=aw["g_out"] * 2.0)
    vw2 = dict(vw, g_out=vw["g_out"] * 2.0)
    assert torch.equal(O.action_velocity(cfg, aw2, O.read_layers(cfg, cache, None), a, 0.7), 2.0 * v1)
    # the video head: one imagine step moves z by (sigma_1 - sigma_0) v-hat
    eps = torch.tensor(inp["eps_v"][0], dtype=f64).reshape(-1, cfg.Cv)
    _, z2, _ = O.video_prefill(cfg, vw2, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    assert torch.allclose(z2 - eps, 2.0 * (z - eps), rtol=1e-12, atol=1e-14)
    assert not torch.allclose(z - eps, torch.zeros_like(z))


def test_gelu_vs_library():
    x = torch.linspace(-8, 8, 1001, dtype=f64)
    assert torch.max(torch.abs(O.gelu(x) - F.gelu(x))) < 1e-15
    assert torch.max(torch.abs(O.gelu(x) - O.gelu(-x) - x)) < 1e-14


def _qkv(r, nq, nk, Hh, dh):
    q = torch.tensor(r.standard_normal((nq, Hh, dh)), dtype=f64)
    k = torch.tensor(r.standard_normal((nk, Hh, dh)), dtype=f64)
    v = torch.tensor(r.standard_normal((nk, Hh, dh)), dtype=f64)
    return q, k, v


def _sdpa(q, k, v, mask=None):
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2), k.permute(1, 0, 2),
                                       v.permute(1, 0, 2), attn_mask=mask)
    return o.permute(1, 0, 2)


def test_attention_vs_library_unmasked_and_masked():
    r = np.random.default_rng(6)
    q, k, v = _qkv(r, 13, 29, 3, 16)
    assert torch.max(torch.abs(O.attention(q, k, v) - _sdpa(q, k, v))) < 1e-13
    m = torch.tensor(r.uniform(size=(13, 29)) < 0.6)
    m[:, 0] = True
    got = O.attention(q, k, v, lambda a, b: m[a:b], q_chunk=4)
    assert torch.max(torch.abs(got - _sdpa(q, k, v, m))) < 1e-13


def test_attention_single_key_returns_value():
    r = np.random.default_rng(7)
    q, k, v = _qkv(r, 5, 9, 2, 8)
    m = torch.zeros((5, 9), dtype=torch.bool)
    m[:, 4] = True
    got = O.attention(q, k, v, lambda a, b: m[a:b])
    assert torch.equal(got, v[4].unsqueeze(0).expand(5, -1, -1))


def test_attention_zero_query_is_mean_of_visible():
    r = np.random.default_rng(8)
    _, k, v = _qkv(r, 1, 16, 2, 8)
    q = torch.zeros((3, 2, 8), dtype=f64)
    m = torch.zeros((3, 16), dtype=torch.bool)
    m[0, :4] = True
    m[1, :8] = True
    m[2, :] = True
    got = O.attention(q, k, v, lambda a, b: m[a:b])
    for i, n in enumerate((4, 8, 16)):
        assert torch.max(torch.abs(got[i] - v[:n].mean(0))) < 1e-15


def test_attention_key_permutation_invariance():
    r = np.random.default_rng(9)
    q, k, v = _qkv(r, 6, 21, 2, 8)
    perm = torch.tensor(r.permutation(21))
    a = O.attention(q, k, v)
    b = O.attention(q, k[perm], v[perm])
    assert torch.max(torch.abs(a - b)) < 1e-14


def _rand_layer(r, D, Fm, std=0.2):
    t = lambda *s: torch.tensor(r.standard_normal(s) * std, dtype=f64)
    return {"g1": 1 + t(D), "wqkv": t(3 * D, D), "wo": t(D, D), "g2": 1 + t(D),
            "w1": t(Fm, D), "w2": t(D, Fm)}


def _library_layer(X, w, Hh, ctx, mask):
    # Same block built from torch library routines (rms_norm, linear, SDPA, gelu).
    n, D = X.shape
    dh = D // Hh
    Y = F.rms_norm(X, (D,), w["g1"], eps=1e-6)
    q, k, v = F.linear(Y, w["wqkv"]).split(D, dim=1)
    q, k, v = (t.reshape(n, Hh, dh) for t in (q, k, v))
    if ctx is not None:
        k = torch.cat([ctx[0], k])
        v = torch.cat([ctx[1], v])
    o = _sdpa(q, k, v, mask).reshape(n, D)
    X = X + F.linear(o, w["wo"])
    h = F.gelu(F.linear(F.rms_norm(X, (D,), w["g2"], eps=1e-6), w["w1"]))
    return X + F.linear(h, w["w2"])


def test_layer_vs_library_composition():
    r = np.random.default_rng(10)
    D, Hh, Fm, n, nc = 48, 3, 80, 11, 17
    w = _rand_layer(r, D, Fm)
    X = torch.tensor(r.standard_normal((n, D)), dtype=f64)
    ctx = (torch.tensor(r.standard_normal((nc, Hh, 16)), dtype=f64),
           torch.tensor(r.standard_normal((nc, Hh, 16)), dtype=f64))
    m = torch.tensor(r.uniform(size=(n, nc + n)) < 0.7)
    m[:, -1] = True
    got, K, V = O.layer(X, w, Hh, ctx, lambda a, b: m[a:b])
    ref = _library_layer(X, w, Hh, ctx, m)
    assert torch.max(torch.abs(got - ref)) < 1e-12
    _, K2, V2 = O.layer(X, w, Hh, ctx, None, kv_only=True)
    assert torch.equal(K, K2) and torch.equal(V, V2)


def test_layer_with_a_wider_attention_interface_vs_library():
    # the expert width D differs from the attention width Hh * dh (the action
    # expert: 1024 wide, 24 heads x 128): Wqkv [3 Dq][D], Wo [D][Dq]
    r = np.random.default_rng(12)
    D, Hh, dh, Fm, n, nc = 40, 3, 32, 72, 9, 13
    Dq = Hh * dh
    t = lambda *sh: torch.tensor(r.standard_normal(sh) * 0.2, dtype=f64)
    w = {"g1": 1 + t(D), "wqkv": t(3 * Dq, D), "wo": t(D, Dq), "g2": 1 + t(D), "w1": t(Fm, D),
         "w2": t(D, Fm)}
    X = torch.tensor(r.standard_normal((n, D)), dtype=f64)
    ctx = (t(nc, Hh, dh), t(nc, Hh, dh))
    got, K, V = O.layer(X, w, Hh, ctx, None)
    Y = F.rms_norm(X, (D,), w["g1"], eps=1e-6)
    q, k, v = F.linear(Y, w["wqkv"]).split(Dq, dim=1)
    q, k, v = (u.reshape(n, Hh, dh) for u in (q, k, v))
    assert torch.equal(K, k) and torch.equal(V, v)
    k = torch.cat([ctx[0], k])
    v = torch.cat([ctx[1], v])
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2), k.permute(1, 0, 2), v.permute(1, 0, 2))
    ref = X + F.linear(o.permute(1, 0, 2).reshape(n, Dq), w["wo"])
    ref = ref + F.linear(F.gelu(F.linear(F.rms_norm(ref, (D,), w["g2"], eps=1e-6), w["w1"])), w["w2"])
    assert torch.max(torch.abs(got - ref)) < 1e-12


def test_real_width_chunk_structure():
    # a chunk whose experts differ in width (video 48 = 3 heads x 16, action 20)
    # keeps the identities: joint sequence == cached path
    cfg = _tiny(D=48, Hh=3, dh=16, Da=20, Fma=36)
    inp = inputs.generate(cfg, threads=1)
    assert inp["action"]["layers"][0]["wqkv"].shape == (3 * 48, 20)
    assert inp["action"]["layers"][0]["wo"].shape == (20, 48)
    vw = O.to_torch_expert(inp["video"], f64)
    aw = O.to_torch_expert(inp["action"], f64)
    cache, z, frames = O.video_prefill(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    t0 = float(O.schedule(cfg.N, 0.0)[0])
    a = torch.tensor(inp["eps_a"][0], dtype=f64)
    v_cached = O.action_velocity(cfg, aw, O.read_layers(cfg, cache, None), a, t0)
    valid_frames = [f for f in range(cfg.Fh) if inp["hist_valid"][0][f]]
    hist_tok = torch.tensor(inp["hist"][0][valid_frames], dtype=f64).reshape(-1, cfg.Cv)
    vtok = torch.cat([hist_tok, z])
    sig_f = float(O.schedule(cfg.V, cfg.sigma_star)[-1])
    vsig = [0.0] * hist_tok.shape[0] + [sig_f] * z.shape[0]
    fvalid = list(inp["hist_valid"][0]) + [1] * cfg.Ff
    v_joint, _ = O.joint_mot_step(cfg, vw, aw, vtok, vsig, frames, fvalid, a, t0)
    assert torch.max(torch.abs(v_joint - v_cached)) < 1e-12


def test_layer_zero_output_projections_is_identity():
    r = np.random.default_rng(11)
    w = _rand_layer(r, 32, 64)
    w["wo"].zero_()
    w["w2"].zero_()
    X = torch.tensor(r.standard_normal((5, 32)), dtype=f64)
    got, _, _ = O.layer(X, w, 2)
    assert torch.equal(got, X)


# ---------------------------------------------------------------- masks
def _brute_visible(frames_q, frames_k, block, valid):
    # Rule of Long-WAM Summary 3.2 / Faster-WAM 3.1 enumerated pair by pair.
    out = np.zeros((len(frames_q), len(frames_k)), dtype=bool)
    for i, fq in enumerate(frames_q):
        for j, fk in enumerate(frames_k):
            earlier_or_same = block[fk] <= block[fq]
            out[i, j] = bool(valid[fk]) and earlier_or_same
    return out


def test_block_causal_per_frame_counts():
    # one frame per block: a query in frame f sees exactly frames 0..f
    P, Fn = 3, 6
    block = torch.arange(Fn)
    valid = torch.ones(Fn, dtype=torch.int64)
    fr = torch.arange(Fn).repeat_interleave(P)
    m = O.video_visible(fr, fr, block, valid)
    for i in range(Fn * P):
        f = i // P
        assert m[i].sum().item() == (f + 1) * P
        assert bool(m[i, : (f + 1) * P].all())


def test_anchor_future_rule():
    # Faster-WAM 3.1: anchor (block 0) never reads future slots; future slots
    # read the anchor and each other.
    P = 4
    block = torch.tensor([0] + [1] * 8)
    valid = torch.ones(9, dtype=torch.int64)
    fr = torch.arange(9).repeat_interleave(P)
    m = O.video_visible(fr, fr, block, valid)
    assert bool(m[:P, :P].all()) and not bool(m[:P, P:].any())
    assert bool(m[P:, :].all())


@pytest.mark.parametrize("seed", range(6))
def test_video_mask_brute_force_ragged(seed):
    r = np.random.default_rng(50 + seed)
    Fn = int(r.integers(2, 7))
    P = int(r.integers(1, 6))
    block = np.sort(r.integers(0, Fn, Fn))
    valid = (r.uniform(size=Fn) < 0.7).astype(np.int64)
    valid[-1] = 1
    fr = np.repeat(np.arange(Fn), P)
    got = O.video_visible(torch.tensor(fr), torch.tensor(fr), torch.tensor(block),
                          torch.tensor(valid)).numpy()
    assert np.array_equal(got, _brute_visible(fr, fr, block, valid))


# ---------------------------------------------------------------- fusion
def _layers(r, n, T=6, Hh=2, dh=4):
    return [(torch.tensor(r.standard_normal((T, Hh, dh)), dtype=torch.float32),
             torch.tensor(r.standard_normal((T, Hh, dh)), dtype=torch.float32))
            for _ in range(n)]


def test_fusion_one_hot_is_exact_layer():
    r = np.random.default_rng(12)
    cache = _layers(r, 8)
    logits = np.full((2, 4), -np.inf, dtype=np.float32)
    logits[0, 2] = 0.0
    logits[1, 1] = 3.5
    fused = O.fuse_interval(cache, ((0, 4), (4, 4)), logits)
    assert torch.equal(fused[0][0], cache[2][0]) and torch.equal(fused[0][1], cache[2][1])
    assert torch.equal(fused[1][0], cache[5][0]) and torch.equal(fused[1][1], cache[5][1])


def test_fusion_identical_layers_and_weights():
    r = np.random.default_rng(13)
    one = _layers(r, 1)[0]
    cache = [(one[0].double(), one[1].double())] * 4
    logits = r.standard_normal((1, 4)).astype(np.float32)
    fused = O.fuse_interval(cache, ((0, 4),), logits)
    assert torch.max(torch.abs(fused[0][0] - cache[0][0])) < 1e-14
    w = O.fusion_weights(logits[0], 4)
    assert abs(w.sum() - 1) < 1e-15 and np.all(w > 0)
    # softmax is invariant to a common logit offset and ordered like the logits
    w2 = O.fusion_weights(logits[0].astype(np.float64) + 7.0, 4)
    assert np.max(np.abs(w - w2)) < 1e-14
    assert np.array_equal(np.argsort(w), np.argsort(logits[0]))


def test_sparse_mot_tables_partition():
    read_map, fuse = configs.sparse_mot_tables(30, 4)
    assert [j for j, m in enumerate(read_map) if m >= 0] == [3, 7, 11, 15, 19, 23, 27, 29]
    covered = [s + i for s, c in fuse for i in range(c)]
    assert covered == list(range(30)) and len(fuse) == 8


# ---------------------------------------------------------------- structural
def _tiny(**kw):
    base = dict(dtype="f32", L=2, D=32, Hh=2, dh=16, Fm=48, Cv=6, A=3, H=5, B=1,
                P=3, Fh=3, Ff=2, frame_block=(0, 1, 2, 3, 4), pad_frames=1, V=2,
                N=2, w_std=0.2, qk_std=0.2, read_map=(0, 1), seed=21)
    base.update(kw)
    return configs.small("T", **base)


@pytest.mark.parametrize("rope", [False, True])
def test_joint_sequence_equals_cached_path(rope):
    # Asymmetric mask => caching is exact: one joint [video ; action] pass with
    # the explicit mask reproduces the cache rows and the first action v-hat.
    # With the rotary option the joint pass takes positions from its own
    # sequence order, the cached path from the history, future and action
    # offsets it computes separately.
    cfg = _tiny(rope=rope)
    inp = inputs.generate(cfg, threads=1)
    vw = O.to_torch_expert(inp["video"], f64)
    aw = O.to_torch_expert(inp["action"], f64)
    cache, z, frames = O.video_prefill(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    t0 = float(O.schedule(cfg.N, 0.0)[0])
    a = torch.tensor(inp["eps_a"][0], dtype=f64)
    v_cached = O.action_velocity(cfg, aw, O.read_layers(cfg, cache, None), a, t0,
                                 int(cache[0][0].shape[0]))

    valid_frames = [f for f in range(cfg.Fh) if inp["hist_valid"][0][f]]
    hist_tok = torch.tensor(inp["hist"][0][valid_frames], dtype=f64).reshape(-1, cfg.Cv)
    vtok = torch.cat([hist_tok, z])
    sig_f = float(O.schedule(cfg.V, cfg.sigma_star)[-1])
    vsig = [0.0] * hist_tok.shape[0] + [sig_f] * z.shape[0]
    fvalid = list(inp["hist_valid"][0]) + [1] * cfg.Ff
    v_joint, kv = O.joint_mot_step(cfg, vw, aw, vtok, vsig, frames, fvalid, a, t0)
    assert torch.max(torch.abs(v_joint - v_cached)) < 1e-12
    for (Kc, Vc), (Kj, Vj) in zip(cache, kv):
        assert torch.max(torch.abs(Kc - Kj)) < 1e-12
        assert torch.max(torch.abs(Vc - Vj)) < 1e-12


def test_cached_history_equals_recompute():
    cfg = _tiny()
    inp = inputs.generate(cfg, threads=1)
    vw = O.to_torch_expert(inp["video"], f64)
    _, z, _ = O.video_prefill(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    z2 = O.imagine_recompute(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    assert torch.max(torch.abs(z - z2)) < 1e-12
    # and the imagined latents did move away from the noise
    assert torch.max(torch.abs(z - torch.tensor(inp["eps_v"][0], dtype=f64).reshape(z.shape))) > 1e-3


def test_padding_invariance_and_dropping():
    cfg = _tiny()
    inp = inputs.generate(cfg, threads=1)
    ref = O.run_chunk(cfg, inp, drop_padded=True)
    kept = O.run_chunk(cfg, inp, drop_padded=False)
    assert np.max(np.abs(ref["actions"] - kept["actions"])) < 1e-12
    inp2 = dict(inp)
    inp2["hist"] = inp["hist"].copy()
    inp2["hist"][0, 0] = 123.0   # contents of the padded frame
    kept2 = O.run_chunk(cfg, inp2, drop_padded=False)
    assert np.array_equal(kept["actions"], kept2["actions"])
    # a valid frame does matter
    inp3 = dict(inp)
    inp3["hist"] = inp["hist"].copy()
    inp3["hist"][0, 1] += 1.0
    assert np.max(np.abs(O.run_chunk(cfg, inp3)["actions"] - ref["actions"])) > 1e-6


def test_batch_independence():
    cfg2 = _tiny(B=2)
    inp2 = inputs.generate(cfg2, threads=1)
    both = O.run_chunk(cfg2, inp2)
    for b in range(2):
        one = {k: (v[b:b + 1] if k in ("hist", "hist_valid", "eps_v", "eps_a") else v)
               for k, v in inp2.items()}
        single = O.run_chunk(_tiny(B=1), one)
        assert np.array_equal(both["actions"][b], single["actions"][0])


def test_sparse_one_hot_stride_one_equals_dense():
    # Stride-1 SparseMoT with one-hot weights on the own layer == dense MoT.
    dense = _tiny(V=0)
    sparse = _tiny(V=0, fuse=((0, 1), (1, 1)))
    inp = inputs.generate(dense, threads=1)
    inp_s = dict(inp)
    inp_s["fuse_logits"] = np.zeros((2, 1), dtype=np.float32)
    a = O.run_chunk(dense, inp)["actions"]
    b = O.run_chunk(sparse, inp_s)["actions"]
    assert np.array_equal(a, b)


def test_action_only_layers_ignore_video():
    # A layer with read_map = -1 must not depend on the cache at all.
    cfg = _tiny(read_map=(-1, -1))
    inp = inputs.generate(cfg, threads=1)
    a1 = O.run_chunk(cfg, inp)["actions"]
    inp2 = dict(inp)
    inp2["hist"] = inp["hist"] * 3.0
    inp2["eps_v"] = inp["eps_v"] * -1.0
    assert np.array_equal(a1, O.run_chunk(cfg, inp2)["actions"])


# ---------------------------------------------------------------- co-denoising
def test_codenoise_video_trajectory_equals_imagine():
    # Video rows never read actions, so CoD's video latents follow exactly the
    # IDM imagine trajectory on the same schedule (here: 2 steps to 0.9).
    cfg = _tiny(V=2, N=2)
    inp = inputs.generate(cfg, threads=1)
    vw = O.to_torch_expert(inp["video"], f64)
    aw = O.to_torch_expert(inp["action"], f64)
    _, z_idm, _ = O.video_prefill(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0])
    _, z_cod, traj, _ = O.codenoise(cfg, vw, aw, inp["hist"][0], inp["hist_valid"][0],
                                    inp["eps_v"][0], inp["eps_a"][0], 2, 0.9)
    assert torch.max(torch.abs(z_cod - z_idm)) < 1e-12
    assert len(traj) == 2


def test_codenoise_one_step_equals_faster_wam():
    # One joint step reads the future at video level 1 (pure noise): the
    # Faster-WAM path (V = 0, future cached at sigma = 1) with N = 1.
    cfg = _tiny(V=0, N=1)
    inp = inputs.generate(cfg, threads=1)
    ref = O.run_chunk(cfg, inp)["actions"]
    cod = O.run_codenoise(cfg, inp, steps=1)["actions"]
    assert np.max(np.abs(cod - ref)) < 1e-12
    # with two steps the second action step sees a moved future
    cfg2 = _tiny(V=0, N=2)
    two_idm = O.run_chunk(cfg2, inp)["actions"]
    two_cod = O.run_codenoise(cfg2, inp, steps=2)["actions"]
    assert np.max(np.abs(two_cod - two_idm)) > 1e-6


@pytest.mark.parametrize("end", [0.0, 0.5])
def test_codenoise_steps_equal_joint_sequence(end):
    # Every CoD step equals one uncached joint pass over [history ; future at
    # the step's video level ; actions at the step's action level]: both
    # velocities, at every step (a stale or wrong-level future would differ).
    # With end = 0.5 a text/state condition rides along: the cached condition
    # K, V of both experts equal the joint pass's own projections.
    cfg = _tiny(N=3, **(dict(Tc=4, Ct=10, S=3) if end else {}))
    inp = inputs.generate(cfg, threads=1)
    vw = O.to_torch_expert(inp["video"], f64)
    aw = O.to_torch_expert(inp["action"], f64)
    ctx = O.episode_condition(cfg, inp, 0, f64)
    a_fin, z_fin, traj, cache = O.codenoise(cfg, vw, aw, inp["hist"][0], inp["hist_valid"][0],
                                            inp["eps_v"][0], inp["eps_a"][0], 3, end,
                                            O.condition_cache(cfg, vw, ctx),
                                            O.condition_cache(cfg, aw, ctx))
    sv = O.schedule(3, end)
    ta = O.schedule(3, 0.0)
    valid_frames = [f for f in range(cfg.Fh) if inp["hist_valid"][0][f]]
    hist_tok = torch.tensor(inp["hist"][0][valid_frames], dtype=f64).reshape(-1, cfg.Cv)
    nh = hist_tok.shape[0]
    frames = torch.tensor(valid_frames + [cfg.Fh + j for j in range(cfg.Ff)]).repeat_interleave(cfg.P)
    fvalid = list(inp["hist_valid"][0]) + [1] * cfg.Ff
    for k, (z_k, a_k, vv_k, va_k) in enumerate(traj):
        vtok = torch.cat([hist_tok, z_k])
        vsig = [0.0] * nh + [float(sv[k])] * z_k.shape[0]
        va, kv, vv = O.joint_mot_step(cfg, vw, aw, vtok, vsig, frames, fvalid, a_k, float(ta[k]),
                                      video_head=True, ctx=ctx)
        assert torch.max(torch.abs(va - va_k)) < 1e-12
        assert torch.max(torch.abs(vv[nh:] - vv_k)) < 1e-12
        if k == len(traj) - 1:
            for (Kc, Vc), (Kj, Vj) in zip(cache, kv):
                assert torch.max(torch.abs(Kc - Kj)) < 1e-12
                assert torch.max(torch.abs(Vc - Vj)) < 1e-12
    # the trajectories end where the schedules say: a_N from the last step
    z_last, a_last, vv_last, va_last = traj[-1]
    assert torch.max(torch.abs(a_fin - (a_last + float(ta[3] - ta[2]) * va_last))) < 1e-12
    assert torch.max(torch.abs(z_fin - (z_last + float(sv[3] - sv[2]) * vv_last))) < 1e-12


# ---------------------------------------------------------------- FP8 (E4M3) cache option
def test_e4m3_codes_closed_form():
    v = O.e4m3_value
    assert v(0x00) == 0.0 and v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6 and v(0x38) == 1.0 and v(0x39) == 1.125
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0 and v(0xB8) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    pos = O._E4M3_POS
    assert len(pos) == 127 and np.all(np.diff(pos) > 0)
    assert sum(not math.isnan(v(c)) for c in range(256)) == 254


def test_e4m3_encode_round_trip_and_ties():
    finite = [c for c in range(256) if not math.isnan(O.e4m3_value(c))]
    vals = np.array([O.e4m3_value(c) if c != 0x80 else -0.0 for c in finite])
    assert np.array_equal(O.e4m3_encode(vals), np.array(finite, dtype=np.uint8))
    pos = O._E4M3_POS
    for i in range(len(pos) - 1):
        mid = 0.5 * (pos[i] + pos[i + 1])
        want = i if i % 2 == 0 else i + 1          # ties go to the even code
        assert O.e4m3_encode([mid])[0] == want
        assert O.e4m3_encode([-mid])[0] == want | 0x80
        assert O.e4m3_encode([np.nextafter(mid, 0)])[0] == i
        assert O.e4m3_encode([np.nextafter(mid, 1e9)])[0] == i + 1
    with pytest.raises(ValueError):
        O.e4m3_encode([448.5])


@pytest.mark.parametrize("seed", [0, 1])
def test_e4m3_encode_is_nearest_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.uniform(-448, 448, 2000), rng.normal(0, 0.01, 2000)])
    got = O.e4m3_decode(O.e4m3_encode(x))
    table = O._E4M3_POS
    best = np.min(np.abs(np.abs(x)[:, None] - table[None, :]), axis=1)
    assert np.array_equal(np.abs(np.abs(got) - np.abs(x)), best)
    assert np.all((got == 0) | (np.sign(got) == np.sign(x)))


def test_kv_tile_exponent_boundaries():
    for e in (-12, -3, 0, 4):
        edge = 448.0 * 2.0 ** e
        assert O.kv_tile_exponent(edge) == e
        assert O.kv_tile_exponent(np.nextafter(edge, 1e30)) == e + 1
        assert O.kv_tile_exponent(np.nextafter(edge, 0)) == e
    assert O.kv_tile_exponent(0.0) == 0
    # the scale stays a normal float32 number: e >= -126, and codes still fit
    # (|x| 2^126 <= 448 whenever the unclamped e would be below -126)
    for a in (1e-37, 448.0 * 2.0 ** -127, 448.0 * 2.0 ** -126, 2.0 ** -130):
        e = O.kv_tile_exponent(a)
        assert e == -126 and a * 2.0 ** 126 <= 448.0
    assert O.kv_tile_exponent(np.nextafter(448.0 * 2.0 ** -126, 1.0)) == -125
    rng = np.random.default_rng(5)
    for a in rng.lognormal(0, 4, 200):
        e = O.kv_tile_exponent(a)
        assert 448.0 * 2.0 ** (e - 1) < a <= 448.0 * 2.0 ** e


def test_quantize_kv_error_bound_and_ragged_tiles():
    rng = np.random.default_rng(9)
    T, Hh, dh = 150, 3, 64                     # two full tiles and a ragged one
    K = torch.tensor(rng.normal(0, 1, (T, Hh, dh)), dtype=f64)
    V = torch.tensor(rng.normal(0, 1, (T, Hh, dh)), dtype=f64)
    V[128:, 1] *= 1e-3                          # a tile of its own scale
    Kq, Vq, (ck, ek, cv, ev) = O.quantize_kv_fp8(K, V)
    assert ek.shape == (Hh, 3) and ev.shape == (Hh, 3)
    for X, Xq, ex in ((K, Kq, ek), (V, Vq, ev)):
        for h in range(Hh):
            for t in range(3):
                blk, q = X[64 * t:64 * t + 64, h].numpy(), Xq[64 * t:64 * t + 64, h].numpy()
                s = 2.0 ** ex[h, t]
                assert np.max(np.abs(blk)) <= 448 * s and np.max(np.abs(blk)) > 224 * s
                # half a step of 3 mantissa bits, or half the subnormal step
                bound = np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * s)
                assert np.all(np.abs(q - blk) <= bound)
    assert ev[1, 2] < ev[1, 1] - 5                # the small tile got its own scale
    # values already on the grid come back exactly
    Kg = torch.tensor(O.e4m3_decode(ck.astype(np.int64)) * 2.0 ** np.repeat(ek.T, 64, axis=0)[:T, :, None])
    Kg2, _, _ = O.quantize_kv_fp8(Kg, V)
    assert torch.equal(Kg2, Kg)


def test_fp8_option_touches_only_what_the_action_layers_read():
    cfg = _tiny()
    inp = inputs.generate(cfg, threads=1)
    a = O.run_chunk(cfg, inp)
    b = O.run_chunk(cfg, inp, kv_fp8=True)
    assert np.array_equal(a["z"], b["z"])
    d = np.linalg.norm(b["actions"] - a["actions"]) / np.linalg.norm(a["actions"])
    assert 0 < d < 0.1


# ---------------------------------------------------------------- streaming history
def _extended_and_full(blocks, pad, n_old, rope=False):
    cfg = _tiny(Fh=5, Ff=2, frame_block=blocks, pad_frames=pad, rope=rope)
    inp = inputs.generate(cfg, threads=1)
    vw = O.to_torch_expert(inp["video"], f64)
    hist, valid = inp["hist"][0], inp["hist_valid"][0]
    full, _, _, _ = O.history_cache(cfg, vw, hist, valid)
    # the first n_old frames alone (later frames marked invalid cannot be seen)
    valid_old = np.array([v if f < n_old else 0 for f, v in enumerate(valid)])
    if valid_old.any():
        part, _, _, _ = O.history_cache(cfg, vw, hist, valid_old)
    else:
        part = [(torch.zeros((0, cfg.Hh, cfg.dh), dtype=f64),) * 2 for _ in range(cfg.L)]
    return full, O.extend_history(cfg, vw, part, n_old, hist, valid)


@pytest.mark.parametrize("blocks,pad,n_old", [
    ((0, 1, 2, 3, 4, 5, 6), 1, 3),        # one frame per block, a padded first frame
    ((0, 0, 1, 1, 2, 3, 4), 0, 2),        # blocks of two frames, the split at a block boundary
    ((0, 1, 2, 3, 4, 5, 6), 2, 1),        # every old frame padded
])
def test_extending_the_history_at_a_block_boundary_equals_one_prefill(blocks, pad, n_old):
    # block causality: appending whole blocks never changes the rows already cached
    full, ext = _extended_and_full(blocks, pad, n_old)
    for (Kf, Vf), (Ke, Ve) in zip(full, ext):
        assert Kf.shape == Ke.shape
        assert torch.max(torch.abs(Kf - Ke)) < 1e-12
        assert torch.max(torch.abs(Vf - Ve)) < 1e-12


def test_extending_inside_a_block_is_not_exact():
    # frames of one block read each other: appending half a block would leave
    # the cached half stale, which is why the C-ABI rejects such a split
    full, ext = _extended_and_full((0, 0, 1, 1, 2, 3, 4), 0, 3)
    assert max(float(torch.max(torch.abs(Kf - Ke))) for (Kf, _), (Ke, _) in zip(full, ext)) > 1e-6


# ---------------------------------------------------------------- rotary option
def test_rope_closed_forms():
    c1, s1, c5, s5 = math.cos(1), math.sin(1), math.cos(5), math.sin(5)
    # one pair (dh = 2): (x0 + i x1) exp(i p)
    x = torch.tensor([[[1.0, 0.0]], [[0.0, 1.0]], [[0.3, -0.7]]], dtype=f64)
    y = O.rope(x, torch.tensor([1, 1, 5]))
    want = torch.tensor([[[c1, s1]], [[-s1, c1]], [[0.3 * c5 + 0.7 * s5, 0.3 * s5 - 0.7 * c5]]],
                        dtype=f64)
    assert torch.max(torch.abs(y - want)) < 1e-15
    # dh = 4: pair 0 turns at rate 1, pair 1 at 10000^(-1/2) = 0.01
    y4 = O.rope(torch.tensor([[[1.0, 0.0, 1.0, 0.0]]], dtype=f64), torch.tensor([100]))
    want4 = torch.tensor([math.cos(100), math.sin(100), c1, s1], dtype=f64)
    assert torch.max(torch.abs(y4[0, 0] - want4)) < 1e-13
    # position 0 is the identity; every pair keeps its length
    r = torch.randn((7, 3, 8), dtype=f64, generator=torch.Generator().manual_seed(3))
    assert torch.equal(O.rope(r, torch.zeros(7, dtype=torch.int64)), r)
    rr = O.rope(r, torch.arange(7) * 977)
    n0 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    n1 = rr[..., 0::2] ** 2 + rr[..., 1::2] ** 2
    assert torch.max(torch.abs(n0 - n1)) < 1e-12


def test_rope_scores_depend_on_relative_position_only():
    g = torch.Generator().manual_seed(5)
    q = torch.randn((1, 2, 16), dtype=f64, generator=g)
    k = torch.randn((1, 2, 16), dtype=f64, generator=g)

    def score(m, n):
        return (O.rope(q, torch.tensor([m])) * O.rope(k, torch.tensor([n]))).sum(-1)

    for m, n, sh in [(3, 0, 11), (0, 40, 1000), (9216, 17, 123)]:
        assert torch.max(torch.abs(score(m, n) - score(m + sh, n + sh))) < 1e-9
    assert torch.max(torch.abs(score(3, 0) - score(4, 0))) > 1e-3


def test_rope_option_padding_and_streaming():
    cfg = _tiny(rope=True)
    inp = inputs.generate(cfg, threads=1)
    ref = O.run_chunk(cfg, inp, drop_padded=True)
    kept = O.run_chunk(cfg, inp, drop_padded=False)
    # positions count valid tokens: padded frames left out or kept and masked agree
    assert np.max(np.abs(ref["actions"] - kept["actions"])) < 1e-12
    # the option does change the result
    assert np.max(np.abs(ref["actions"] - O.run_chunk(_tiny(), inp)["actions"])) > 1e-6
    # appending whole blocks leaves every cached row (and its position) unchanged
    full, ext = _extended_and_full((0, 1, 2, 3, 4, 5, 6), 1, 3, rope=True)
    for (Kf, Vf), (Ke, Ve) in zip(full, ext):
        assert torch.max(torch.abs(Kf - Ke)) < 1e-12
        assert torch.max(torch.abs(Vf - Ve)) < 1e-12


# ---------------------------------------------------------------- sharp variant
@pytest.mark.parametrize("D,qk_std", [(256, 0.12), (1024, 0.06)])
def test_sharp_variant_scores_are_peaked(D, qk_std):
    # the diagnostic variant does what it is for: Wq, Wk ~ N(0, qk_std^2) give
    # pre-softmax scores of std about D qk_std^2 (3.7 here) in the first video
    # layer, against about 0.4 with 0.02 at width 1024
    cfg = configs.small("SH", dtype="f32", L=1, D=D, Hh=D // 64, Fm=256, P=64, Fh=2, Ff=1,
                        frame_block=(0, 1, 2), pad_frames=0, V=1, N=1, read_map=(0,),
                        qk_std=qk_std)
    inp = inputs.generate(cfg)
    w = O.to_torch_expert(inp["video"], f64)
    x = torch.from_numpy(inp["hist"][0].reshape(-1, cfg.Cv)).double()
    X = O.embed(x, w["w_in"], 0.0, cfg.D)
    lw = w["layers"][0]
    qkv = O.rmsnorm(X, lw["g1"]) @ lw["wqkv"].T
    q = qkv[:, :cfg.D].reshape(-1, cfg.Hh, cfg.dh).permute(1, 0, 2)
    k = qkv[:, cfg.D:2 * cfg.D].reshape(-1, cfg.Hh, cfg.dh).permute(1, 2, 0)
    s = torch.matmul(q, k) / math.sqrt(cfg.dh)
    assert 2.5 < float(s.std()) < 5.5


# ---------------------------------------------------------------- text/state condition
def test_condition_sequence_closed_form():
    # the text tokens as they are, then one proprio token: the robot state
    # through one linear layer, of the text width ("Fast-WAM 精读" section 四.5)
    r = np.random.default_rng(30)
    text = torch.tensor(r.standard_normal((5, 12)), dtype=f64)
    state = torch.tensor(r.standard_normal(7), dtype=f64)
    W = torch.tensor(r.standard_normal((12, 7)), dtype=f64)     # [Ct][S]
    ctx = O.condition(text, state, W)
    assert tuple(ctx.shape) == (6, 12)
    assert torch.equal(ctx[:5], text)
    assert torch.max(torch.abs(ctx[5] - F.linear(state, W))) < 1e-13


def _cond_weights(r, D, Dq, Ct, Fm, std=0.2):
    t = lambda *sh: torch.tensor(r.standard_normal(sh) * std, dtype=f64)
    return {"g1": 1 + t(D), "wqkv": t(3 * Dq, D), "wo": t(D, Dq), "g2": 1 + t(D), "w1": t(Fm, D),
            "w2": t(D, Fm), "gx": 1 + t(D), "wqx": t(Dq, D), "wkvx": t(2 * Dq, Ct), "wox": t(D, Dq)}


def test_cross_attention_layer_vs_library():
    # self-attention, then cross-attention to the condition, then the MLP, with
    # the expert width (40), the attention width (48 = 3 x 16) and the
    # condition width (24) all different, so a transposed or swapped weight fails
    r = np.random.default_rng(31)
    D, Hh, dh, Ct, Fm, n, nc, Tc = 40, 3, 16, 24, 56, 9, 11, 7
    Dq = Hh * dh
    w = _cond_weights(r, D, Dq, Ct, Fm)
    X = torch.tensor(r.standard_normal((n, D)), dtype=f64)
    sctx = (torch.tensor(r.standard_normal((nc, Hh, dh)), dtype=f64),
            torch.tensor(r.standard_normal((nc, Hh, dh)), dtype=f64))
    c = torch.tensor(r.standard_normal((Tc, Ct)), dtype=f64)
    cond = O.condition_kv(c, w, Hh)
    kc, vc = F.linear(c, w["wkvx"]).split(Dq, dim=1)
    assert torch.equal(cond[0], kc.reshape(Tc, Hh, dh)) and torch.equal(cond[1], vc.reshape(Tc, Hh, dh))
    got, _, _ = O.layer(X, w, Hh, sctx, None, cond=cond)

    sdpa = lambda q, k, v: F.scaled_dot_product_attention(
        q.permute(1, 0, 2), k.permute(1, 0, 2), v.permute(1, 0, 2)).permute(1, 0, 2)
    Y = F.rms_norm(X, (D,), w["g1"], eps=1e-6)
    q, k, v = (u.reshape(n, Hh, dh) for u in F.linear(Y, w["wqkv"]).split(Dq, dim=1))
    X1 = X + F.linear(sdpa(q, torch.cat([sctx[0], k]), torch.cat([sctx[1], v])).reshape(n, Dq), w["wo"])
    qx = F.linear(F.rms_norm(X1, (D,), w["gx"], eps=1e-6), w["wqx"]).reshape(n, Hh, dh)
    X2 = X1 + F.linear(sdpa(qx, kc.reshape(Tc, Hh, dh), vc.reshape(Tc, Hh, dh)).reshape(n, Dq), w["wox"])
    ref = X2 + F.linear(F.gelu(F.linear(F.rms_norm(X2, (D,), w["g2"], eps=1e-6), w["w1"])), w["w2"])
    assert torch.max(torch.abs(got - ref)) < 1e-12
    # the sub-layer is there: without it the result differs
    plain, _, _ = O.layer(X, w, Hh, sctx, None)
    assert torch.max(torch.abs(got - plain)) > 1e-3


def test_cross_attention_zero_output_is_the_plain_layer():
    r = np.random.default_rng(32)
    w = _cond_weights(r, 32, 32, 20, 48)
    w["wox"] = torch.zeros_like(w["wox"])
    X = torch.tensor(r.standard_normal((6, 32)), dtype=f64)
    cond = O.condition_kv(torch.tensor(r.standard_normal((5, 20)), dtype=f64), w, 2)
    a, _, _ = O.layer(X, w, 2, None, None, cond=cond)
    b, _, _ = O.layer(X, w, 2, None, None)
    assert torch.equal(a, b)


def test_single_condition_token_reads_its_value():
    # one condition token: every query's cross-attention returns that token's
    # V exactly (softmax over one key), so with the other residual branches
    # zeroed the layer adds V_c Wox^T to every row
    r = np.random.default_rng(33)
    D, Hh, Ct = 32, 2, 20
    w = _cond_weights(r, D, D, Ct, 48)
    w["wo"] = torch.zeros_like(w["wo"])
    w["w2"] = torch.zeros_like(w["w2"])
    X = torch.tensor(r.standard_normal((6, D)), dtype=f64)
    c = torch.tensor(r.standard_normal((1, Ct)), dtype=f64)
    got, _, _ = O.layer(X, w, Hh, None, None, cond=O.condition_kv(c, w, Hh))
    vc = F.linear(c, w["wkvx"])[:, D:]
    assert torch.max(torch.abs(got - (X + F.linear(vc, w["wox"])))) < 1e-13


@pytest.mark.parametrize("rope", [False, True])
def test_joint_sequence_with_condition_equals_cached_path(rope):
    # The text/state K, V computed once per call (condition_cache) equal the
    # joint pass's own projections of the condition: the cache rows and the
    # action v-hat of one uncached joint [video ; action] pass, in which every
    # row reads the condition through its expert's cross-attention.
    cfg = _tiny(rope=rope, Tc=4, Ct=10, S=3)
    inp = inputs.generate(cfg, threads=1)
    assert inp["text"].shape == (1, 3, 10) and inp["proprio_w"].shape == (10, 3)
    vw = O.to_torch_expert(inp["video"], f64)
    aw = O.to_torch_expert(inp["action"], f64)
    ctx = O.episode_condition(cfg, inp, 0, f64)
    condv, conda = O.condition_cache(cfg, vw, ctx), O.condition_cache(cfg, aw, ctx)
    cache, z, frames = O.video_prefill(cfg, vw, inp["hist"][0], inp["hist_valid"][0], inp["eps_v"][0],
                                       cond=condv)
    t0 = float(O.schedule(cfg.N, 0.0)[0])
    a = torch.tensor(inp["eps_a"][0], dtype=f64)
    v_cached = O.action_velocity(cfg, aw, O.read_layers(cfg, cache, None), a, t0,
                                 int(cache[0][0].shape[0]), conda)
    valid_frames = [f for f in range(cfg.Fh) if inp["hist_valid"][0][f]]
    hist_tok = torch.tensor(inp["hist"][0][valid_frames], dtype=f64).reshape(-1, cfg.Cv)
    vtok = torch.cat([hist_tok, z])
    sig_f = float(O.schedule(cfg.V, cfg.sigma_star)[-1])
    vsig = [0.0] * hist_tok.shape[0] + [sig_f] * z.shape[0]
    fvalid = list(inp["hist_valid"][0]) + [1] * cfg.Ff
    v_joint, kv = O.joint_mot_step(cfg, vw, aw, vtok, vsig, frames, fvalid, a, t0, ctx=ctx)
    assert torch.max(torch.abs(v_joint - v_cached)) < 1e-12
    for (Kc, Vc), (Kj, Vj) in zip(cache, kv):
        assert torch.max(torch.abs(Kc - Kj)) < 1e-12
        assert torch.max(torch.abs(Vc - Vj)) < 1e-12
    # and the condition matters: the chunk moves when the state changes
    inp2 = dict(inp, state=inp["state"] + 1.0)
    assert np.max(np.abs(O.run_chunk(cfg, inp)["actions"] - O.run_chunk(cfg, inp2)["actions"])) > 1e-4
