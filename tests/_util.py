"""Helpers shared by the tests (comparison metrics, device <-> host)."""
import numpy as np


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float32).numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def gpu_cache_layer(dc, l, b, n):
    """K [n, Hh, dh] and V [n, Hh, dh] of episode b, layer l, first n rows, from the
    device cache (k: [L][B][Hh][cap][dh], v: [L][B][Hh][dh][cap])."""
    k = to_np(dc.cache.k[l, b, :, :n, :]).transpose(1, 0, 2)
    v = to_np(dc.cache.v[l, b, :, :, :n]).transpose(2, 0, 1)
    return k, v


def print_case(msg):
    print(msg, flush=True)
