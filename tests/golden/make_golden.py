"""Write the expected values of the full-size workloads C1-C6 by running the
CPU oracle (and nothing else) on the seeded inputs.

    python tests/golden/make_golden.py C1 C2 C3 C4 C5 C6 C1+fp8 C1+sharp C6+fp8

A name may carry options after "+": ``fp8`` (the E4M3 cache option),
``sharp`` (the diagnostic variant with Wq, Wk ~ N(0, 0.06^2): peaked
attention, score std about 3.7 at width 1024) and ``cond`` (the text/state
condition of ``configs.CONDITION``); the file is then
``<config>_<option>.json``.

Each ``<name>.json`` holds the input fingerprint, the final action chunk of
every episode, the v-hat of the first and last action steps, and sampled
cache rows (and fused rows for SparseMoT, imagined latents where the video
expert runs imagine steps), so the GPU tests can compare at full size
without re-running the oracle there.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from kv_cached_flow_amd import configs, inputs  # noqa: E402
from oracle import wam_oracle as O  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
N_SAMPLES = 16


def sample_points(cfg, seed=12345):
    """(row, head) pairs per episode in the valid cache, and the sampled layers."""
    rng = np.random.default_rng(seed)
    T = cfg.tokens_valid
    rows = np.sort(rng.choice(T, size=N_SAMPLES, replace=False))
    heads = rng.integers(0, cfg.Hh, size=N_SAMPLES)
    layers = sorted({0, cfg.L // 2, cfg.L - 1})
    return rows, heads, layers


def main(names):
    torch.set_num_threads(int(os.environ.get("ORACLE_THREADS", "8")))
    for name in names:
        # "<config>+<option>+...": the same workload with options
        base, *opts = name.split("+")
        kw = {}
        for o in opts:
            if o == "fp8":
                kw["kv_fp8"] = True
            elif o == "sharp":
                kw["qk_std"] = 0.06
            elif o == "cond":
                kw.update(configs.CONDITION)
            else:
                raise SystemExit(f"unknown option {o}")
        cfg = configs.get(base, **kw)
        fname = "_".join([base] + opts)
        t0 = time.time()
        inp = inputs.generate(cfg)
        rows, heads, layers = sample_points(cfg)
        samples = {"cache": [], "fused": []}

        def sampler(b, cache, fused):
            ent = {}
            for l in layers:
                K, V = cache[l]
                ent[str(l)] = {"k": K[rows, heads].double().numpy().tolist(),
                               "v": V[rows, heads].double().numpy().tolist()}
            samples["cache"].append(ent)
            if fused is not None:
                fe = {}
                for m in (0, len(fused) - 1):
                    K, V = fused[m]
                    fe[str(m)] = {"k": K[rows, heads].double().numpy().tolist(),
                                  "v": V[rows, heads].double().numpy().tolist()}
                samples["fused"].append(fe)

        if cfg.joint:
            out = O.run_codenoise(cfg, inp, cache_sampler=sampler)
        else:
            out = O.run_chunk(cfg, inp, cache_sampler=sampler, kv_fp8=cfg.kv_fp8)
        zrows = np.sort(np.random.default_rng(777).choice(cfg.Ff * cfg.P, size=64, replace=False))
        rec = {
            "config": name,
            "kv_fp8": cfg.kv_fp8,
            "qk_std": cfg.qk_std,
            "Tc": cfg.Tc,
            "seed": cfg.seed,
            "fingerprint": inputs.fingerprint(inp),
            "source": ("oracle/wam_oracle.py " + ("run_codenoise" if cfg.joint else "run_chunk")
                       + " (float32), tests/golden/make_golden.py"),
            "actions": out["actions"].tolist(),
            "vhat_first": out["vhat"][0].tolist(),
            "vhat_last": out["vhat"][-1].tolist(),
            "sample_rows": rows.tolist(),
            "sample_heads": heads.tolist(),
            "sample_layers": layers,
            "cache": samples["cache"],
            "fused": samples["fused"],
            "z_rows": zrows.tolist(),
            "z": out["z"][:, zrows].tolist() if (cfg.V >= 1 or cfg.joint) else None,
            "oracle_seconds": time.time() - t0,
        }
        with open(os.path.join(HERE, f"{fname}.json"), "w") as f:
            json.dump(rec, f)
        print(f"{name}: {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["C1", "C2", "C3", "C4", "C5"])
