"""Build libwam.so (HIP, gfx950) in-tree with hipcc.

    python -m kv_cached_flow_amd.build          # compile + link
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwam.so")
OBJ = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _resources(stderr: str) -> list:
    """(kernel, VGPRs, AGPRs, scratch bytes per lane, waves per SIMD) from the
    compiler's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in stderr.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        val = val.strip()
        if key == "Function Name":
            cur = {"name": val}
            out.append(cur)
        elif cur is not None and key in ("VGPRs", "AGPRs", "ScratchSize [bytes/lane]",
                                         "Occupancy [waves/SIMD]"):
            cur[key.split()[0]] = int(val)
    return out


def _compile(src: str) -> tuple:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj, _resources(r.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    res = [k for _, ks in done for k in ks]
    # No kernel may spill to scratch: a spill is a silent slowdown (and a
    # sign that a register budget was overrun).
    with open(os.path.join(OBJ, "resources.txt"), "w") as f:
        for k in sorted(res, key=lambda k: k["name"]):
            f.write(f"{k.get('VGPRs', '?'):>4} vgpr {k.get('AGPRs', '?'):>4} agpr "
                    f"{k.get('ScratchSize', '?'):>5} scratch {k.get('Occupancy', '?'):>2} waves  {k['name']}\n")
    spill = [k["name"] for k in res if k.get("ScratchSize", 0) > 0]
    if spill:
        raise RuntimeError("kernels use scratch memory (register spills):\n  " + "\n  ".join(spill))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
