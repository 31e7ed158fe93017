"""Build libindexer_fp4.so for gfx950 with hipcc (one object per source, then a shared link)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libindexer_fp4.so")
SOURCES = ["errors.hip", "quant_cache.hip", "schedule.hip", "score_decode.hip", "score_prefill.hip", "topk.hip"]
# a measurement kernel of its own (bench.py --mfma-valu-probe), kept out of the product library
PROBE_SOURCE = "probe_mfma_valu.hip"
PROBE_LIB_PATH = os.path.join(HERE, "libindexer_fp4_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
    "-Wno-unused-command-line-argument",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs (no copies out of accumulation registers)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; anything else is shown
    noise = "not a recognized feature for this target"
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out)
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, path)


def build(jobs: int = 8) -> str:
    """Compile every source and link libindexer_fp4.so (and the probe library); always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
