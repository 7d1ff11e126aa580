"""Compile libkvcluster.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
SOURCES = ["kvc_build.hip", "kvc_decode.hip", "kvc_api.cpp", "kvc_host.cpp"]
OUT = os.path.join(_HERE, "libkvcluster.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         # packed fp32 arithmetic stays off: only scalar fp32 instructions are emitted
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def command(out: str = OUT) -> list[str]:
    src = [os.path.join(_HERE, "csrc", s) for s in SOURCES]
    return [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(_HERE, "csrc"), *src, "-o", out]


def build(out: str = OUT) -> str:
    tmp = out + ".tmp"
    res = subprocess.run(command(tmp), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msg}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
