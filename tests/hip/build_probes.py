"""Build the test-only HIP probes in this folder (hipcc, gfx950) into
lib<name>.so beside their sources.  Called by __graft_entry__.build()."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> list:
    built = []
    for src in sorted(glob.glob(os.path.join(HERE, "*.hip"))):
        name = os.path.splitext(os.path.basename(src))[0]
        lib = os.path.join(HERE, f"lib{name}.so")
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", tmp]
        subprocess.run(cmd, check=True, capture_output=True)
        os.replace(tmp, lib)
        built.append(lib)
    return built


if __name__ == "__main__":
    print("\n".join(build()))
