"""Build libradamw.so (gfx950) in-tree with hipcc.

    python -m optimizer_step_dl_amd.build [-DNAME=VALUE ...] [--out PATH]

The HIP sources are compiled for gfx950 only.  Packed-FP32 instruction
selection is disabled (``-packed-fp32-ops``): the update is scalar FP32 per
element by design and the packed forms are not wanted here.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libradamw.so")
SOURCES = ["radamw_api.cpp", "radamw_update.hip", "radamw_stats.hip", "radamw_staged.hip", "radamw_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-x", "hip",
]


def build(defines: list[str] | None = None, out: str | None = None, quiet: bool = True) -> str:
    out = out or LIB_PATH
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *[f"-D{d}" for d in (defines or [])],
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if not quiet:
        sys.stderr.write(res.stderr)
    os.replace(out + ".tmp", out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    print(build(args.defines, args.out, quiet=False))


if __name__ == "__main__":
    main()
