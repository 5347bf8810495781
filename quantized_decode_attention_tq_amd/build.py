"""Build libtq.so (the C-ABI library) in-tree with hipcc for gfx950.

    python quantized_decode_attention_tq_amd/build.py             # libtq.so + libtq_probe.so
    python quantized_decode_attention_tq_amd/build.py --no-probe

(Run it by path: importing the package itself requires the built library.)

libtq_probe.so holds small kernels that tests use to check compiler-builtin
lane layouts and rounding on the GPU; it is not part of the product path.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")

LIB_SOURCES = ["tq_host.cpp", "tq_store.hip", "tq_decode.hip", "tq_dequant.hip"]
PROBE_SOURCES = ["tests/tq_probe.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed-FP32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libtq")
    return h


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"compile failed: {os.path.basename(src)}")
    noisy = [l for l in (r.stderr or "").splitlines() if "warning" in l and "packed-fp32-ops" not in l]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")


def _link(objs, out) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"link failed: {os.path.basename(out)}")
    os.replace(tmp, out)


def build_lib(name: str, sources, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in sources]
    objs = [os.path.join(BUILD, name + "_" + os.path.basename(s).replace(".", "_") + ".o") for s in sources]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
    out = os.path.join(HERE, f"lib{name}.so")
    _link(objs, out)
    return out


def build(probe: bool = True) -> list:
    outs = [build_lib("tq", LIB_SOURCES)]
    if probe:
        outs.append(build_lib("tq_probe", PROBE_SOURCES))
    return outs


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--no-probe", action="store_true")
    args = ap.parse_args()
    for o in build(probe=not args.no_probe):
        print(o)


if __name__ == "__main__":
    main()
