"""Build libbsfa.so in-tree with hipcc for gfx950.

    python -m block_sparse_long_amd.build_lib [--isa DIR]

Compiles csrc/*.hip and csrc/*.cpp as HIP sources and links block_sparse_long_amd/libbsfa.so.
`--isa DIR` also keeps the device assembly there (for reading register use and schedules).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsfa.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the scores feed the softmax VALU directly instead of being
    # copied out of accumulation registers
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def build(isa_dir: str | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *FLAGS, "-x", "hip", "-c", src, "-o", obj]
        r = subprocess.run(cmd, cwd=BUILD_DIR, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if isa_dir and src.endswith(".hip"):
            os.makedirs(isa_dir, exist_ok=True)
            asm = os.path.join(isa_dir, os.path.basename(src)[:-4] + "-gfx950.s")
            subprocess.run([hipcc, *FLAGS, "-x", "hip", "--offload-device-only", "-S",
                            src, "-o", asm], check=True, capture_output=True)
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None, help="keep device assembly in this directory")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.isa, args.verbose))


if __name__ == "__main__":
    main()
