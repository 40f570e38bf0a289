"""Build the mgattn HIP library in-tree for gfx950 (hipcc cross-compiles; no GPU needed).

    python -m vit_perception_encoder_amd.build [--asm DIR]

The result is ``vit_perception_encoder_amd/_lib/libmgattn.so``.  ``--asm DIR`` also
writes the device assembly, for reading register and LDS use.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
SOURCES = [CSRC / "mgattn.hip"]
HEADERS = sorted(CSRC.glob("*.hpp")) + [ROOT / "include" / "mgattn.h"]
LIB_DIR = PKG / "_lib"
LIB = LIB_DIR / "libmgattn.so"
ARCH = "gfx950"

# Packed-f32 VALU forms are kept out of the code object: ordinary scalar f32 code only.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", str(ROOT / "include"),
          "-Wall", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(exe).exists():
        raise RuntimeError("hipcc not found: the mgattn library needs ROCm's hipcc to build")
    return exe


def build(asm_dir: str | None = None, verbose: bool = False) -> Path:
    LIB_DIR.mkdir(exist_ok=True)
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-shared", "-o", str(tmp), *map(str, SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if asm_dir:
        out = Path(asm_dir)
        out.mkdir(parents=True, exist_ok=True)
        subprocess.run([hipcc(), *COMMON, *DEVICE_FLAGS, "--cuda-device-only", "-S", "-o",
                        str(out / "mgattn-gfx950.s"), *map(str, SOURCES)], check=True)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="also write device assembly into this directory")
    args = ap.parse_args()
    print(build(args.asm, verbose=True))


if __name__ == "__main__":
    main()
