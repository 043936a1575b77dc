"""Build the HIP library libfa_fwd.so (forward and backward kernels) in-tree for
gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "fa_fwd.hip", PKG / "csrc" / "fa_bwd.hip"]
HEADERS = [ROOT / "include" / "fa_fwd.h", ROOT / "include" / "fa_bwd.h"]
LIB = PKG / "libfa_fwd.so"
# Race-check builds of the forward source (not the product): LDS poisoned
# with NaN patterns at kernel start, and tile loads serialised behind the
# reads; both must reproduce the product's outputs bit for bit.
DEBUG_LIBS = {
    "poison": (PKG / "libfa_fwd_debug_poison.so", ["-DFA_DEBUG_LDS_POISON"]),
    "serial": (PKG / "libfa_fwd_debug_serial.so", ["-DFA_DEBUG_SERIAL_TILES"]),
}

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> Path:
    """Compile every source into LIB (always recompiles)."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{ROOT / 'include'}", *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_debug(verbose: bool = False) -> list:
    """Compile the race-check builds of the forward source (always recompiles)."""
    out = []
    for path, defs in DEBUG_LIBS.values():
        tmp = path.with_suffix(".so.tmp")
        cmd = [hipcc(), *HIPCC_FLAGS, *defs, f"-I{ROOT / 'include'}", str(SOURCES[0]), "-o",
               str(tmp)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
        out.append(path)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_debug(verbose=True))
