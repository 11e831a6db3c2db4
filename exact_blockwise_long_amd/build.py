"""Build libblockattn.so in-tree with hipcc for gfx950.

    python -m exact_blockwise_long_amd.build

Compiles every ``csrc/*.hip`` into ``exact_blockwise_long_amd/libblockattn.so``.
Packed fp32 VALU forms are disabled for device code (``-packed-fp32-ops``).
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libblockattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # No kernel input or intermediate is NaN by construction (infinities are
    # used and kept); this lets fmaxf map to v_max/v_max3 without canonicalising.
    "-fno-honor-nans",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def sources_digest() -> str:
    """SHA-256 over the kernel sources and the public header (identifies a build)."""
    import hashlib
    h = hashlib.sha256()
    for path in sources() + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(INCLUDE, "blockattn.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile the library to ``out`` (the package's libblockattn.so by default);
    ``extra_flags`` go to hipcc after the standard ones (e.g. -D tuning macros)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{log}")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
