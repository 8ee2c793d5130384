"""Build the gfx950 library ``libdeltanet.so`` in-tree with hipcc.

    python -m chunkwise_delta_rule_amd.build

The library is the C-ABI declared in ``include/deltanet.h``: the host layer
(``csrc/api.cpp``) and the kernels (``csrc/kernels.hip``, ``csrc/chain_bf16.hip``,
``csrc/decode.hip``) and the no-allocation entry point (``csrc/noalloc.hip``),
compiled for gfx950
only. Packed-fp32 VALU instructions are switched off for all device code.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdeltanet.so")
SOURCES = [os.path.join(PKG, "csrc", "kernels.hip"), os.path.join(PKG, "csrc", "chain_bf16.hip"),
           os.path.join(PKG, "csrc", "bwd_grad.hip"), os.path.join(PKG, "csrc", "decode.hip"),
           os.path.join(PKG, "csrc", "noalloc.hip"), os.path.join(PKG, "csrc", "api.cpp")]
HEADERS = [os.path.join(PKG, "csrc", "dn_internal.h"), os.path.join(PKG, "csrc", "dn_work.h"),
           os.path.join(ROOT, "include", "deltanet.h")]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out: str = LIB, extra=None) -> list[str]:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", out]
    if extra:
        cmd[1:1] = list(extra)
    return cmd


def build(out: str = LIB, verbose: bool = False, extra=None) -> str:
    """Compile the library (always; the caller decides when). Returns its path."""
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
