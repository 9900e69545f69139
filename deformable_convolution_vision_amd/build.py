"""Build libdcn_hip.so for gfx950 in-tree with hipcc.

    python -m deformable_convolution_vision_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdcn_hip.so")
SOURCES = ["dcn_api.hip", "dcn_kernels.hip", "dcn_box.hip", "dcn_direct.hip", "dcn_backward.hip", "dcn_roi.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out_path: str = LIB, extra_flags: tuple[str, ...] = (), verbose: bool = False) -> str:
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only target feature; that warning is harmless
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
