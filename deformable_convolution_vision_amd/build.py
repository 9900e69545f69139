"""Build libdcn_hip.so for gfx950 in-tree with hipcc.

    python -m deformable_convolution_vision_amd.build

Each source is compiled to its own object in parallel (a build directory next to
the library, kept out of the repository), then the objects are linked.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdcn_hip.so")
SOURCES = ["dcn_api.hip", "dcn_kernels.hip", "dcn_box.hip", "dcn_box_inst_a.hip", "dcn_box_inst_b.hip",
           "dcn_box_inst_c.hip", "dcn_box_inst_d.hip", "dcn_direct.hip", "dcn_backward.hip", "dcn_roi.hip",
           "dcn_om.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _messages(r: subprocess.CompletedProcess) -> list[str]:
    # hipcc's host pass does not know the device-only target feature; that warning is harmless
    return [l for l in (r.stdout + r.stderr).splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "is not a recognized feature" not in l]


def build(out_path: str = LIB, extra_flags: tuple[str, ...] = (), verbose: bool = False,
          sources: tuple[str, ...] | None = None, extra_objects: tuple[str, ...] = (),
          link_flags: tuple[str, ...] = ("-shared",)) -> str:
    """Compile the sources (default: every kernel and host file) with the extra flags and
    link them, with any extra objects, into out_path (a shared library by default)."""
    srcs = [os.path.join(CSRC, s) for s in (SOURCES if sources is None else sources)]
    objdir = os.path.join(os.path.dirname(out_path), "_build", os.path.basename(out_path))
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = _messages(r)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(msgs))
        if msgs and verbose:
            print("\n".join(msgs), file=sys.stderr)
        return obj

    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", *link_flags, *extra_flags, *objs, *extra_objects, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_messages(r)))
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
