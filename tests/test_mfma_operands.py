"""CPU check of the library's device code as compiled for gfx950: no matrix instruction
may read an A or B operand from registers that overlap its own result registers.

An MFMA whose accumulator input the compiler folded to the inline constant 0 (an
accumulator it can prove zero, e.g. in a peeled first step) was once given a B operand
inside its 16 result registers, and the products came out wrong on the GPU.  The
kernels avoid that form; this test compiles every source to gfx950 assembly (with the
library's own flags) and checks each matrix instruction's operands."""

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from deformable_convolution_vision_amd import build as libbuild

_MFMA = re.compile(r"^\s*(v_mfma\S*)\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)")


def _regs(op: str):
    op = op.rstrip(",")
    m = re.fullmatch(r"[va]\[(\d+):(\d+)\]", op)
    if m:
        return op[0], int(m.group(1)), int(m.group(2))
    m = re.fullmatch(r"([va])(\d+)", op)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(2))
    return None


def _overlap(x, y) -> bool:
    return x is not None and y is not None and x[0] == y[0] and not (x[2] < y[1] or x[1] > y[2])


def _asm(src: str, out: str) -> str:
    cmd = [libbuild.hipcc(), *libbuild.HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr[-2000:]}")
    return out


def test_no_matrix_operand_overlaps_its_result():
    if not os.path.exists(libbuild.hipcc()):
        pytest.skip("hipcc not found")
    srcs = [os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES]
    with tempfile.TemporaryDirectory() as d:
        outs = [os.path.join(d, os.path.basename(s) + ".s") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(_asm, srcs, outs))
        n = 0
        bad = []
        for s, o in zip(srcs, outs):
            for line in open(o):
                m = _MFMA.match(line)
                if not m:
                    continue
                n += 1
                dst, a, b = _regs(m.group(2)), _regs(m.group(3)), _regs(m.group(4))
                if _overlap(dst, a) or _overlap(dst, b):
                    bad.append(f"{os.path.basename(s)}: {line.strip()}")
    assert n > 0, "no matrix instruction found in the compiled library"
    assert not bad, "matrix instructions reading operands from their own result registers:\n" + "\n".join(bad[:10])
