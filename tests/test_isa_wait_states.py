"""Wait states around the GEMV's inline-assembly DPP dots, checked in the
compiled gfx950 code (CPU only: hipcc's device assembly of lutq_matmul.hip).

The compiler inserts no wait states around inline assembly. The DPP dot chain
(lutq_device.h, dot2_bcast4) carries its own, and relies on one rule: a
v_dot2c_f32_f16_dpp result is read by a plain VALU instruction only after 3
or more wait states, while another DPP dot on the same accumulator may read
it at once. The compiler schedules the code around the asm blocks, so this
test scans every GEMV kernel of every code width for the first instruction
after each DPP dot that touches its destination register: it must be the
next DPP dot of the chain, or come after at least 3 wait states (s_nop N
counts N + 1, any other instruction 1).
"""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from weight_only_lut_amd import build

pytestmark = pytest.mark.skipif(
    not (os.environ.get("HIPCC") or shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
    reason="needs hipcc")

DOT = re.compile(r"v_dot2c_f32_f16_dpp (v\d+),")
NOP = re.compile(r"s_nop (\d+)")
RANGE = re.compile(r"v\[(\d+):(\d+)\]")


def _device_asm(bits, tmp_path):
    out = os.path.join(tmp_path, f"matmul{bits}.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, f"-DLUTQ_MATMUL_BITS={bits}", "-I", os.path.join(build.ROOT, "include"),
           "--cuda-device-only", "-S", "-o", out, os.path.join(build.CSRC, "lutq_matmul.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as fh:
        return fh.read()


def _kernels(asm, bits):
    # the GEMV instantiations: matmul_kernel<BITS, false, ...>
    for name in re.findall(r"^(_ZN4lutq13matmul_kernelILi%dELb0[^:\s]*):" % bits, asm, re.M):
        start = asm.index(name + ":")
        body = asm[start:asm.index(".Lfunc_end", start)]
        yield name, [ln.strip() for ln in body.splitlines()
                     if ln.strip() and not ln.strip().startswith((";", "."))]


def _violations(lines):
    found = []
    for i, line in enumerate(lines):
        m = DOT.match(line)
        if not m:
            continue
        reg, n = m.group(1), int(m.group(1)[1:])
        waits = 0
        for nxt in lines[i + 1:i + 64]:
            nop = NOP.match(nxt)
            if nop:
                waits += int(nop.group(1)) + 1
                continue
            touches = re.search(r"\b%s\b" % reg, nxt) or any(
                int(a) <= n <= int(b) for a, b in RANGE.findall(nxt))
            if touches:
                if not nxt.startswith(f"v_dot2c_f32_f16_dpp {reg},") and waits < 3:
                    found.append((line, nxt, waits))
                break
            waits += 1
    return found


def test_dpp_dot_results_wait_three_states(tmp_path):
    with ThreadPoolExecutor(3) as pool:
        asms = dict(zip((2, 3, 4), pool.map(lambda b: _device_asm(b, str(tmp_path)), (2, 3, 4))))
    kernels = dots = 0
    for bits, asm in asms.items():
        for name, lines in _kernels(asm, bits):
            kernels += 1
            dots += sum(1 for ln in lines if DOT.match(ln))
            bad = _violations(lines)
            assert not bad, f"{name}: {bad[:3]}"
    # every width has GEMV kernels, and they use the DPP dot chain
    assert kernels >= 3 * 32 and dots > 1000, (kernels, dots)
