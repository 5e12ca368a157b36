"""Host-side pieces of bench.py on the CPU: the kernel each profiled case
launches exists in the library under the name the profile summary looks
for; the measured-floor interpolation and the roofline fractions."""

import os
import shutil
import subprocess

import pytest

import bench
import weight_only_lut_amd as lutq
from synth import workloads


def _built_kernels():
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-C", lutq.library_path()], capture_output=True, text=True).stdout
    names = set()
    for ln in out.splitlines():
        if "lutq::matmul_kernel<" in ln:
            names.add(ln[ln.index("matmul_kernel<"):].replace("(lutq::MatmulParams)", "").strip())
    return names


def test_profiled_kernels_exist():
    lutq.load_library()
    names = _built_kernels()
    for label, wname, mat, M in bench.PROFILE_CASES:
        w = workloads.WORKLOADS[wname]
        _, m = w.matrix(mat)
        sig = bench.kernel_signature(w.bits, w.group, M, lutq.plan(M, m.N, m.K, w.bits))
        assert sig in names, (label, sig)
    # every config row's kernel as well (plain tables, fp16)
    for wname, w in workloads.WORKLOADS.items():
        for m in w.matrices:
            for M in w.batches:
                sig = bench.kernel_signature(w.bits, w.group, M, lutq.plan(M, m.N, m.K, w.bits))
                assert sig in names, (wname, m.name, M, sig)


def test_stream_floor_and_roofs():
    f = bench.StreamFloor([(1 << 20, 2.0), (30 << 20, 6.0), (512 << 20, 78.0)], 1.6)
    assert f(1 << 20) == 2.0 and f(30 << 20) == 6.0
    assert f(1000) == 1.6                                      # never below the launch floor
    mid = f(15 << 20)
    assert 2.0 < mid < 6.0
    assert f(1 << 30) > 78.0                                   # extrapolated past the largest size
    assert abs(f.gbps() - (482 << 20) / (72.0 * 1e3)) < 1e-6
    r = bench.row_stats(8.0, 32_000_000, 10**8)
    assert r["bound"] == "hbm" and abs(r["frac_of_roof"] - 0.5) < 1e-9
    r = bench.row_stats(10.0, 1_000_000, 25 * 10**9)          # 10 us at 2.5 PFLOP/s
    assert r["bound"] == "mfma" and abs(r["frac_of_roof"] - 1.0) < 1e-9
    bench.measured_roof(r, f, 2000.0)
    assert abs(r["measured_roof_us"] - 12.5) < 1e-9 and r["frac_of_measured_roof"] == 1.25
