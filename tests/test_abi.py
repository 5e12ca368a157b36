"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments before any HIP call (so these run without a GPU).
Also the numpy reading of the packed layout against hand-derived bytes."""

import ctypes
import os
import re

import numpy as np
import pytest

import weight_only_lut_amd as lutq
from weight_only_lut_amd import _lib

from . import layout_spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, EINVAL, EBITS, EGROUP, EALIGN, EMISMATCH, ESIZE, EHIP, EUNSUP, ECAPTURE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def lib():
    return lutq.load_library()


def _declared():
    """Every function any header in include/ declares."""
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(lutq_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_covers_every_code(lib):
    for c in (OK, EINVAL, EBITS, EGROUP, EALIGN, EMISMATCH, ESIZE, EHIP, EUNSUP, ECAPTURE):
        assert lutq.strerror(c) != "unknown lutq status"
    assert lutq.strerror(-99) == "unknown lutq status"


def _cpu_packed(N, K, bits, group):
    import torch
    d = _desc(N=N, K=K, bits=bits, group=group)
    return _lib.Packed(torch.zeros(max(1, N * K * bits // 8), dtype=torch.uint8), d)


def test_binding_checks_every_tensor_before_calling():
    """Shapes, sizes and dtypes of every tensor argument are checked before
    any call into the library (here on CPU tensors, which are then refused
    for not being on the GPU)."""
    import torch
    f16, u8 = torch.float16, torch.uint8
    N, K = 64, 256
    P = _cpu_packed(N, K, 4, 128)
    x = torch.zeros((2, K), dtype=f16)
    lut = torch.zeros(16, dtype=f16)
    sc = torch.zeros((N, K // 128), dtype=f16)
    bad = [
        dict(x=torch.zeros((2, K + 128), dtype=f16)),          # K differs from the packed matrix
        dict(lut=torch.zeros(8, dtype=f16)),                   # 2^bits entries
        dict(scales=torch.zeros((N, 1), dtype=f16)),           # N * K / group entries
        dict(zeros=torch.zeros((N,), dtype=f16)),
        dict(types=torch.zeros((N, 1), dtype=u8)),
        dict(types=torch.zeros((N, 2), dtype=u8), lut=torch.zeros((5, 16), dtype=f16)),  # <= 4 tables
        dict(out=torch.zeros((2, N + 1), dtype=f16)),
    ]
    for over in bad:
        kw = dict(x=x, lut=lut, scales=sc)
        kw.update(over)
        with pytest.raises(ValueError):
            lutq.matmul(kw.pop("x"), P, kw.pop("lut"), kw.pop("scales"), **kw)
    with pytest.raises(TypeError):
        lutq.matmul(x, P, lut.float(), sc)
    with pytest.raises(TypeError):                             # right shapes, but on the CPU
        lutq.matmul(x, P, lut, sc)
    with pytest.raises(TypeError):
        lutq.matmul(x, "not packed", lut, sc)
    # binary coding: q planes of alphas and the output shape
    Pq = _cpu_packed(N, K, 3, 128)
    with pytest.raises(ValueError):
        lutq.matmul_bcq(x, Pq, torch.zeros((2, N, K // 128), dtype=f16))
    with pytest.raises(ValueError):
        lutq.matmul_bcq(x, Pq, torch.zeros((3, N, K // 128), dtype=f16),
                        out=torch.zeros((2, N - 1), dtype=f16))
    with pytest.raises(TypeError):
        lutq.matmul_bcq(x, Pq, torch.zeros((3, N, K // 128), dtype=f16))
    # the fused launch: per-matrix checks and K across matrices
    P2 = _cpu_packed(32, K, 4, 128)
    sc2 = torch.zeros((32, K // 128), dtype=f16)
    with pytest.raises(ValueError):
        lutq.matmul_multi(x, [(P, lut, sc), (P2, lut, sc)])
    with pytest.raises(ValueError):
        lutq.matmul_multi(x, [(P, lut, sc), (_cpu_packed(32, 2 * K, 4, 128), lut, sc2)])
    with pytest.raises(ValueError):
        lutq.matmul_multi(x, [(P, lut, sc)], outs=[])
    with pytest.raises(TypeError):
        lutq.matmul_multi(x, [(P, lut, sc), (P2, lut, sc2)])
    # the quantizer: 2-D weights and a 2^bits table
    w = torch.zeros((N, K), dtype=torch.float32)
    with pytest.raises(ValueError):
        lutq.quantize(w, torch.zeros(8, dtype=f16), 4, 128)
    with pytest.raises(ValueError):
        lutq.quantize(w.view(-1), lut, 4, 128)
    with pytest.raises(TypeError):
        lutq.quantize(w, lut, 4, 128)


def test_peaks_validate_before_launching(lib):
    P = ctypes.c_void_p
    assert lib.lutq_peak_stream_sink_bytes() == 2048 * 4 * 16
    assert lib.lutq_peak_stream(P(0), 1024, 0, P(0x1000), None) == EINVAL
    assert lib.lutq_peak_stream(P(0x1000), 0, 0, P(0x1000), None) == EINVAL
    assert lib.lutq_peak_stream(P(0x1000), 1000, 0, P(0x1000), None) == EINVAL   # not 16-byte units
    assert lib.lutq_peak_stream(P(0x1008), 1024, 1, P(0x1000), None) == EALIGN
    assert lib.lutq_peak_stream(P(0x1000), 1024, 1, P(0), None) == EINVAL
    assert lib.lutq_peak_mfma(2, 1, 10, P(0x1000), None) == EINVAL              # unknown kind
    assert lib.lutq_peak_mfma(0, 5, 10, P(0x1000), None) == EINVAL              # waves per SIMD
    assert lib.lutq_peak_mfma(0, 1, 0, P(0x1000), None) == EINVAL
    assert lib.lutq_peak_mfma(0, 1, 10, P(0), None) == EINVAL
    assert lib.lutq_peak_lds(17, 10, P(0x1000), None) == EINVAL
    assert lib.lutq_peak_lds(4, 0, P(0x1000), None) == EINVAL
    assert lib.lutq_peak_lds(4, 10, P(0), None) == EINVAL


def test_packed_bytes():
    assert lutq.packed_bytes(14336, 4096, 4, 128) == 14336 * 4096 // 2
    assert lutq.packed_bytes(4096, 14336, 3, 128) == 4096 * 14336 * 3 // 8
    assert lutq.packed_bytes(1000, 256, 4, 128) == 1008 * 256 // 2  # rows padded to 16
    assert lutq.packed_bytes(16, 128, 2, 0) == 16 * 128 // 4
    for bad in [(16, 128, 5, 128), (16, 128, 1, 128), (16, 100, 4, 0), (16, 256, 4, 64),
                (16, 384, 4, 256), (-1, 128, 4, 128), (0, 128, 4, 128)]:
        assert lutq.packed_bytes(*bad) == 0, bad


def _desc(N=64, K=256, bits=4, group=128, data=0x10000):
    d = _lib.PackedDesc()
    d.magic, d.version = _lib.LUTQ_MAGIC, _lib.LUTQ_LAYOUT_VERSION
    d.N, d.K, d.bits, d.group = N, K, bits, group
    d.nbytes = lutq.packed_bytes(N, K, bits, group)
    d.data = data
    return d


def test_repack_validates_before_launching(lib):
    out = _lib.PackedDesc()
    P = ctypes.c_void_p
    good = dict(codes=P(0x1000), N=64, K=256, bits=4, group=128, dst=P(0x20000), nb=1 << 20)

    def call(**kw):
        a = {**good, **kw}
        return lib.lutq_repack(a["codes"], a["N"], a["K"], a["bits"], a["group"], a["dst"],
                               a["nb"], ctypes.byref(out), None)

    assert call(bits=5) == EBITS
    assert call(bits=1) == EBITS
    assert call(group=64) == EGROUP
    assert call(K=200) == EGROUP
    assert call(K=384, group=256) == EGROUP
    assert call(N=-1) == EINVAL
    assert call(N=1 << 25) == EUNSUP
    assert call(codes=P(0)) == EINVAL
    assert call(dst=P(0)) == EINVAL
    assert call(dst=P(0x20008)) == EALIGN
    assert call(codes=P(0x1004)) == EALIGN          # codes are read 8 at a time
    assert call(nb=100) == ESIZE
    assert call(codes=P(0x20000)) == EINVAL           # overlapping buffers
    assert lib.lutq_repack(P(0x1000), 64, 256, 4, 128, P(0x20000), 1 << 20, None, None) == EINVAL
    # empty matrix: descriptor filled, nothing enqueued
    assert call(N=0) == OK and out.nbytes == 0 and out.N == 0 and out.magic == _lib.LUTQ_MAGIC


def test_matmul_validates_before_launching(lib):
    P = ctypes.c_void_p
    d = _desc()
    x, lut, sc, y = P(0x1000), P(0x2000), P(0x3000), P(0x4000)

    def call(desc=d, M=1, N=64, K=256, x=x, lut=lut, sc=sc, y=y, opts=None):
        return lib.lutq_matmul_ex(x, ctypes.byref(desc) if desc is not None else None, lut, sc, y,
                                  M, N, K, opts, None)

    assert call(desc=None) == EINVAL
    bad = _desc(); bad.magic = 0
    assert call(desc=bad) == EMISMATCH
    bad = _desc(); bad.version = 2
    assert call(desc=bad) == EMISMATCH
    bad = _desc(); bad.nbytes += 1
    assert call(desc=bad) == EMISMATCH
    assert call(desc=_desc(data=0x10004)) == EALIGN
    assert call(desc=_desc(data=0)) == EINVAL
    assert call(N=65) == EMISMATCH
    assert call(K=128) == EMISMATCH
    assert call(M=-1) == EINVAL
    assert call(x=P(0)) == EINVAL
    assert call(y=P(0)) == EINVAL
    assert call(x=P(0x1008)) == EALIGN
    assert call(sc=P(0x3001)) == EALIGN
    assert call(lut=P(0x2002)) == EALIGN     # the table is read as 4-byte words
    o = _lib.Options(); o.path = 7
    assert call(opts=ctypes.byref(o)) == EINVAL
    o = _lib.Options(); o.ksplit = -1
    assert call(opts=ctypes.byref(o)) == EINVAL
    o = _lib.Options(); o.reserved[3] = 1
    assert call(opts=ctypes.byref(o)) == EINVAL
    o = _lib.Options(); o.dtype = 2
    assert call(opts=ctypes.byref(o)) == EINVAL
    # bf16 activations run plain tables only
    o = _lib.Options(); o.dtype = 1
    z, ty = P(0x5000), P(0x6000)
    assert lib.lutq_matmul_zp(x, ctypes.byref(d), lut, sc, z, y, 1, 64, 256, ctypes.byref(o),
                              None) == EUNSUP
    assert lib.lutq_matmul_typed(x, ctypes.byref(d), lut, 2, ty, sc, None, y, 1, 64, 256,
                                 ctypes.byref(o), None) == EUNSUP
    d3 = _desc(bits=3)
    assert lib.lutq_matmul_bcq(x, ctypes.byref(d3), sc, y, 1, 64, 256, ctypes.byref(o),
                               None) == EUNSUP
    for path, tiles in [(0, 2), (1, 8), (1, 4), (1, 7), (2, 5), (2, 3), (2, 6), (1, -1)]:
        o = _lib.Options(); o.path, o.tiles = path, tiles
        assert call(opts=ctypes.byref(o)) == EINVAL, (path, tiles)
    # nothing to do: M == 0 (no HIP call is made)
    assert call(M=0) == OK
    assert lib.lutq_unpack(None, P(0x1000), None) == EINVAL


def test_matmul_multi_validates_before_launching(lib):
    P = ctypes.c_void_p
    descs = [_desc(), _desc(N=32), _desc(N=16)]

    def items(n=3, **over):
        arr = (_lib.MatmulItem * max(n, 1))()
        for i in range(n):
            d = over.get(f"desc{i}", descs[i % 3])
            arr[i].packed = ctypes.pointer(d) if d is not None else None
            arr[i].lut = over.get(f"lut{i}", 0x2000 + 0x100 * i)
            arr[i].scales = over.get(f"sc{i}", 0x3000 + 0x100 * i)
            arr[i].y = over.get(f"y{i}", 0x4000 + 0x1000 * i)
        return arr

    def call(arr=None, count=3, M=1, K=256, x=P(0x1000), opts=None):
        arr = items(count) if arr is None else arr
        return lib.lutq_matmul_multi(x, arr, count, M, K, opts, None)

    assert lib.lutq_matmul_multi(P(0x1000), None, 1, 1, 256, None, None) == EINVAL
    assert call(count=0) == EINVAL
    assert call(count=_lib.MAX_FUSED + 1, arr=items(_lib.MAX_FUSED + 1)) == EINVAL
    assert call(K=128) == EMISMATCH                          # K differs from the descriptors
    assert call(arr=items(desc1=_desc(N=32, bits=3))) == EMISMATCH
    assert call(arr=items(desc2=_desc(N=16, group=0))) == EMISMATCH
    bad = _desc(); bad.magic = 0
    assert call(arr=items(desc1=bad)) == EMISMATCH
    assert call(arr=items(desc0=None)) == EINVAL
    assert call(M=-1) == EINVAL
    assert call(x=P(0)) == EINVAL
    assert call(x=P(0x1008)) == EALIGN
    assert call(arr=items(y1=0)) == EINVAL
    assert call(arr=items(y2=0x4001)) == EALIGN
    assert call(arr=items(lut0=0x2002)) == EALIGN
    assert call(arr=items(sc1=0x3001)) == EALIGN
    assert call(arr=items(lut2=0)) == EINVAL
    o = _lib.Options(); o.path, o.tiles = 1, 4
    assert call(opts=ctypes.byref(o)) == EINVAL
    # nothing to do (no HIP call): M == 0, or every matrix empty
    assert call(M=0) == OK
    empty = [_desc(N=0), _desc(N=0)]
    arr = (_lib.MatmulItem * 2)()
    for i in range(2):
        arr[i].packed = ctypes.pointer(empty[i])
    assert lib.lutq_matmul_multi(P(0x1000), arr, 2, 4, 256, None, None) == OK


def test_matmul_zp_validates_before_launching(lib):
    P = ctypes.c_void_p
    x, lut, sc, z, y = P(0x1000), P(0x2000), P(0x3000), P(0x5000), P(0x4000)

    def call(desc=None, M=1, N=64, K=256, z=z, opts=None):
        d = _desc(N=N, K=K) if desc is None else desc
        return lib.lutq_matmul_zp(x, ctypes.byref(d), lut, sc, z, y, M, N, K, opts, None)

    assert call(desc=_desc(group=0)) == EGROUP          # zero points are per group
    assert call(z=P(0)) == EINVAL
    assert call(z=P(0x5001)) == EALIGN
    assert call(N=65, desc=_desc()) == EMISMATCH
    assert call(M=0) == OK
    # the fused launch: zeros on a tensor-wise matrix, misaligned zeros
    arr = (_lib.MatmulItem * 2)()
    d0, d1 = _desc(), _desc(N=32, group=0)
    for i, d in enumerate((d0, d1)):
        arr[i].packed, arr[i].lut, arr[i].scales, arr[i].y = ctypes.pointer(d), 0x2000, 0x3000, 0x4000
    arr[1].zeros = 0x5000
    assert lib.lutq_matmul_multi(x, arr, 2, 1, 256, None, None) == EMISMATCH   # groups differ
    d1b = _desc(N=32)
    arr[1].packed = ctypes.pointer(d1b)
    arr[1].zeros = 0x5001
    assert lib.lutq_matmul_multi(x, arr, 2, 1, 256, None, None) == EALIGN
    d2, d3 = _desc(group=0), _desc(N=32, group=0)
    arr[0].packed, arr[1].packed = ctypes.pointer(d2), ctypes.pointer(d3)
    arr[1].zeros = 0x5000
    assert lib.lutq_matmul_multi(x, arr, 2, 1, 256, None, None) == EGROUP


def test_matmul_typed_validates_before_launching(lib):
    P = ctypes.c_void_p
    x, luts, ty, sc, y = P(0x1000), P(0x2000), P(0x6000), P(0x3000), P(0x4000)

    def call(desc=None, nt=2, types=ty, M=1, N=64, K=256, luts=luts):
        d = _desc(N=N, K=K) if desc is None else desc
        return lib.lutq_matmul_typed(x, ctypes.byref(d), luts, nt, types, sc, None, y, M, N, K,
                                     None, None)

    assert call(desc=_desc(group=0)) == EGROUP
    assert call(nt=0) == EINVAL and call(nt=_lib.MAX_TYPES + 1) == EINVAL
    assert call(types=P(0)) == EINVAL
    assert call(luts=P(0x2002)) == EALIGN
    assert call(M=0) == OK


def test_matmul_bcq_validates_before_launching(lib):
    P = ctypes.c_void_p
    x, al, y = P(0x1000), P(0x3000), P(0x4000)

    def call(desc=None, alphas=al, M=1, opts=None):
        d = _desc(bits=3) if desc is None else desc
        return lib.lutq_matmul_bcq(x, ctypes.byref(d), alphas, y, M, d.N, d.K, opts, None)

    assert call(desc=_desc(bits=3, group=0)) == EGROUP
    assert call(alphas=P(0)) == EINVAL
    assert call(alphas=P(0x3001)) == EALIGN
    o = _lib.Options(); o.path, o.tiles = 2, 3
    assert call(opts=ctypes.byref(o)) == EINVAL          # no 3-tile MFMA shape
    assert call(M=0) == OK


def test_quantizer_validates_before_launching(lib):
    P = ctypes.c_void_p
    err = ctypes.c_double(0)
    good = dict(w=P(0x1000), lut=P(0x2000), bits=4, N=8, K=256, group=128, rule=0,
                codes=P(0x3000), scales=P(0x4000))

    def q(**kw):
        a = {**good, **kw}
        return lib.lutq_quantize(a["w"], a["lut"], a["bits"], a["N"], a["K"], a["group"], a["rule"],
                                 a["codes"], a["scales"], None)

    assert q(bits=5) == EBITS
    assert q(group=64) == EGROUP
    assert q(K=200) == EGROUP
    assert q(rule=2) == EINVAL
    assert q(N=-1) == EINVAL
    assert q(N=1 << 25) == EUNSUP
    assert q(w=P(0)) == EINVAL
    assert q(codes=P(0)) == EINVAL
    assert q(w=P(0x1008)) == EALIGN          # weights read 16 bytes at a time
    assert q(codes=P(0x3002)) == EALIGN      # codes written 4 at a time
    assert q(scales=P(0x4001)) == EALIGN
    assert q(N=0) == OK and q(K=0) == OK     # nothing to do, no HIP call
    # 16-bit weights: another dtype is rejected, and they need 8-byte alignment
    qx = lambda w, wdt: lib.lutq_quantize_ex(w, wdt, P(0x2000), 4, 8, 256, 128, 0, P(0x3000),
                                             P(0x4000), None)
    assert qx(P(0x1000), 3) == EINVAL
    assert qx(P(0x1004), 1) == EALIGN and qx(P(0x1004), 2) == EALIGN
    # table tuning
    upd = ctypes.c_int32(-1)
    tt = lambda **k: lib.lutq_tune_table(k.get("w", P(0x1000)), 0, P(0x2000), 4, k.get("N", 8), 256,
                                         128, 0, k.get("iters", 3), None, None, k.get("upd", ctypes.byref(upd)),
                                         None)
    assert tt(upd=None) == EINVAL and tt(iters=-1) == EINVAL
    assert tt(w=P(0x1004)) == EALIGN
    errs = (ctypes.c_double * 4)(1, 1, 1, 1)
    assert lib.lutq_tune_table(P(0x1000), 0, P(0x2000), 4, 0, 256, 128, 0, 3, None, errs,
                               ctypes.byref(upd), None) == OK
    assert upd.value == 0 and list(errs) == [0.0] * 4
    assert lib.lutq_quant_error(P(0x1000), P(0x2000), 4, 8, 256, 128, 0, None, None) == EINVAL
    assert lib.lutq_quant_error(P(0x1000), P(0x2000), 4, 0, 256, 128, 0, ctypes.byref(err), None) == OK
    assert err.value == 0.0
    best = ctypes.c_int32(-1)
    bases = (ctypes.c_double * 3)(1.5, 2.0, 1.0)
    assert lib.lutq_log_base_search(P(0x1000), 4, 8, 256, 128, bases, 3, ctypes.byref(best), None,
                                    None) == EINVAL          # a base <= 1
    bases = (ctypes.c_double * 1)(1.0001)                     # the table repeats an fp16 value
    assert lib.lutq_log_base_search(P(0x1000), 4, 8, 256, 128, bases, 1, ctypes.byref(best), None,
                                    None) == EINVAL
    bases = (ctypes.c_double * 2)(1.5, 2.0)
    assert lib.lutq_log_base_search(P(0x1000), 4, 8, 256, 128, bases, 0, ctypes.byref(best), None,
                                    None) == EINVAL
    assert lib.lutq_log_base_search(P(0x1000), 4, 0, 256, 128, bases, 2, ctypes.byref(best), None,
                                    None) == OK and best.value == 0


def test_plan_switches_paths_by_batch():
    # Without a GPU the device is taken to have 256 compute units.
    # wide matrices (>= 512 tiles): GEMV for one row only
    assert lutq.plan(1, 14336, 4096, 4)["path"] == "gemv"
    assert lutq.plan(2, 14336, 4096, 4)["path"] == "mfma"
    assert lutq.plan(32, 28672, 8192, 4)["path"] == "mfma"
    # narrow, short K: GEMV up to 4 rows
    assert lutq.plan(4, 4096, 4096, 3)["path"] == "gemv"
    assert lutq.plan(5, 4096, 4096, 3)["path"] == "mfma"
    assert lutq.plan(4, 1024, 4096, 4)["path"] == "gemv"
    assert lutq.plan(8, 1024, 4096, 4)["path"] == "mfma"
    # narrow, long K (>= 8192): GEMV up to 2 rows
    assert lutq.plan(2, 4096, 14336, 3)["path"] == "gemv"
    assert lutq.plan(3, 4096, 14336, 3)["path"] == "mfma"


def test_plan_shapes_and_split():
    # 28672 rows = 1792 tiles = 7 per CU: 7 tiles per wave (one workgroup
    # on every CU) at any MFMA batch, no split.
    assert lutq.plan(32, 28672, 8192, 4) == {"path": "mfma", "ksplit": 1, "tiles": 7}
    assert lutq.plan(16, 28672, 8192, 4)["tiles"] == 7
    assert lutq.plan(2, 28672, 4096, 4)["tiles"] == 7
    # Wider (> 7 tiles per CU): 8 tiles per wave at 32 batch rows, 4 at 16.
    assert lutq.plan(32, 32768, 8192, 4) == {"path": "mfma", "ksplit": 1, "tiles": 8}
    assert lutq.plan(16, 32768, 8192, 4)["tiles"] == 4
    # Exactly 6 tiles per CU keeps the earlier rules: 8 at 32 rows, 4 at 16.
    assert lutq.plan(32, 24576, 8192, 4)["tiles"] == 8
    assert lutq.plan(16, 24576, 8192, 4)["tiles"] == 4
    # GEMV: 2 tiles per wave only when that still gives 2 row blocks per CU
    assert lutq.plan(1, 14336, 4096, 4) == {"path": "gemv", "ksplit": 1, "tiles": 2}
    assert lutq.plan(1, 4096, 4096, 4) == {"path": "gemv", "ksplit": 1, "tiles": 1}
    # GEMV: a short K is never split, however few the row blocks
    assert lutq.plan(1, 1024, 4096, 4) == {"path": "gemv", "ksplit": 1, "tiles": 1}
    # GEMV, long K on fewer row blocks than CUs: split until the CUs are
    # covered, keeping >= 32 chunks per split
    assert lutq.plan(1, 16, 1 << 20, 4)["ksplit"] == 256
    assert lutq.plan(1, 16, 16384, 4)["ksplit"] == 4
    assert lutq.plan(2, 4096, 14336, 3) == {"path": "gemv", "ksplit": 1, "tiles": 1}
    # MFMA, at most one tile per CU on a short K (< 64 chunks): one tile per
    # wave; K split only above 16 batch rows on at most a quarter of the
    # CUs, until half of them are covered (1024 rows = 64 blocks -> 2)
    assert lutq.plan(16, 1024, 4096, 4) == {"path": "mfma", "ksplit": 1, "tiles": 1}
    assert lutq.plan(8, 1024, 4096, 4) == {"path": "mfma", "ksplit": 1, "tiles": 1}
    assert lutq.plan(32, 1024, 4096, 4) == {"path": "mfma", "ksplit": 2, "tiles": 1}
    assert lutq.plan(32, 4096, 4096, 4) == {"path": "mfma", "ksplit": 1, "tiles": 1}
    assert lutq.plan(32, 256, 4096, 4) == {"path": "mfma", "ksplit": 8, "tiles": 1}
    # 257 tiles (more than one per CU) keep two tiles per wave
    assert lutq.plan(8, 4112, 4096, 4)["tiles"] == 2
    # MFMA, 2 tiles: split once the row blocks cover at most half the CUs,
    # from 9 batch rows or on a long K (4096 rows = 128 blocks -> 2)
    assert lutq.plan(4, 4096, 14336, 3) == {"path": "mfma", "ksplit": 2, "tiles": 2}
    assert lutq.plan(16, 4096, 14336, 4) == {"path": "mfma", "ksplit": 2, "tiles": 2}
    assert lutq.plan(32, 14336, 4096, 4) == {"path": "mfma", "ksplit": 1, "tiles": 4}
    # explicit fields are kept (the split is clamped to the chunk count)
    assert lutq.plan(1, 14336, 4096, 4, path="mfma", tiles=8, ksplit=3) == \
        {"path": "mfma", "ksplit": 3, "tiles": 8}
    assert lutq.plan(1, 16, 256, 4, ksplit=100)["ksplit"] == 2
    with pytest.raises(lutq.LutqError):
        lutq.plan(1, 14336, 4096, 4, path="gemv", tiles=8)


# -- the layout as documented in include/lutq.h -------------------------------

def test_layout_hand_example_bits4():
    # one row, K = 128, code k = k % 16. Slot 0 (q = 0, r = 0), k-step j covers
    # k = 32 j + 0..7 -> codes 0..7 -> bytes 0x10 0x32 0x54 0x76.
    codes = (np.arange(128) % 16).astype(np.uint8)[None]
    b = layout_spec.encode(codes, 4)
    assert b.size == 16 * 128 // 2
    assert bytes(b[:16]) == bytes([0x10, 0x32, 0x54, 0x76] * 4)
    # slot 16 (q = 1, r = 0): k = 32 j + 8..15 -> codes 8..15
    assert bytes(b[16 * 16:16 * 16 + 4]) == bytes([0x98, 0xBA, 0xDC, 0xFE])
    # slot 1 (r = 1) is a padding row
    assert not np.any(b[16:32])


def test_layout_hand_example_bits3():
    # one row, K = 128, every code = 5 (binary 101: low bits 01, high bit 1)
    codes = np.full((1, 128), 5, np.uint8)
    w = layout_spec.encode(codes, 3)[:12].view("<u4")
    # low planes: each nibble = 01 | 01 << 2 = 0x5, so every byte 0x55
    assert w[0] == 0x55555555 and w[1] == 0x55555555
    # high pairs (1 | 1 << 1 = 3) at bit offsets 4, 6, 0, 2 of every byte
    assert w[2] == 0xFFFFFFFF
    codes = np.zeros((1, 128), np.uint8)
    codes[0, 32 * 1 + 2] = 4  # k-step j = 1, e = 2 (pair 1, even): high bit at byte 1, bit 6
    w = layout_spec.encode(codes, 3)[:12].view("<u4")
    assert w[0] == 0 and w[1] == 0 and w[2] == 1 << (8 + 6)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (64, 256), (100, 1024)])
def test_layout_encode_decode_roundtrip(bits, N, K):
    from synth import draw
    c = draw.integers((N, K), 1 << bits, (31, bits, N, K))
    b = layout_spec.encode(c, bits)
    assert b.size == -(-N // 16) * 16 * K * bits // 8
    assert np.array_equal(layout_spec.decode(b, N, K, bits), c)
