"""ctypes binding of liblutq.so (argument marshalling only).

Every function here forwards to the C entry point of the same name; tensors
are passed as raw device pointers and the stream is PyTorch's current one.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))

PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2
_PATHS = {"auto": PATH_AUTO, "gemv": PATH_GEMV, "mfma": PATH_MFMA}

LUTQ_MAGIC = 0x5154554C
LUTQ_LAYOUT_VERSION = 1

# every symbol include/lutq.h declares
EXPORTS = (
    "lutq_packed_bytes", "lutq_repack", "lutq_unpack", "lutq_matmul", "lutq_matmul_ex",
    "lutq_plan", "lutq_strerror", "lutq_last_hip_error", "lutq_shutdown",
    "lutq_quantize", "lutq_quant_error", "lutq_log_base_search", "lutq_matmul_multi",
    "lutq_matmul_zp", "lutq_matmul_typed", "lutq_matmul_bcq",
    "lutq_quantize_ex", "lutq_quant_error_ex", "lutq_log_base_search_ex", "lutq_tune_table",
    "lutq_matmul_noalloc",
    # include/lutq_peaks.h
    "lutq_peak_empty", "lutq_peak_stream_sink_bytes", "lutq_peak_stream", "lutq_peak_mfma",
    "lutq_peak_lds",
)

MAX_TYPES = 4

MAX_FUSED = 4

RULE_ABSMAX, RULE_RANGE = 0, 1
_RULES = {"absmax": RULE_ABSMAX, "range": RULE_RANGE}


class PackedDesc(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
        ("nbytes", ctypes.c_uint64), ("data", ctypes.c_void_p),
    ]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("ksplit", ctypes.c_int32),
                ("tiles", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 4)]


class MatmulItem(ctypes.Structure):
    _fields_ = [("packed", ctypes.POINTER(PackedDesc)), ("lut", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class LutqError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        msg = strerror(code)
        if code == -7:  # LUTQ_EHIP
            msg += f" (hipError {_lib().lutq_last_hip_error()})"
        super().__init__(f"{where}: lutq error {code}: {msg}" if where else f"lutq error {code}: {msg}")


_LIB = None


def library_path() -> str:
    return os.environ.get("LUTQ_LIBRARY", os.path.join(HERE, "liblutq.so"))


def load_library():
    """Load liblutq.so (built by ``weight_only_lut_amd.build``); raise if missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m weight_only_lut_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.lutq_packed_bytes.argtypes = [i32, i32, i32, i32]
    lib.lutq_packed_bytes.restype = sz
    lib.lutq_repack.argtypes = [vp, i32, i32, i32, i32, vp, sz, ctypes.POINTER(PackedDesc), vp]
    lib.lutq_repack.restype = i32
    lib.lutq_unpack.argtypes = [ctypes.POINTER(PackedDesc), vp, vp]
    lib.lutq_unpack.restype = i32
    lib.lutq_matmul.argtypes = [vp, ctypes.POINTER(PackedDesc), vp, vp, vp, i32, i32, i32, vp]
    lib.lutq_matmul.restype = i32
    lib.lutq_matmul_ex.argtypes = [vp, ctypes.POINTER(PackedDesc), vp, vp, vp, i32, i32, i32,
                                   ctypes.POINTER(Options), vp]
    lib.lutq_matmul_ex.restype = i32
    lib.lutq_matmul_noalloc.argtypes = [vp, ctypes.POINTER(PackedDesc), vp, vp, vp, i32, i32, i32,
                                        ctypes.POINTER(Options), vp]
    lib.lutq_matmul_noalloc.restype = i32
    lib.lutq_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(Options), ctypes.POINTER(Options)]
    lib.lutq_matmul_multi.argtypes = [vp, ctypes.POINTER(MatmulItem), i32, i32, i32,
                                      ctypes.POINTER(Options), vp]
    lib.lutq_matmul_multi.restype = i32
    lib.lutq_matmul_zp.argtypes = [vp, ctypes.POINTER(PackedDesc), vp, vp, vp, vp, i32, i32, i32,
                                   ctypes.POINTER(Options), vp]
    lib.lutq_matmul_zp.restype = i32
    lib.lutq_matmul_typed.argtypes = [vp, ctypes.POINTER(PackedDesc), vp, i32, vp, vp, vp, vp, i32,
                                      i32, i32, ctypes.POINTER(Options), vp]
    lib.lutq_matmul_typed.restype = i32
    lib.lutq_matmul_bcq.argtypes = [vp, ctypes.POINTER(PackedDesc), vp, vp, i32, i32, i32,
                                    ctypes.POINTER(Options), vp]
    lib.lutq_matmul_bcq.restype = i32
    lib.lutq_quantize_ex.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.lutq_quantize_ex.restype = i32
    lib.lutq_quant_error_ex.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32,
                                        ctypes.POINTER(ctypes.c_double), vp]
    lib.lutq_quant_error_ex.restype = i32
    lib.lutq_log_base_search_ex.argtypes = [vp, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(ctypes.c_double), i32,
                                            ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_double), vp]
    lib.lutq_log_base_search_ex.restype = i32
    lib.lutq_tune_table.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, vp,
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32), vp]
    lib.lutq_tune_table.restype = i32
    lib.lutq_plan.restype = i32
    lib.lutq_strerror.argtypes = [i32]
    lib.lutq_strerror.restype = ctypes.c_char_p
    lib.lutq_last_hip_error.argtypes = []
    lib.lutq_last_hip_error.restype = i32
    lib.lutq_shutdown.argtypes = []
    lib.lutq_shutdown.restype = None
    lib.lutq_quantize.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.lutq_quantize.restype = i32
    lib.lutq_quant_error.argtypes = [vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_double), vp]
    lib.lutq_quant_error.restype = i32
    lib.lutq_log_base_search.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_double), i32,
                                         ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double), vp]
    lib.lutq_log_base_search.restype = i32
    lib.lutq_peak_empty.argtypes = [vp]
    lib.lutq_peak_empty.restype = i32
    lib.lutq_peak_stream_sink_bytes.argtypes = []
    lib.lutq_peak_stream_sink_bytes.restype = sz
    lib.lutq_peak_stream.argtypes = [vp, sz, i32, vp, vp]
    lib.lutq_peak_stream.restype = i32
    lib.lutq_peak_mfma.argtypes = [i32, i32, i32, vp, vp]
    lib.lutq_peak_mfma.restype = i32
    lib.lutq_peak_lds.argtypes = [i32, i32, vp, vp]
    lib.lutq_peak_lds.restype = i32
    _LIB = lib
    return lib


def _lib():
    return load_library()


def strerror(code: int) -> str:
    return _lib().lutq_strerror(code).decode()


def packed_bytes(N: int, K: int, bits: int, group: int) -> int:
    return int(_lib().lutq_packed_bytes(N, K, bits, group))


DTYPE_F16, DTYPE_BF16 = 0, 1


def _options(path: str, ksplit: int, tiles: int, dtype: int = DTYPE_F16) -> Options:
    o = Options()
    o.path = _PATHS[path]
    o.ksplit = ksplit
    o.tiles = tiles
    o.dtype = dtype
    return o


def _act_dtype(x):
    """(torch dtype, lutq dtype) of fp16 or bf16 activations."""
    import torch
    if isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16:
        return torch.bfloat16, DTYPE_BF16
    return torch.float16, DTYPE_F16


def plan(M: int, N: int, K: int, bits: int, *, path: str = "auto", ksplit: int = 0,
         tiles: int = 0) -> dict:
    """lutq_plan: the options lutq_matmul_ex resolves for this call, as
    {"path": "gemv" | "mfma", "ksplit": int, "tiles": int}."""
    req, out = _options(path, ksplit, tiles), Options()
    rc = _lib().lutq_plan(M, N, K, bits, ctypes.byref(req), ctypes.byref(out))
    if rc:
        raise LutqError(rc, "lutq_plan")
    return {"path": {1: "gemv", 2: "mfma"}[out.path], "ksplit": out.ksplit, "tiles": out.tiles}


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check(t, name, dtype, shape=None, numel=None):
    """Type, dtype, contiguity and size of one tensor argument (no device
    check: see _on_device). ``shape`` is the exact shape, ``numel`` the exact
    element count, either may be None."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and numel > 0 and t.numel() != numel:   # 0: nothing is read
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _on_device(*tensors):
    """Every tensor is a CUDA (HIP) tensor on the device of the first."""
    dev = None
    for name, t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


def _need_cuda(t, name, dtype):
    _check(t, name, dtype)
    _on_device((name, t))


def _groups(p) -> int:
    """Scale-like entries per matrix: N * K / group, or 1 for one scale per
    tensor; 0 for an empty matrix (nothing is read)."""
    if p.N == 0 or p.K == 0:
        return 0
    return p.N * (p.K // p.group) if p.group else 1


class Packed:
    """Packed weights: the device buffer plus its host descriptor."""

    def __init__(self, data, desc: PackedDesc):
        self.data = data          # torch uint8 tensor owning the device bytes
        self.desc = desc

    N = property(lambda self: self.desc.N)
    K = property(lambda self: self.desc.K)
    bits = property(lambda self: self.desc.bits)
    group = property(lambda self: self.desc.group)
    nbytes = property(lambda self: self.desc.nbytes)


def repack(codes, bits: int, group: int) -> Packed:
    """lutq_repack: uint8 codes [N, K] on the GPU -> Packed (wave-block layout)."""
    import torch
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise ValueError("codes must be a 2-D tensor [N, K]")
    _need_cuda(codes, "codes", torch.uint8)
    N, K = codes.shape
    nbytes = packed_bytes(N, K, bits, group)
    dst = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    desc = PackedDesc()
    rc = _lib().lutq_repack(_ptr(codes), N, K, bits, group, _ptr(dst), dst.numel(),
                            ctypes.byref(desc), _stream(codes.device))
    if rc:
        raise LutqError(rc, "lutq_repack")
    return Packed(dst, desc)


def unpack(p: Packed):
    """lutq_unpack: Packed -> uint8 codes [N, K] on the GPU."""
    import torch
    out = torch.empty((p.N, p.K), dtype=torch.uint8, device=p.data.device)
    rc = _lib().lutq_unpack(ctypes.byref(p.desc), _ptr(out), _stream(p.data.device))
    if rc:
        raise LutqError(rc, "lutq_unpack")
    return out


def matmul(x, p: Packed, lut, scales, *, zeros=None, types=None, path: str = "auto",
           ksplit: int = 0, tiles: int = 0, out=None):
    """lutq_matmul_ex (lutq_matmul_zp with ``zeros``; lutq_matmul_typed with
    ``types``, uint8 [N, K/group], and ``lut`` fp16 [ntypes, 2^bits]):
    y[M, N] = x[M, K] . dequant(p, lut, scales[, zeros][, types])^T, fp16 out."""
    import torch
    tdt, ldt = _act_dtype(x)
    if not isinstance(p, Packed):
        raise TypeError("p must be a Packed (from repack)")
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [M, K]")
    M, K = x.shape
    _check(x, "x", tdt, shape=(M, p.K))
    L = 1 << p.bits
    if types is not None:
        _check(lut, "lut", torch.float16)
        nt = lut.shape[0] if lut.dim() == 2 else 1
        if lut.numel() != nt * L or not 1 <= nt <= MAX_TYPES:
            raise ValueError(f"lut must be [ntypes, {L}] with 1 <= ntypes <= {MAX_TYPES}")
        _check(types, "types", torch.uint8, numel=_groups(p))
    else:
        _check(lut, "lut", torch.float16, numel=L)
    _check(scales, "scales", torch.float16, numel=_groups(p))
    if zeros is not None:
        _check(zeros, "zeros", torch.float16, numel=_groups(p))
    if out is not None:
        _check(out, "out", tdt, shape=(M, p.N))
    _on_device(("x", x), ("packed data", p.data), ("lut", lut), ("scales", scales),
               ("zeros", zeros), ("types", types), ("out", out))
    if out is None:
        out = torch.empty((M, p.N), dtype=tdt, device=x.device)
    opts = _options(path, ksplit, tiles, ldt)
    if types is not None:
        rc = _lib().lutq_matmul_typed(_ptr(x), ctypes.byref(p.desc), _ptr(lut), nt, _ptr(types),
                                      _ptr(scales), _ptr(zeros), _ptr(out), M, p.N, K,
                                      ctypes.byref(opts), _stream(x.device))
    elif zeros is None:
        rc = _lib().lutq_matmul_ex(_ptr(x), ctypes.byref(p.desc), _ptr(lut), _ptr(scales),
                                   _ptr(out), M, p.N, K, ctypes.byref(opts), _stream(x.device))
    else:
        rc = _lib().lutq_matmul_zp(_ptr(x), ctypes.byref(p.desc), _ptr(lut), _ptr(scales),
                                   _ptr(zeros), _ptr(out), M, p.N, K, ctypes.byref(opts),
                                   _stream(x.device))
    if rc:
        raise LutqError(rc, "lutq_matmul")
    return out


def matmul_noalloc(x, p: Packed, lut, scales, *, path: str = "auto", ksplit: int = 0,
                   tiles: int = 0, out=None):
    """lutq_matmul_noalloc: lutq_matmul_ex with its split-K scratch in the
    library's fixed per-GPU array (no device allocation by the library);
    bit-identical to ``matmul`` with the same options."""
    import torch
    tdt, ldt = _act_dtype(x)
    if not isinstance(p, Packed):
        raise TypeError("p must be a Packed (from repack)")
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [M, K]")
    M, K = x.shape
    _check(x, "x", tdt, shape=(M, p.K))
    _check(lut, "lut", torch.float16, numel=1 << p.bits)
    _check(scales, "scales", torch.float16, numel=_groups(p))
    if out is not None:
        _check(out, "out", tdt, shape=(M, p.N))
    _on_device(("x", x), ("packed data", p.data), ("lut", lut), ("scales", scales), ("out", out))
    if out is None:
        out = torch.empty((M, p.N), dtype=tdt, device=x.device)
    opts = _options(path, ksplit, tiles, ldt)
    rc = _lib().lutq_matmul_noalloc(_ptr(x), ctypes.byref(p.desc), _ptr(lut), _ptr(scales), _ptr(out),
                                    M, p.N, K, ctypes.byref(opts), _stream(x.device))
    if rc:
        raise LutqError(rc, "lutq_matmul_noalloc")
    return out


def matmul_multi(x, mats, *, path: str = "auto", ksplit: int = 0, tiles: int = 0, outs=None):
    """lutq_matmul_multi: one fused launch (per batch slice) for several
    matrices sharing x: ``mats`` is a list of (Packed, lut, scales) or
    (Packed, lut, scales, zeros); returns the list of fp16 outputs y_i [M, N_i]."""
    import torch
    tdt, ldt = _act_dtype(x)
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [M, K]")
    M, K = x.shape
    _check(x, "x", tdt)
    if not 1 <= len(mats) <= MAX_FUSED:
        raise ValueError(f"1 to {MAX_FUSED} matrices per fused launch")
    if outs is not None and len(outs) != len(mats):
        raise ValueError("one output per matrix")
    items = (MatmulItem * len(mats))()
    ys = []
    args = []
    for i, mat in enumerate(mats):       # shapes and sizes of every matrix first
        p, lut, scales = mat[:3]
        zeros = mat[3] if len(mat) > 3 else None
        if not isinstance(p, Packed):
            raise TypeError(f"matrix {i}: the first entry must be a Packed (from repack)")
        if p.K != K:
            raise ValueError(f"matrix {i} has K = {p.K}, x has K = {K}")
        _check(lut, f"lut[{i}]", torch.float16, numel=1 << p.bits)
        _check(scales, f"scales[{i}]", torch.float16, numel=_groups(p))
        if zeros is not None:
            _check(zeros, f"zeros[{i}]", torch.float16, numel=_groups(p))
        y = None if outs is None else outs[i]
        if y is not None:
            _check(y, f"out[{i}]", tdt, shape=(M, p.N))
        args.append((p, lut, scales, zeros, y))
    for i, (p, lut, scales, zeros, y) in enumerate(args):
        _on_device(("x", x), (f"packed data[{i}]", p.data), (f"lut[{i}]", lut),
                   (f"scales[{i}]", scales), (f"zeros[{i}]", zeros), (f"out[{i}]", y))
        if zeros is not None:
            items[i].zeros = zeros.data_ptr()
        if y is None:
            y = torch.empty((M, p.N), dtype=tdt, device=x.device)
        ys.append(y)
        items[i].packed = ctypes.pointer(p.desc)
        items[i].lut, items[i].scales, items[i].y = lut.data_ptr(), scales.data_ptr(), y.data_ptr()
    opts = _options(path, ksplit, tiles, ldt)
    rc = _lib().lutq_matmul_multi(_ptr(x), items, len(mats), M, K, ctypes.byref(opts),
                                  _stream(x.device))
    if rc:
        raise LutqError(rc, "lutq_matmul_multi")
    return ys


def matmul_bcq(x, p: Packed, alphas, *, path: str = "auto", ksplit: int = 0, tiles: int = 0,
               out=None):
    """lutq_matmul_bcq: binary-coded weights (p packed with bits = q planes,
    alphas fp16 [q, N, K/group]) -> y[M, N] fp16."""
    import torch
    if not isinstance(p, Packed):
        raise TypeError("p must be a Packed (from repack)")
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [M, K]")
    M, K = x.shape
    _check(x, "x", torch.float16, shape=(M, p.K))
    _check(alphas, "alphas", torch.float16, numel=p.bits * _groups(p))
    if out is not None:
        _check(out, "out", torch.float16, shape=(M, p.N))
    _on_device(("x", x), ("packed data", p.data), ("alphas", alphas), ("out", out))
    if out is None:
        out = torch.empty((M, p.N), dtype=torch.float16, device=x.device)
    opts = _options(path, ksplit, tiles)
    rc = _lib().lutq_matmul_bcq(_ptr(x), ctypes.byref(p.desc), _ptr(alphas), _ptr(out), M, p.N, K,
                                ctypes.byref(opts), _stream(x.device))
    if rc:
        raise LutqError(rc, "lutq_matmul_bcq")
    return out


WEIGHT_F32, WEIGHT_F16, WEIGHT_BF16 = 0, 1, 2


def _weight_dtype(w) -> int:
    """The LUTQ_WEIGHT_* value of a weight tensor (fp32, fp16 or bf16 [N, K] on the GPU)."""
    import torch
    codes = {torch.float32: WEIGHT_F32, torch.float16: WEIGHT_F16, torch.bfloat16: WEIGHT_BF16}
    if not isinstance(w, torch.Tensor) or w.dtype not in codes:
        raise TypeError("w must be a float32, float16 or bfloat16 tensor")
    if w.dim() != 2:
        raise ValueError("w must be a 2-D tensor [N, K]")
    _check(w, "w", w.dtype)
    return codes[w.dtype]


def quantize(w, lut, bits: int, group: int, rule: str = "absmax"):
    """lutq_quantize_ex: fp32, fp16 or bf16 weights [N, K] -> (uint8 codes [N, K], fp16 scales
    [N, K/group] or [1]), round-to-nearest onto the table ``lut``."""
    import torch
    wdt = _weight_dtype(w)
    _check(lut, "lut", torch.float16, numel=1 << bits)
    _on_device(("w", w), ("lut", lut))
    N, K = w.shape
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // group) if group else (1,), dtype=torch.float16, device=w.device)
    rc = _lib().lutq_quantize_ex(_ptr(w), wdt, _ptr(lut), bits, N, K, group, _RULES[rule], _ptr(codes),
                              _ptr(scales), _stream(w.device))
    if rc:
        raise LutqError(rc, "lutq_quantize")
    return codes, scales


def quant_error(w, lut, bits: int, group: int, rule: str = "absmax") -> float:
    """lutq_quant_error: sum (w - s * T[c])^2 (fp64) of that quantization."""
    import torch
    wdt = _weight_dtype(w)
    _check(lut, "lut", torch.float16, numel=1 << bits)
    _on_device(("w", w), ("lut", lut))
    N, K = w.shape
    err = ctypes.c_double(0.0)
    rc = _lib().lutq_quant_error_ex(_ptr(w), wdt, _ptr(lut), bits, N, K, group, _RULES[rule],
                                 ctypes.byref(err), _stream(w.device))
    if rc:
        raise LutqError(rc, "lutq_quant_error")
    return err.value


def log_base_search(w, bits: int, group: int, bases):
    """lutq_log_base_search: (index of the best base, [error of each base])."""
    wdt = _weight_dtype(w)
    _on_device(("w", w))
    N, K = w.shape
    nb = len(bases)
    arr = (ctypes.c_double * nb)(*[float(b) for b in bases])
    errs = (ctypes.c_double * nb)()
    best = ctypes.c_int32(-1)
    rc = _lib().lutq_log_base_search_ex(_ptr(w), wdt, bits, N, K, group, arr, nb, ctypes.byref(best),
                                     errs, _stream(w.device))
    if rc:
        raise LutqError(rc, "lutq_log_base_search")
    return best.value, list(errs)


def tune_table(w, lut, bits: int, group: int, rule: str = "absmax", iters: int = 10):
    """lutq_tune_table: Lloyd iterations on the weight error with fixed scales.
    Returns (tuned table fp16 [2^bits], fixed scales fp16, [error of each table])."""
    import torch
    wdt = _weight_dtype(w)
    _check(lut, "lut", torch.float16, numel=1 << bits)
    _on_device(("w", w), ("lut", lut))
    N, K = w.shape
    T = lut.clone()
    scales = torch.empty((N, K // group) if group else (1,), dtype=torch.float16, device=w.device)
    errs = (ctypes.c_double * (iters + 1))()
    upd = ctypes.c_int32(0)
    rc = _lib().lutq_tune_table(_ptr(w), wdt, _ptr(T), bits, N, K, group, _RULES[rule], iters,
                                _ptr(scales), errs, ctypes.byref(upd), _stream(w.device))
    if rc:
        raise LutqError(rc, "lutq_tune_table")
    return T, scales, list(errs)[: upd.value + 1]


# ---- peak microbenchmarks (include/lutq_peaks.h) ------------------------------

PEAK_MFMA_16X16X32, PEAK_MFMA_32X32X16 = 0, 1
PEAK_MFMA_FLOPS_PER_ROUND = 131072   # per wave and round, either kind


def _peak_rc(rc, where):
    if rc:
        raise LutqError(rc, where)


def peak_empty():
    """lutq_peak_empty on the current stream."""
    import torch
    _peak_rc(_lib().lutq_peak_empty(_stream(torch.cuda.current_device())), "lutq_peak_empty")


def peak_stream_sink_bytes() -> int:
    return int(_lib().lutq_peak_stream_sink_bytes())


def peak_stream(buf, nbytes: int, store: bool, sink):
    """lutq_peak_stream: read ``nbytes`` of the uint8 device tensor ``buf``."""
    import torch
    _check(buf, "buf", torch.uint8)
    _check(sink, "sink", torch.uint8)
    _on_device(("buf", buf), ("sink", sink))
    if nbytes > buf.numel() or sink.numel() < peak_stream_sink_bytes():
        raise ValueError("buffer or sink too small")
    _peak_rc(_lib().lutq_peak_stream(_ptr(buf), nbytes, int(bool(store)), _ptr(sink),
                                     _stream(buf.device)), "lutq_peak_stream")


def peak_mfma(kind: int, waves_per_simd: int, iters: int, sink):
    """lutq_peak_mfma: ``sink`` fp32, at least CUs * 16 entries."""
    import torch
    _check(sink, "sink", torch.float32)
    _on_device(("sink", sink))
    _peak_rc(_lib().lutq_peak_mfma(kind, waves_per_simd, iters, _ptr(sink), _stream(sink.device)),
             "lutq_peak_mfma")


def peak_lds(waves_per_cu: int, iters: int, sink):
    """lutq_peak_lds: ``sink`` int32 (one entry used)."""
    import torch
    _check(sink, "sink", torch.int32)
    _on_device(("sink", sink))
    _peak_rc(_lib().lutq_peak_lds(waves_per_cu, iters, _ptr(sink), _stream(sink.device)),
             "lutq_peak_lds")
