"""Named workloads: shapes, tables, weight distributions and seeds.

Shapes are (N, K) = (out, in) of Llama-3-8B / Llama-70B linear layers; the
source pages quantize LLaMA3 and Qwen3 checkpoints that are not available
here, so synthetic weights of those shapes and distributions stand in for
them.

Seeds: weights ``(workload_id, matrix_id, 0)``, activations
``(workload_id, matrix_id, 1, M)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import draw, rtn, tables


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int
    K: int


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    bits: int
    table: str          # int | nf | lloyd_max | log
    group: int          # 0 = one scale per tensor
    dist: str
    dist_kw: dict = field(default_factory=dict)
    matrices: tuple = ()
    batches: tuple = (1,)
    table_kw: dict = field(default_factory=dict)

    @property
    def scale_rule(self) -> str:
        return "int" if self.table == "int" else "absmax"

    def matrix(self, name: str | None = None) -> tuple[int, Matrix]:
        if name is None:
            return 0, self.matrices[0]
        for i, m in enumerate(self.matrices):
            if m.name == name:
                return i, m
        raise KeyError(name)


WORKLOADS = {
    w.name: w
    for w in (
        Workload(1, "nf4_1k", 4, "nf", 128, "normal", {"sigma": 0.02},
                 (Matrix("w", 1024, 1024),), (1,)),
        Workload(2, "int4_up_proj", 4, "int", 128, "normal_outliers",
                 {"sigma": 0.02, "p": 1e-3, "mult": 10.0},
                 (Matrix("up", 14336, 4096),), (1,)),
        Workload(3, "lm3", 3, "lloyd_max", 128, "student_t", {"nu": 4.0, "scale": 0.02},
                 (Matrix("sq", 4096, 4096), Matrix("wide", 4096, 14336)), (1, 4, 8)),
        Workload(4, "log4_70b", 4, "log", 0, "laplace", {"b": 0.015},
                 (Matrix("up", 28672, 8192),), (1, 8, 32), {"base": math.sqrt(2.0)}),
        Workload(5, "nf4_layer", 4, "nf", 128, "normal", {"sigma": 0.02},
                 (Matrix("q", 4096, 4096), Matrix("k", 1024, 4096), Matrix("v", 1024, 4096),
                  Matrix("o", 4096, 4096), Matrix("gate", 14336, 4096),
                  Matrix("up", 14336, 4096), Matrix("down", 4096, 14336)),
                 (1, 8, 16, 32)),
    )
}


def lut(w: Workload) -> np.ndarray:
    return tables.make(w.table, w.bits, **w.table_kw)


def weights(w: Workload, mat: str | None = None) -> np.ndarray:
    mi, m = w.matrix(mat)
    return draw.weights(w.dist, m.N, m.K, (w.wid, mi, 0), **w.dist_kw)


def activations(w: Workload, M: int, mat: str | None = None) -> np.ndarray:
    mi, m = w.matrix(mat)
    return draw.activations(M, m.K, (w.wid, mi, 1, M))


def quantized(w: Workload, mat: str | None = None):
    """(codes u8 [N,K], lut fp16, scales fp16) for one matrix of a workload."""
    T = lut(w)
    W = weights(w, mat)
    c, s = rtn.quantize(W, T, w.group, w.scale_rule)
    return c, T, s


def small_case(bits: int, table: str, group: int, M: int, N: int, K: int, seed: int,
               dist: str = "normal", **dist_kw):
    """A small seeded case (codes, lut, scales, x) for parity tests."""
    T = tables.make(table, bits)
    W = draw.weights(dist, N, K, (100, seed, 0), **(dist_kw or {"sigma": 0.02}))
    rule = "int" if table == "int" else "absmax"
    c, s = rtn.quantize(W, T, group, rule)
    x = draw.activations(M, K, (100, seed, 1, M))
    return c, T, s, x
