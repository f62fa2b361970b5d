"""Seeded synthetic inputs for the selective-scan workloads.

This package only generates inputs: it holds none of the scan's arithmetic. The CPU oracle and
the HIP path's tests and bench both take their inputs from here, so both sides see identical
bits. Values come from a counter-based SplitMix64 stream (see ``ssm_gen.c`` for the exact
definition), so any slice of any tensor can be regenerated on its own: the oracle uses that to
check sampled channels of workloads whose full inputs would not fit in host memory twice.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libssmgen.so")

NORMAL, UNIFORM, INV_SOFTPLUS_UNIFORM, NEG_ARANGE = 0, 1, 2, 3
F64, F32, BF16 = 0, 1, 2

TENSOR_IDS = {"x": 1, "delta": 2, "B": 3, "C": 4, "D": 5, "z": 6, "delta_bias": 7, "A": 8,
              "A_imag": 9}
SEED_BASE = 0x53534D5336323400


def build(verbose: bool = False) -> str:
    """Compile the generator with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           os.path.join(_HERE, "ssm_gen.c"), "-o", _SO + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_SO)
        lib.ssmgen_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_int]
        lib.ssmgen_fill.restype = ctypes.c_int
        lib.ssmgen_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.ssmgen_raw.restype = ctypes.c_uint64
        lib.ssmgen_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.ssmgen_f32_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_NP_DTYPE = {F64: np.float64, F32: np.float32, BF16: np.uint16}


def fill(seed: int, tensor_id: int, dist: int, p0: float, p1: float, count: int,
         dtype: int, start: int = 0, nthreads: Optional[int] = None) -> np.ndarray:
    """Values start..start+count of stream (seed, tensor_id), as a 1-D array.

    BF16 results are returned as their uint16 bit patterns.
    """
    out = np.empty(int(count), dtype=_NP_DTYPE[dtype])
    rc = _load().ssmgen_fill(seed & (2**64 - 1), tensor_id, dist, float(p0), float(p1), int(start),
                             int(count), dtype, out.ctypes.data if count else None,
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"ssmgen_fill rejected dist={dist} dtype={dtype} p0={p0}")
    return out


def raw(seed: int, tensor_id: int, i: int) -> int:
    return int(_load().ssmgen_raw(seed & (2**64 - 1), tensor_id, i))


def f32_to_bf16_bits(v: float) -> int:
    return int(_load().ssmgen_f32_to_bf16(float(v)))


@dataclass(frozen=True)
class Dist:
    kind: int
    p0: float = 0.0
    p1: float = 1.0


@dataclass(frozen=True)
class ScanConfig:
    """Shape and input recipe of one scan workload (canonical contiguous layout)."""
    name: str
    batch: int
    dim: int          # channels (d_inner)
    L: int            # sequence length
    N: int            # state size per channel
    ngroups: int = 1  # B/C groups; channel d uses group d // (dim // ngroups)
    headdim: int = 1  # channels per head; >1 with a_mode == "head"
    a_mode: str = "diag"  # "diag": A is (dim, N); "head": one scalar per head; "complex": A is
    #                       (dim, N) complex, stored (dim, N, 2), and B/C hold 2N rows per group
    #                       (real parts, then imaginary parts)
    io: str = "bf16"  # dtype of x, delta, B, C, z and y
    gate: bool = True
    softplus: bool = True
    has_D: bool = True
    has_bias: bool = True
    seed: int = SEED_BASE
    dists: Dict[str, Dist] = field(default_factory=dict)

    @property
    def nheads(self) -> int:
        return self.dim // self.headdim

    @property
    def delta_rows(self) -> int:
        return self.nheads if self.a_mode == "head" else self.dim

    @property
    def io_code(self) -> int:
        return BF16 if self.io == "bf16" else F32

    @property
    def tokch(self) -> int:
        return self.batch * self.dim * self.L

    @property
    def bc_rows(self) -> int:
        return 2 * self.N if self.a_mode == "complex" else self.N

    def shapes(self) -> Dict[str, Tuple[int, ...]]:
        if self.a_mode == "head":
            a_shape = (self.nheads,)
        elif self.a_mode == "complex":
            a_shape = (self.dim, self.N, 2)
        else:
            a_shape = (self.dim, self.N)
        s = {
            "x": (self.batch, self.dim, self.L),
            "delta": (self.batch, self.delta_rows, self.L),
            "A": a_shape,
            "B": (self.batch, self.ngroups, self.bc_rows, self.L),
            "C": (self.batch, self.ngroups, self.bc_rows, self.L),
        }
        if self.has_D:
            s["D"] = (self.dim,)
        if self.gate:
            s["z"] = (self.batch, self.dim, self.L)
        if self.has_bias:
            s["delta_bias"] = (self.delta_rows,)
        return s

    def dtype_of(self, name: str) -> int:
        return F32 if name in ("A", "D", "delta_bias") else self.io_code

    def dist_of(self, name: str) -> Dist:
        if name in self.dists:
            return self.dists[name]
        if name == "delta":
            return Dist(NORMAL, 0.0, 0.5)
        if name == "delta_bias":
            return Dist(INV_SOFTPLUS_UNIFORM, 0.001, 0.1)
        if name == "A":
            if self.a_mode == "complex":  # the real parts
                return Dist(UNIFORM, -0.75, -0.25)
            return Dist(UNIFORM, -16.0, -1.0) if self.a_mode == "head" else Dist(NEG_ARANGE, self.N)
        if name == "A_imag":  # jitter added to pi n
            return Dist(UNIFORM, -0.5, 0.5)
        return Dist(NORMAL, 0.0, 1.0)

    def algorithmic_bytes(self) -> int:
        """Every input read once and y written once (the state is never stored)."""
        total = 0
        for name, shp in self.shapes().items():
            elem = 4 if self.dtype_of(name) == F32 else 2
            total += int(np.prod(shp)) * elem
        total += self.batch * self.dim * self.L * (4 if self.io == "f32" else 2)  # y
        return total


def _cfg(i: int, **kw) -> ScanConfig:
    return ScanConfig(seed=SEED_BASE + i, **kw)


# The five workloads: shapes and distributions from the published Mamba layer shapes.
CONFIGS: Dict[int, ScanConfig] = {
    0: _cfg(0, name="tiny-fp32: batch 1, 64 channels, N 16, L 256", batch=1, dim=64, L=256, N=16,
            io="f32", gate=False),
    1: _cfg(1, name="mamba-130m layer: batch 8, d_inner 1536, N 16, L 2048", batch=8, dim=1536,
            L=2048, N=16),
    2: _cfg(2, name="mamba-1.4b layer: batch 8, d_inner 4096, N 16, L 4096", batch=8, dim=4096,
            L=4096, N=16),
    3: _cfg(3, name="million-token: batch 1, d_inner 2048, N 16, L 1048576", batch=1, dim=2048,
            L=1 << 20, N=16),
    4: _cfg(4, name="scalar-decay heads: batch 4, 64 heads x 64, N 128, L 8192", batch=4,
            dim=4096, L=8192, N=128, headdim=64, a_mode="head"),
}


# Decoding workloads (one step per sequence, L = 1; the state is an extra fp32 input/output).
DECODE_CONFIGS: Dict[str, ScanConfig] = {
    "mamba14b_decode": ScanConfig(name="mamba-1.4b layer decode: batch 1024, d_inner 4096, N 16",
                                  batch=1024, dim=4096, L=1, N=16, seed=SEED_BASE + 16),
    "heads_decode": ScanConfig(name="scalar-decay heads decode: batch 64, 64 heads x 64, N 128",
                               batch=64, dim=4096, L=1, N=128, headdim=64, a_mode="head",
                               seed=SEED_BASE + 17),
}


# The complex-A scan at the Mamba-130M layer's shape (A, B and C complex; delta, x and z real).
COMPLEX_CONFIG = ScanConfig(name="complex-A layer: batch 8, d_inner 1536, N 16, L 2048", batch=8,
                            dim=1536, L=2048, N=16, a_mode="complex", seed=SEED_BASE + 18)


def _complex_a(cfg: ScanConfig, d0: int, d1: int) -> np.ndarray:
    """Rows [d0, d1) of a complex A as (rows, N, 2) float32 (real, imaginary) pairs: real parts
    from the "A" stream, imaginary parts pi n (a linear ladder of frequencies over the states)
    plus jitter from the "A_imag" stream."""
    N, rows = cfg.N, d1 - d0
    dr, di = cfg.dist_of("A"), cfg.dist_of("A_imag")
    re = fill(cfg.seed, TENSOR_IDS["A"], dr.kind, dr.p0, dr.p1, rows * N, F32, d0 * N)
    jit = fill(cfg.seed, TENSOR_IDS["A_imag"], di.kind, di.p0, di.p1, rows * N, F32, d0 * N)
    im = (np.float32(np.pi) * np.arange(N, dtype=np.float32))[None, :] + jit.reshape(rows, N)
    return np.stack([re.reshape(rows, N), im.astype(np.float32)], axis=-1)


def make_tensor(cfg: ScanConfig, name: str, nthreads: Optional[int] = None) -> np.ndarray:
    if name == "A" and cfg.a_mode == "complex":
        return _complex_a(cfg, 0, cfg.dim)
    shp = cfg.shapes()[name]
    d = cfg.dist_of(name)
    arr = fill(cfg.seed, TENSOR_IDS[name], d.kind, d.p0, d.p1, int(np.prod(shp)),
               cfg.dtype_of(name), 0, nthreads)
    return arr.reshape(shp)


def make_inputs(cfg: ScanConfig, nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs of ``cfg`` in canonical layout; bf16 tensors as uint16 bit arrays."""
    return {name: make_tensor(cfg, name, nthreads) for name in cfg.shapes()}


def make_channel(cfg: ScanConfig, b: int, d: int) -> Dict[str, np.ndarray]:
    """Inputs of the single channel (b, d), regenerated from the streams without building the
    full tensors. Shapes are those of a batch-1, dim-1 problem (head mode: headdim 1, one head).
    """
    L, N, R = cfg.L, cfg.N, cfg.bc_rows
    g = d // (cfg.dim // cfg.ngroups)
    row = d // cfg.headdim if cfg.a_mode == "head" else d

    def part(name, start, count, shape):
        dd = cfg.dist_of(name)
        return fill(cfg.seed, TENSOR_IDS[name], dd.kind, dd.p0, dd.p1, count, cfg.dtype_of(name),
                    start).reshape(shape)

    out = {
        "x": part("x", (b * cfg.dim + d) * L, L, (1, 1, L)),
        "delta": part("delta", (b * cfg.delta_rows + row) * L, L, (1, 1, L)),
        "B": part("B", (b * cfg.ngroups + g) * R * L, R * L, (1, 1, R, L)),
        "C": part("C", (b * cfg.ngroups + g) * R * L, R * L, (1, 1, R, L)),
    }
    if cfg.a_mode == "head":
        out["A"] = part("A", row, 1, (1,))
    elif cfg.a_mode == "complex":
        out["A"] = _complex_a(cfg, d, d + 1)
    else:
        out["A"] = part("A", d * N, N, (1, N))
    if cfg.has_D:
        out["D"] = part("D", d, 1, (1,))
    if cfg.gate:
        out["z"] = part("z", (b * cfg.dim + d) * L, L, (1, 1, L))
    if cfg.has_bias:
        out["delta_bias"] = part("delta_bias", row, 1, (1,))
    return out


def make_batch_entry(cfg: ScanConfig, b: int, nthreads: Optional[int] = None
                     ) -> Dict[str, np.ndarray]:
    """Inputs of batch entry ``b`` alone (shapes of the batch-1 problem), regenerated from the
    streams at their offsets; per-channel parameters (A, D, delta_bias) are whole."""
    out = {}
    one = with_shape(cfg, batch=1)
    for name, shp in one.shapes().items():
        if name == "A" and cfg.a_mode == "complex":
            out[name] = _complex_a(cfg, 0, cfg.dim)
            continue
        d = cfg.dist_of(name)
        count = int(np.prod(shp))
        start = b * count if name in ("x", "delta", "B", "C", "z") else 0
        out[name] = fill(cfg.seed, TENSOR_IDS[name], d.kind, d.p0, d.p1, count,
                         cfg.dtype_of(name), start, nthreads).reshape(shp)
    return out


def make_channel_block(cfg: ScanConfig, b: int, d0: int, d1: int,
                       nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of channels [d0, d1) of batch entry ``b`` alone, regenerated from the streams at
    their offsets, as the batch-1 problem of ``block_config(cfg, d0, d1)``. The block must lie
    inside one B/C group and, in head mode, cover whole heads."""
    gsize = cfg.dim // cfg.ngroups
    if not (0 <= d0 < d1 <= cfg.dim) or d0 // gsize != (d1 - 1) // gsize:
        raise ValueError("the channel block must lie inside one B/C group")
    if cfg.a_mode == "head" and (d0 % cfg.headdim or d1 % cfg.headdim):
        raise ValueError("the channel block must cover whole heads")
    L, N, R, nch = cfg.L, cfg.N, cfg.bc_rows, d1 - d0
    g = d0 // gsize
    r0, r1 = (d0 // cfg.headdim, d1 // cfg.headdim) if cfg.a_mode == "head" else (d0, d1)

    def part(name, start, count, shape):
        dd = cfg.dist_of(name)
        return fill(cfg.seed, TENSOR_IDS[name], dd.kind, dd.p0, dd.p1, count, cfg.dtype_of(name),
                    start, nthreads).reshape(shape)

    out = {
        "x": part("x", (b * cfg.dim + d0) * L, nch * L, (1, nch, L)),
        "delta": part("delta", (b * cfg.delta_rows + r0) * L, (r1 - r0) * L, (1, r1 - r0, L)),
        "B": part("B", (b * cfg.ngroups + g) * R * L, R * L, (1, 1, R, L)),
        "C": part("C", (b * cfg.ngroups + g) * R * L, R * L, (1, 1, R, L)),
    }
    if cfg.a_mode == "head":
        out["A"] = part("A", r0, r1 - r0, (r1 - r0,))
    elif cfg.a_mode == "complex":
        out["A"] = _complex_a(cfg, d0, d1)
    else:
        out["A"] = part("A", d0 * N, nch * N, (nch, N))
    if cfg.has_D:
        out["D"] = part("D", d0, nch, (nch,))
    if cfg.gate:
        out["z"] = part("z", (b * cfg.dim + d0) * L, nch * L, (1, nch, L))
    if cfg.has_bias:
        out["delta_bias"] = part("delta_bias", r0, r1 - r0, (r1 - r0,))
    return out


def block_config(cfg: ScanConfig, d0: int, d1: int) -> ScanConfig:
    """The batch-1, one-group problem that ``make_channel_block`` returns."""
    return replace(cfg, batch=1, dim=d1 - d0, ngroups=1)


def with_shape(cfg: ScanConfig, **kw) -> ScanConfig:
    """A copy of ``cfg`` with some fields replaced (same recipe, different sizes)."""
    return replace(cfg, **kw)
