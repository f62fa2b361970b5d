"""CPU oracle for the selective-scan forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg may import this
package. It shares no code with the HIP path (``selective_state_space_24_amd``) and never imports
it. The arithmetic lives in ``ssm_oracle.c`` (plain fp64, sequential over time, one channel per
task); this module only converts arrays to fp64 and calls it.

Pinned by the CPU tests (closed-form geometric series, B = 0 skip path, brute-force
semiseparable matrix, LTI convolution kernel, Theorem 1 gated-RNN form, linearity, causality,
segment composition, head-mode broadcast, the A = 0 and large-step limits; for the complex-A
scan: the real reduction, a closed form in Python's cmath, a rotating phasor, the materialised
semiseparable matrix and conjugation symmetry). Nothing here is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple, Union

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libssm_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc: -O2, IEEE semantics (no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math",
           "-ffp-contract=off", os.path.join(_HERE, "ssm_oracle.c"), "-o", _SO + ".tmp", "-lm",
           "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def load_library(path: str):
    """ctypes handle of an oracle build at ``path`` (the tests also load mutated copies)."""
    lib = ctypes.CDLL(path)
    i64, ci = ctypes.c_int64, ctypes.c_int
    lib.ssm_oracle_scan.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci, ci] + [_dp] * 11 + [ci]
    lib.ssm_oracle_scan.restype = ci
    lib.ssm_oracle_scan_bwd.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci, ci] + [_dp] * 20 + [ci]
    lib.ssm_oracle_scan_bwd.restype = ci
    lib.ssm_oracle_scan_complex.argtypes = [i64, i64, i64, i64, i64, ci] + [_dp] * 12 + [ci]
    lib.ssm_oracle_scan_complex.restype = ci
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is not built; run __graft_entry__.build() first")
        _lib = load_library(_SO)
    return _lib


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(a) -> Optional[np.ndarray]:
    """float32/float64 arrays as float64; uint16 arrays are read as bf16 bit patterns."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return a.ctypes.data_as(_dp) if a is not None else None


def cpu_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def selective_scan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, *,
                   headdim: int = 1, head_mode: bool = False, zoh: bool = False, h0=None,
                   return_final_state: bool = False, nthreads: Optional[int] = None, lib=None
                   ) -> Union[np.ndarray, Tuple[np.ndarray, np.ndarray]]:
    """fp64 selective scan. Shapes (L contiguous):

    x, z: (batch, dim, L); delta: (batch, dim, L), or (batch, nheads, L) in head mode;
    A: (dim, N), or (nheads,) in head mode; B, C: (batch, ngroups, N, L); D: (dim,);
    delta_bias: (dim,) or (nheads,); h0: (batch, dim, N).
    Returns y (batch, dim, L) as float64 [and the final state (batch, dim, N)].
    """
    x, delta, A, B, C = (as_f64(t) for t in (x, delta, A, B, C))
    D, z, delta_bias, h0 = (as_f64(t) for t in (D, z, delta_bias, h0))
    batch, dim, L = x.shape
    _, ngroups, N, L2 = B.shape
    if L2 != L or C.shape != B.shape:
        raise ValueError("B/C shape mismatch")
    nheads = dim // headdim
    if head_mode:
        assert A.shape == (nheads,) and delta.shape == (batch, nheads, L)
    else:
        assert A.shape == (dim, N) and delta.shape == (batch, dim, L)
    y = np.empty((batch, dim, L), dtype=np.float64)
    hT = np.empty((batch, dim, N), dtype=np.float64) if return_final_state else None
    rc = (lib or _load()).ssm_oracle_scan(batch, dim, L, N, ngroups, headdim, int(head_mode),
                                 int(bool(delta_softplus)), int(zoh), _ptr(x), _ptr(delta),
                                 _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                 _ptr(h0), _ptr(y), _ptr(hT), nthreads or cpu_threads())
    if rc != 0:
        raise ValueError("oracle rejected the problem sizes")
    return (y, hT) if return_final_state else y


def selective_scan_bwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                       dy=None, *, headdim: int = 1, head_mode: bool = False, zoh: bool = False,
                       h0=None, dh_final=None, want_dh0: bool = False,
                       nthreads: Optional[int] = None, lib=None) -> dict:
    """fp64 gradients of ``selective_scan`` with respect to every input, given ``dy`` (the
    gradient of y, shaped like x) and optionally ``dh_final`` (the gradient of the final state,
    (batch, dim, N)). Returns a dict with dx, ddelta, dA, dB, dC, and dD, dz, ddelta_bias for the
    optional inputs that were given, and dh0 when h0 was given or ``want_dh0``."""
    x, delta, A, B, C = (as_f64(t) for t in (x, delta, A, B, C))
    D, z, delta_bias, h0, dy = (as_f64(t) for t in (D, z, delta_bias, h0, dy))
    dh_final = as_f64(dh_final)
    batch, dim, L = x.shape
    _, ngroups, N, _ = B.shape
    out = {"dx": np.empty_like(x), "ddelta": np.empty_like(delta), "dA": np.empty_like(A),
           "dB": np.empty_like(B), "dC": np.empty_like(C)}
    if D is not None:
        out["dD"] = np.empty_like(D)
    if z is not None:
        out["dz"] = np.empty_like(z)
    if delta_bias is not None:
        out["ddelta_bias"] = np.empty_like(delta_bias)
    if h0 is not None or want_dh0:
        out["dh0"] = np.empty((batch, dim, N), dtype=np.float64)
    rc = (lib or _load()).ssm_oracle_scan_bwd(
        batch, dim, L, N, ngroups, headdim, int(head_mode), int(bool(delta_softplus)), int(zoh),
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")), _ptr(out.get("dz")),
        _ptr(out.get("ddelta_bias")), _ptr(out.get("dh0")), nthreads or cpu_threads())
    if rc != 0:
        raise ValueError("oracle backward rejected the problem sizes")
    return out


def selective_scan_complex(x, delta, A, B, C, D=None, z=None, delta_bias=None,
                           delta_softplus=True, *, nthreads=None, lib=None):
    """y of the complex-A scan (ssm_oracle.c, complex section): A complex (dim, N); B, C
    complex (batch, ngroups, N, L); x, delta, z real (batch, dim, L); D, delta_bias (dim,)."""
    lib = lib or _load()
    x, delta = as_f64(x), as_f64(delta)
    A, B, C = (np.ascontiguousarray(np.asarray(v, dtype=np.complex128)) for v in (A, B, C))
    batch, dim, L = x.shape
    ngroups, N = B.shape[1], B.shape[2]
    parts = [np.ascontiguousarray(v) for v in (A.real, A.imag, B.real, B.imag, C.real, C.imag)]
    D, z, delta_bias = as_f64(D), as_f64(z), as_f64(delta_bias)
    y = np.empty((batch, dim, L), dtype=np.float64)
    rc = lib.ssm_oracle_scan_complex(batch, dim, L, N, ngroups, int(bool(delta_softplus)),
                                     _ptr(x), _ptr(delta), *[_ptr(v) for v in parts], _ptr(D),
                                     _ptr(z), _ptr(delta_bias), _ptr(y),
                                     nthreads or cpu_threads())
    if rc != 0:
        raise ValueError(f"ssm_oracle_scan_complex: bad sizes (rc {rc})")
    return y


def scan_inputs_complex(inputs: dict, cfg=None, **kw):
    """``selective_scan_complex`` on a dict of generated inputs in the library's layout: A as
    (dim, N, 2) (real, imaginary) pairs, B and C as (batch, ngroups, 2N, L) with the real parts
    in rows 0..N-1 and the imaginary parts in rows N..2N-1."""
    if cfg is not None:
        kw.setdefault("delta_softplus", cfg.softplus)
    A = np.asarray(inputs["A"], dtype=np.float64)
    A = A[..., 0] + 1j * A[..., 1]
    N = A.shape[1]
    B, C = as_f64(inputs["B"]), as_f64(inputs["C"])
    B = B[:, :, :N] + 1j * B[:, :, N:]
    C = C[:, :, :N] + 1j * C[:, :, N:]
    return selective_scan_complex(inputs["x"], inputs["delta"], A, B, C, inputs.get("D"),
                                  inputs.get("z"), inputs.get("delta_bias"), **kw)


def scan_inputs_bwd(inputs: dict, dy, cfg=None, **kw) -> dict:
    """``selective_scan_bwd`` on a dict of generated inputs."""
    if cfg is not None:
        kw.setdefault("headdim", cfg.headdim)
        kw.setdefault("head_mode", cfg.a_mode == "head")
        kw.setdefault("delta_softplus", cfg.softplus)
    return selective_scan_bwd(inputs["x"], inputs["delta"], inputs["A"], inputs["B"], inputs["C"],
                              inputs.get("D"), inputs.get("z"), inputs.get("delta_bias"),
                              dy=dy, **kw)


def scan_inputs(inputs: dict, cfg=None, **kw):
    """Run the oracle on a dict of generated inputs (names as produced by ``ssmgen``)."""
    if cfg is not None:
        kw.setdefault("headdim", cfg.headdim)
        kw.setdefault("head_mode", cfg.a_mode == "head")
        kw.setdefault("delta_softplus", cfg.softplus)
    return selective_scan(inputs["x"], inputs["delta"], inputs["A"], inputs["B"], inputs["C"],
                          inputs.get("D"), inputs.get("z"), inputs.get("delta_bias"), **kw)


def rel_err(y, y_ref) -> float:
    """max_i |y_i - yref_i| / max(|yref_i|, rms(yref)): the parity metric."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    denom = np.maximum(np.abs(y_ref), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(y - y_ref) / denom))
