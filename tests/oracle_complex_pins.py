"""Pins for the oracle's complex-A scan (ssm_oracle.c, complex section): each checks it against
something other than itself. Every pin takes ``scan``, a function with the signature of
``oracle.selective_scan_complex``, so the same pins run against planted mistakes
(test_oracle_mutants.py), and returns the observed error.

Sources of the expected values:
  real_reduction        imaginary parts zero: the real scan (the oracle's own real path, itself
                        pinned by oracle_pins)
  closed_form           constant inputs: h_tn = beta_n (1 - r_n^(t+1)) / (1 - r_n), r = e^(delta A),
                        beta = delta B x, evaluated with Python's cmath
  bruteforce            y = Re(M x) + D x (times silu z) with M_ij = sum_n C_in (prod_{k=j+1..i}
                        Abar_kn) Bbar_jn materialised in numpy complex128 (the semiseparable
                        form of the Transformers-are-SSMs review page, complex case)
  conjugation           conjugating A, B and C conjugates every state, so Re(C h) and y are
                        unchanged
  rotation              A purely imaginary (|Abar| = 1): the closed form above with r on the
                        unit circle; the state is a rotating phasor sum
"""
from __future__ import annotations

import cmath
import math

import numpy as np

import oracle


def _softplus(v: float) -> float:
    return math.log(1.0 + math.exp(v)) if v < 30 else v + math.log1p(math.exp(-v))


def _problem(seed, b=2, d=4, L=20, N=3, G=2, gate=True):
    r = np.random.default_rng(seed)
    p = dict(x=r.normal(size=(b, d, L)), delta=r.normal(-1.0, 0.7, size=(b, d, L)),
             A=-np.exp(r.normal(-0.5, 0.5, size=(d, N))) + 1j * r.normal(0, 2.0, size=(d, N)),
             B=r.normal(size=(b, G, N, L)) + 1j * r.normal(size=(b, G, N, L)),
             C=r.normal(size=(b, G, N, L)) + 1j * r.normal(size=(b, G, N, L)),
             D=r.normal(size=d), z=r.normal(size=(b, d, L)) if gate else None,
             delta_bias=r.normal(0, 0.3, size=d))
    return p


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def real_reduction(scan, seed=21):
    p = _problem(seed)
    A, B, C = p["A"].real.copy(), p["B"].real.copy(), p["C"].real.copy()
    y = scan(p["x"], p["delta"], A.astype(np.complex128), B.astype(np.complex128),
             C.astype(np.complex128), p["D"], p["z"], p["delta_bias"], True)
    yr = oracle.selective_scan(p["x"], p["delta"], A, B, C, p["D"], p["z"], p["delta_bias"], True)
    return _rel(y, yr)


def closed_form(scan, seed=22, rotation=False):
    r = np.random.default_rng(seed)
    d, N, L = 3, 4, 40
    delta = 0.3
    xv = 0.7
    A = (-np.exp(r.normal(-1, 0.3, size=(d, N))) if not rotation else np.zeros((d, N))) \
        + 1j * r.normal(0, 1.5, size=(d, N))
    Bc = r.normal(size=N) + 1j * r.normal(size=N)
    Cc = r.normal(size=N) + 1j * r.normal(size=N)
    D = r.normal(size=d)
    x = np.full((1, d, L), xv)
    dl = np.full((1, d, L), delta)
    B = np.broadcast_to(Bc[None, None, :, None], (1, 1, N, L)).copy()
    C = np.broadcast_to(Cc[None, None, :, None], (1, 1, N, L)).copy()
    y = scan(x, dl, A, B, C, D, None, None, False)
    ref = np.empty((1, d, L))
    for c in range(d):
        for t in range(L):
            acc = 0.0
            for n in range(N):
                rr = cmath.exp(delta * complex(A[c, n]))
                beta = delta * complex(Bc[n]) * xv
                h = beta * (1 - rr ** (t + 1)) / (1 - rr)
                acc += (complex(Cc[n]) * h).real
            ref[0, c, t] = acc + D[c] * xv
    return _rel(y, ref)


def rotation(scan, seed=23):
    return closed_form(scan, seed, rotation=True)


def bruteforce(scan, seed=24):
    p = _problem(seed)
    x, dr, A, B, C, D, z, bias = (p[k] for k in ("x", "delta", "A", "B", "C", "D", "z", "delta_bias"))
    b, d, L = x.shape
    G, N = B.shape[1], B.shape[2]
    y = scan(x, dr, A, B, C, D, z, bias, True)
    ref = np.empty((b, d, L))
    for bb in range(b):
        for c in range(d):
            g = c // (d // G)
            dl = np.array([_softplus(dr[bb, c, t] + bias[c]) for t in range(L)])
            Abar = np.exp(dl[:, None] * A[c][None, :])          # (L, N)
            Bbar = dl[:, None] * B[bb, g].T                      # (L, N)
            M = np.zeros((L, L), dtype=np.complex128)
            for i in range(L):
                for j in range(i + 1):
                    prod = np.prod(Abar[j + 1:i + 1], axis=0) if i > j else np.ones(N)
                    M[i, j] = np.sum(C[bb, g][:, i] * prod * Bbar[j])
            yy = (M @ x[bb, c]).real + D[c] * x[bb, c]
            yy *= z[bb, c] / (1.0 + np.exp(-z[bb, c]))
            ref[bb, c] = yy
    return _rel(y, ref)


def conjugation(scan, seed=25):
    p = _problem(seed)
    args = (p["D"], p["z"], p["delta_bias"], True)
    y1 = scan(p["x"], p["delta"], p["A"], p["B"], p["C"], *args)
    y2 = scan(p["x"], p["delta"], np.conj(p["A"]), np.conj(p["B"]), np.conj(p["C"]), *args)
    return _rel(y2, y1)


PINS = {"real_reduction": (real_reduction, 1e-14), "closed_form": (closed_form, 1e-12),
        "rotation": (rotation, 1e-12), "bruteforce": (bruteforce, 1e-12),
        "conjugation": (conjugation, 1e-14)}


def run_all(scan):
    out = {}
    for name, (fn, tol) in PINS.items():
        err = fn(scan)
        out[name] = (err, err <= tol)
    return out
