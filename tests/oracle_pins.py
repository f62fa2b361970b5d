"""Pins for the fp64 oracle: each checks the oracle against something other than itself.

Every pin takes ``scan``, a function with the signature of ``oracle.selective_scan``, so the same
pins can be run against deliberately broken copies of the oracle (see test_oracle_mutants.py).
Each returns the observed error; the caller compares it with the stated bound.

Sources of the expected values (none of them re-types the oracle's loop):
  closed_form_geometric   geometric series of the constant-input recurrence
  skip_path               B = 0 leaves only D x (times silu(z))
  semiseparable_bruteforce  y = M x + D x with the materialised matrix
                          M_ij = sum_n C_in (prod_{k=j+1..i} Abar_kn) Bbar_jn (Transformers-are-SSMs
                          review page: SSMs as semiseparable matrices)
  lti_convolution         LTI case as a causal convolution with kernel K_k = sum_n C_n r_n^k dB_n
                          (NL-345 page, §2 "Computation", eq. (3), and "LTI")
  theorem1_gate           Theorem 1 (memo page, "数式解説" item 4): N=1, A=-1, B=1, softplus gives
                          the gated RNN h = (1 - g) h + g x with g = sigmoid(v) under ZOH
  linearity, causality, segment_composition, head_broadcast, limit_A0, limit_fast_decay
"""
from __future__ import annotations

import math

import numpy as np


def _softplus(v: float) -> float:
    # independent of the oracle's formula: direct definition, safe for |v| < 700
    return math.log(1.0 + math.exp(v)) if v < 30 else v + math.log1p(math.exp(-v))


def _sigmoid(v: float) -> float:
    return 1.0 / (1.0 + math.exp(-v))


def _rng(seed):
    return np.random.default_rng(seed)


def closed_form_geometric(scan, seed=1):
    """delta, x, B_n, C_n constant in t: h_tn = beta_n (1 - r_n^(t+1)) / (1 - r_n)."""
    r = _rng(seed)
    L, N = 200, 5
    dval, xval = 0.037, 1.3
    a = -r.uniform(0.5, 4.0, N)
    Bn, Cn = r.normal(size=N), r.normal(size=N)
    Dv = 0.4
    x = np.full((1, 1, L), xval)
    delta = np.full((1, 1, L), dval)
    B = np.broadcast_to(Bn[:, None], (N, L)).reshape(1, 1, N, L).copy()
    C = np.broadcast_to(Cn[:, None], (N, L)).reshape(1, 1, N, L).copy()
    y = scan(x, delta, a.reshape(1, N), B, C, np.array([Dv]), None, None, False)
    t = np.arange(L)[:, None]
    rn = np.exp(dval * a)[None, :]
    beta = (dval * Bn * xval)[None, :]
    h = beta * (1 - rn ** (t + 1)) / (1 - rn)
    yref = (h * Cn[None, :]).sum(1) + Dv * xval
    return float(np.max(np.abs(y[0, 0] - yref) / np.maximum(np.abs(yref), 1e-300)))


def skip_path(scan, seed=2):
    """B = 0: y = D x silu(z), bit for bit (same two products)."""
    r = _rng(seed)
    b, d, L, N = 2, 3, 50, 4
    x, z = r.normal(size=(b, d, L)), r.normal(size=(b, d, L))
    delta = r.normal(size=(b, d, L))
    A = -r.uniform(1, 5, (d, N))
    B = np.zeros((b, 1, N, L))
    C = r.normal(size=(b, 1, N, L))
    Dv = r.normal(size=d)
    bias = r.normal(size=d)
    y = scan(x, delta, A, B, C, Dv, z, bias, True)
    yref = np.empty_like(x)
    for bi in range(b):
        for di in range(d):
            for t in range(L):
                zz = z[bi, di, t]
                yref[bi, di, t] = (0.0 + Dv[di] * x[bi, di, t]) * (zz / (1.0 + math.exp(-zz)))
    return float(np.max(np.abs(y - yref)))


def _problem(seed, b=2, d=4, L=24, N=3, G=2, headdim=1, head_mode=False, gate=True):
    r = _rng(seed)
    nh = d // headdim
    rows = nh if head_mode else d
    p = dict(
        x=r.normal(size=(b, d, L)),
        delta=0.5 * r.normal(size=(b, rows, L)),
        A=-r.uniform(0.5, 6.0, (nh,) if head_mode else (d, N)),
        B=r.normal(size=(b, G, N, L)),
        C=r.normal(size=(b, G, N, L)),
        D=r.normal(size=d),
        z=r.normal(size=(b, d, L)) if gate else None,
        delta_bias=np.log(np.expm1(r.uniform(0.05, 0.5, rows))),
    )
    return p


def semiseparable_bruteforce(scan, seed=3, head_mode=False, zoh=False):
    """y = M x + D x (then gate), M built entry by entry from the discretised parameters."""
    headdim = 2 if head_mode else 1
    p = _problem(seed, headdim=headdim, head_mode=head_mode)
    b, d, L = p["x"].shape
    G, N = p["B"].shape[1], p["B"].shape[2]
    y = scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True,
             headdim=headdim, head_mode=head_mode, zoh=zoh)
    yref = np.zeros((b, d, L))
    for bi in range(b):
        for di in range(d):
            row = di // headdim if head_mode else di
            g = di // (d // G)
            dl = [_softplus(p["delta"][bi, row, t] + p["delta_bias"][row]) for t in range(L)]
            for n in range(N):
                a = p["A"][row] if head_mode else p["A"][di, n]
                Abar = [math.exp(dl[t] * a) for t in range(L)]
                if zoh:
                    Bbar = [(math.exp(dl[t] * a) - 1.0) / a * p["B"][bi, g, n, t] for t in range(L)]
                else:
                    Bbar = [dl[t] * p["B"][bi, g, n, t] for t in range(L)]
                for i in range(L):
                    for j in range(i + 1):
                        prod = 1.0
                        for k in range(j + 1, i + 1):
                            prod *= Abar[k]
                        yref[bi, di, i] += p["C"][bi, g, n, i] * prod * Bbar[j] * p["x"][bi, di, j]
            for t in range(L):
                yref[bi, di, t] += p["D"][di] * p["x"][bi, di, t]
                zz = p["z"][bi, di, t]
                yref[bi, di, t] *= zz * _sigmoid(zz)
    scale = np.sqrt(np.mean(yref ** 2))
    return float(np.max(np.abs(y - yref)) / scale)


def lti_convolution(scan, seed=4):
    """Constant delta, B, C: y_t = sum_k K_k x_(t-k) + D x_t with K_k = sum_n C_n r_n^k delta B_n."""
    r = _rng(seed)
    L, N = 300, 6
    dval = 0.05
    a = -r.uniform(0.2, 3.0, N)
    Bn, Cn = r.normal(size=N), r.normal(size=N)
    x = r.normal(size=(1, 1, L))
    Dv = -0.7
    B = np.repeat(Bn[:, None], L, 1).reshape(1, 1, N, L)
    C = np.repeat(Cn[:, None], L, 1).reshape(1, 1, N, L)
    y = scan(x, np.full((1, 1, L), dval), a.reshape(1, N), B, C, np.array([Dv]), None, None, False)
    k = np.arange(L)
    K = (Cn[None, :] * np.exp(dval * a)[None, :] ** k[:, None] * (dval * Bn)[None, :]).sum(1)
    xs = x[0, 0]
    yref = np.array([np.dot(K[: t + 1][::-1], xs[: t + 1]) for t in range(L)]) + Dv * xs
    return float(np.max(np.abs(y[0, 0] - yref)) / np.sqrt(np.mean(yref ** 2)))


def theorem1_gate(scan, seed=5, zoh=True):
    """N=1, A=-1, B=C=1, D=0, softplus: ZOH gives h = (1 - sigmoid(v)) h + sigmoid(v) x;
    the delta*B rule gives h = sigmoid(-v) h + softplus(v) x."""
    r = _rng(seed)
    L = 400
    v = 1.5 * r.normal(size=L)
    x = r.normal(size=L)
    y = scan(x.reshape(1, 1, L), v.reshape(1, 1, L), np.array([[-1.0]]), np.ones((1, 1, 1, L)),
             np.ones((1, 1, 1, L)), None, None, None, True, zoh=zoh)
    h, yref = 0.0, np.empty(L)
    for t in range(L):
        if zoh:
            g = _sigmoid(v[t])
            h = (1.0 - g) * h + g * x[t]
        else:
            h = _sigmoid(-v[t]) * h + _softplus(v[t]) * x[t]
        yref[t] = h
    return float(np.max(np.abs(y[0, 0] - yref)) / np.sqrt(np.mean(yref ** 2)))


def linearity(scan, seed=6):
    p = _problem(seed, gate=False)
    r = _rng(seed + 100)
    x2 = r.normal(size=p["x"].shape)
    al, be = 0.7, -1.9

    def run(x):
        return scan(x, p["delta"], p["A"], p["B"], p["C"], p["D"], None, p["delta_bias"], True)
    lhs = run(al * p["x"] + be * x2)
    rhs = al * run(p["x"]) + be * run(x2)
    return float(np.max(np.abs(lhs - rhs)) / np.sqrt(np.mean(rhs ** 2)))


def causality(scan, seed=7):
    """Changing every input at t0 leaves y_t for t < t0 bit-identical; returns the max change."""
    p = _problem(seed, L=40)
    t0 = 17
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    for k in ("x", "delta", "z"):
        q[k][..., t0:] += 0.3
    q["B"][..., t0:] *= -1.0
    q["C"][..., t0:] += 1.0
    y1 = scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True)
    y2 = scan(q["x"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"], q["delta_bias"], True)
    before = float(np.max(np.abs(y1[..., :t0] - y2[..., :t0])))
    after = float(np.min(np.max(np.abs(y1[..., t0:] - y2[..., t0:]), axis=-1)))
    return before, after


def segment_composition(scan, seed=8):
    """[0, m) then [m, L) from the carried state equals [0, L), bit for bit."""
    p = _problem(seed, L=50)
    m = 21
    full, hfull = scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                       p["delta_bias"], True, return_final_state=True)
    sl = lambda a, s: np.ascontiguousarray(a[..., s])  # noqa: E731
    y1, h1 = scan(sl(p["x"], slice(0, m)), sl(p["delta"], slice(0, m)), p["A"],
                  sl(p["B"], slice(0, m)), sl(p["C"], slice(0, m)), p["D"], sl(p["z"], slice(0, m)),
                  p["delta_bias"], True, return_final_state=True)
    y2, h2 = scan(sl(p["x"], slice(m, None)), sl(p["delta"], slice(m, None)), p["A"],
                  sl(p["B"], slice(m, None)), sl(p["C"], slice(m, None)), p["D"],
                  sl(p["z"], slice(m, None)), p["delta_bias"], True, h0=h1, return_final_state=True)
    return (float(np.max(np.abs(np.concatenate([y1, y2], -1) - full))),
            float(np.max(np.abs(h2 - hfull))))


def head_broadcast(scan, seed=9):
    """Head mode equals per-channel mode with A, delta and bias repeated over each head."""
    headdim = 2
    p = _problem(seed, headdim=headdim, head_mode=True)
    d, N = p["x"].shape[1], p["B"].shape[2]
    yh = scan(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True,
              headdim=headdim, head_mode=True)
    A_full = np.repeat(np.repeat(p["A"], headdim)[:, None], N, 1)
    yc = scan(p["x"], np.repeat(p["delta"], headdim, axis=1), A_full, p["B"], p["C"], p["D"],
              p["z"], np.repeat(p["delta_bias"], headdim), True)
    assert A_full.shape == (d, N)
    return float(np.max(np.abs(yh - yc)))


def limit_A0(scan, seed=10):
    """A = 0: Abar = 1, so h_t is the running sum of delta_s B_s x_s."""
    r = _rng(seed)
    L, N = 120, 3
    x = r.normal(size=(1, 1, L))
    delta = r.uniform(0.01, 0.2, (1, 1, L))
    B, C = r.normal(size=(1, 1, N, L)), r.normal(size=(1, 1, N, L))
    y = scan(x, delta, np.zeros((1, N)), B, C, None, None, None, False)
    h = np.cumsum(delta[0, 0][None, :] * B[0, 0] * x[0, 0][None, :], axis=1)
    yref = (C[0, 0] * h).sum(0)
    return float(np.max(np.abs(y[0, 0] - yref)) / np.sqrt(np.mean(yref ** 2)))


def limit_fast_decay(scan, seed=11):
    """delta * A << 0: Abar ~ 0 (below 1e-40), the state forgets: h_t = delta_t B_t x_t."""
    r = _rng(seed)
    L, N = 80, 3
    x = r.normal(size=(1, 1, L))
    delta = r.uniform(0.5, 1.0, (1, 1, L))
    B, C = r.normal(size=(1, 1, N, L)), r.normal(size=(1, 1, N, L))
    y = scan(x, delta, np.full((1, N), -200.0), B, C, None, None, None, False)
    yref = (C[0, 0] * delta[0, 0][None, :] * B[0, 0] * x[0, 0][None, :]).sum(0)
    return float(np.max(np.abs(y[0, 0] - yref)) / np.sqrt(np.mean(yref ** 2)))


def run_all(scan):
    """All pins with their bounds; returns {name: (value, passed)}."""
    res = {}
    res["closed_form_geometric"] = (v := closed_form_geometric(scan)), v < 1e-12
    res["skip_path"] = (v := skip_path(scan)), v == 0.0
    res["semiseparable"] = (v := semiseparable_bruteforce(scan)), v < 1e-12
    res["semiseparable_head"] = (v := semiseparable_bruteforce(scan, head_mode=True)), v < 1e-12
    res["semiseparable_zoh"] = (v := semiseparable_bruteforce(scan, zoh=True)), v < 1e-12
    res["lti_convolution"] = (v := lti_convolution(scan)), v < 1e-12
    res["theorem1_zoh"] = (v := theorem1_gate(scan, zoh=True)), v < 1e-13
    res["theorem1_euler"] = (v := theorem1_gate(scan, zoh=False)), v < 1e-13
    res["linearity"] = (v := linearity(scan)), v < 1e-12
    before, after = causality(scan)
    res["causality"] = (before, after), before == 0.0 and after > 0.0
    ys, hs = segment_composition(scan)
    res["segment_composition"] = (ys, hs), ys == 0.0 and hs == 0.0
    res["head_broadcast"] = (v := head_broadcast(scan)), v == 0.0
    res["limit_A0"] = (v := limit_A0(scan)), v < 1e-12
    res["limit_fast_decay"] = (v := limit_fast_decay(scan)), v < 1e-12
    return res
