"""Pins for the fp64 oracle's backward pass: each checks the gradients against something other
than the backward code itself.

  finite_differences   central differences of f = sum(dy * y) through the (separately pinned)
                       forward oracle, for every entry of every input, in several modes
  torch_autograd       an independent forward written with plain torch fp64 ops, differentiated
                       by torch.autograd
  dx_closed_form       without a gate y = (M + diag D) x with the materialised semiseparable
                       matrix M (Transformers-are-SSMs review page), so dx = (M + diag D)^T dy
  final_state_fd       central differences of f = sum(dy * y) + sum(dhf * h_final): the gradient
                       that enters through the final state (a sequence scanned in pieces)
  two_pieces           a sequence split at step m: the second piece's backward from the state
                       the forward oracle reaches at m gives dh0, which fed as the first piece's
                       final-state gradient must reproduce the whole sequence's gradients

Every pin takes ``bwd`` with the signature of ``oracle.selective_scan_bwd`` (and the finite
differences also ``fwd`` = ``oracle.selective_scan``), so the same pins can run against broken
copies of the oracle. Each returns the observed error; callers compare it with the stated bound.
"""
from __future__ import annotations

import math

import numpy as np

GRAD_NAMES = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


def problem(seed, b=2, d=4, L=9, N=3, G=2, headdim=1, head_mode=False, gate=True, h0=True,
            D=True, bias=True):
    r = np.random.default_rng(seed)
    nh = d // headdim
    rows = nh if head_mode else d
    return dict(
        x=r.normal(size=(b, d, L)),
        delta=0.5 * r.normal(size=(b, rows, L)),
        A=-r.uniform(0.5, 6.0, (nh,) if head_mode else (d, N)),
        B=r.normal(size=(b, G, N, L)),
        C=r.normal(size=(b, G, N, L)),
        D=r.normal(size=d) if D else None,
        z=r.normal(size=(b, d, L)) if gate else None,
        delta_bias=np.log(np.expm1(r.uniform(0.05, 0.5, rows))) if bias else None,
        h0=r.normal(size=(b, d, N)) if h0 else None,
    )


def _positive_step(p, seed):
    """Without softplus the step is raw + bias itself: draw both positive (a decaying scan)."""
    r = np.random.default_rng(seed + 50)
    p["delta"] = r.uniform(0.02, 0.3, p["delta"].shape)
    if p["delta_bias"] is not None:
        p["delta_bias"] = r.uniform(0.001, 0.05, p["delta_bias"].shape)


def _call_fwd(fwd, p, softplus, headdim, head_mode, zoh):
    return fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
               softplus, headdim=headdim, head_mode=head_mode, zoh=zoh, h0=p["h0"])


def _call_bwd(bwd, p, dy, softplus, headdim, head_mode, zoh):
    return bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
               softplus, dy, headdim=headdim, head_mode=head_mode, zoh=zoh, h0=p["h0"])


def finite_differences(bwd, fwd, seed=1, head_mode=False, zoh=False, softplus=True, gate=True):
    """max over inputs and entries of |grad - fd| / max(1, max|fd of that input|)."""
    headdim = 2 if head_mode else 1
    p = problem(seed, headdim=headdim, head_mode=head_mode, gate=gate)
    if not softplus:
        _positive_step(p, seed)
    r = np.random.default_rng(seed + 100)
    dy = r.normal(size=p["x"].shape)
    g = _call_bwd(bwd, p, dy, softplus, headdim, head_mode, zoh)
    f = lambda q: float(np.sum(dy * _call_fwd(fwd, q, softplus, headdim, head_mode, zoh)))
    worst = 0.0
    for name in GRAD_NAMES:
        if p[name] is None:
            continue
        base = p[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p)
            up = base.copy(); up[idx] += eps
            dn = base.copy(); dn[idx] -= eps
            q[name] = up
            fu = f(q)
            q[name] = dn
            fdn = f(q)
            fd[idx] = (fu - fdn) / (2 * eps)
        scale = max(1.0, float(np.max(np.abs(fd))))
        worst = max(worst, float(np.max(np.abs(g["d" + name] - fd))) / scale)
    return worst


def _torch_forward(torch, p, softplus, headdim, head_mode, zoh):
    """The scan in plain torch fp64 ops (independent of the oracle's C code)."""
    x, dl_raw, A, B, C = p["x"], p["delta"], p["A"], p["B"], p["C"]
    b, d, L = x.shape
    G, N = B.shape[1], B.shape[2]
    rows = torch.arange(d) // headdim if head_mode else torch.arange(d)
    grp = torch.arange(d) // (d // G)
    v = dl_raw[:, rows, :]
    if p["delta_bias"] is not None:
        v = v + p["delta_bias"][rows][None, :, None]
    dl = torch.nn.functional.softplus(v) if softplus else v
    a = A[rows][:, None].expand(d, N) if head_mode else A
    h = p["h0"] if p["h0"] is not None else torch.zeros(b, d, N, dtype=x.dtype)
    ys = []
    for t in range(L):
        Bt, Ct = B[:, grp, :, t], C[:, grp, :, t]            # (b, d, N)
        ex = dl[:, :, t, None] * a[None]                    # (b, d, N)
        Abar = torch.exp(ex)
        f = torch.expm1(ex) / a[None] if zoh else dl[:, :, t, None]
        h = Abar * h + f * Bt * x[:, :, t, None]
        y = (Ct * h).sum(-1)
        if p["D"] is not None:
            y = y + p["D"][None] * x[:, :, t]
        if p["z"] is not None:
            zt = p["z"][:, :, t]
            y = y * zt * torch.sigmoid(zt)
        ys.append(y)
    return torch.stack(ys, dim=-1)


def torch_autograd(bwd, seed=2, head_mode=False, zoh=False, softplus=True):
    """max relative difference between the oracle's gradients and torch autograd's."""
    import torch
    headdim = 4 if head_mode else 1
    p = problem(seed, b=2, d=8, L=40, N=4, G=2, headdim=headdim, head_mode=head_mode)
    if not softplus:
        _positive_step(p, seed)
    dy = np.random.default_rng(seed + 7).normal(size=p["x"].shape)
    g = _call_bwd(bwd, p, dy, softplus, headdim, head_mode, zoh)
    tp = {k: (torch.tensor(v, dtype=torch.float64, requires_grad=True) if v is not None else None)
          for k, v in p.items()}
    y = _torch_forward(torch, tp, softplus, headdim, head_mode, zoh)
    names = [k for k in GRAD_NAMES if tp[k] is not None]
    grads = torch.autograd.grad((y * torch.tensor(dy)).sum(), [tp[k] for k in names])
    worst = 0.0
    for k, gt in zip(names, grads):
        gt = gt.numpy()
        scale = max(1e-300, float(np.max(np.abs(gt))))
        worst = max(worst, float(np.max(np.abs(g["d" + k] - gt))) / scale)
    return worst


def dx_closed_form(bwd, seed=3):
    """No gate: dx = (M + diag D)^T dy, M_ij = sum_n C_in (prod_{k=j+1..i} Abar_kn) Bbar_jn."""
    p = problem(seed, b=2, d=3, L=14, N=3, G=1, gate=False, h0=False)
    b, d, L = p["x"].shape
    N = p["B"].shape[2]
    dy = np.random.default_rng(seed + 5).normal(size=p["x"].shape)
    g = _call_bwd(bwd, p, dy, True, 1, False, False)
    sp = lambda v: math.log1p(math.exp(v)) if v < 30 else v
    ref = np.zeros_like(p["x"])
    for bi in range(b):
        for di in range(d):
            dl = [sp(p["delta"][bi, di, t] + p["delta_bias"][di]) for t in range(L)]
            M = np.zeros((L, L))
            for n in range(N):
                a = p["A"][di, n]
                Ab = [math.exp(dl[t] * a) for t in range(L)]
                for i in range(L):
                    for j in range(i + 1):
                        prod = 1.0
                        for k in range(j + 1, i + 1):
                            prod *= Ab[k]
                        M[i, j] += p["C"][bi, 0, n, i] * prod * dl[j] * p["B"][bi, 0, n, j]
            M += np.diag(np.full(L, p["D"][di]))
            ref[bi, di] = M.T @ dy[bi, di]
    return float(np.max(np.abs(g["dx"] - ref)) / np.max(np.abs(ref)))


def final_state_fd(bwd, fwd, seed=5, head_mode=False, zoh=False):
    """Like finite_differences, with a random gradient of the final state as well."""
    headdim = 2 if head_mode else 1
    p = problem(seed, headdim=headdim, head_mode=head_mode, gate=True)
    r = np.random.default_rng(seed + 200)
    dy = r.normal(size=p["x"].shape)
    dhf = r.normal(size=p["h0"].shape)
    g = bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True,
            dy, headdim=headdim, head_mode=head_mode, zoh=zoh, h0=p["h0"], dh_final=dhf)

    def f(q):
        y, hT = fwd(q["x"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"], q["delta_bias"],
                    True, headdim=headdim, head_mode=head_mode, zoh=zoh, h0=q["h0"],
                    return_final_state=True)
        return float(np.sum(dy * y) + np.sum(dhf * hT))
    worst = 0.0
    for name in GRAD_NAMES:
        base = p[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p)
            up = base.copy(); up[idx] += eps
            dn = base.copy(); dn[idx] -= eps
            q[name] = up
            fu = f(q)
            q[name] = dn
            fd[idx] = (fu - f(q)) / (2 * eps)
        scale = max(1.0, float(np.max(np.abs(fd))))
        worst = max(worst, float(np.max(np.abs(g["d" + name] - fd))) / scale)
    return worst


def two_pieces(bwd, fwd, seed=6, head_mode=False, zoh=False, m=11):
    """max relative difference between the whole sequence's gradients and the two pieces'."""
    headdim = 2 if head_mode else 1
    p = problem(seed, b=2, d=4, L=25, N=3, headdim=headdim, head_mode=head_mode)
    dy = np.random.default_rng(seed + 300).normal(size=p["x"].shape)
    kw = dict(headdim=headdim, head_mode=head_mode, zoh=zoh)
    cut = lambda a, lo, hi: None if a is None else a[..., lo:hi].copy()

    def piece(lo, hi, h0, dhf):
        return bwd(cut(p["x"], lo, hi), cut(p["delta"], lo, hi), p["A"], cut(p["B"], lo, hi),
                   cut(p["C"], lo, hi), p["D"], cut(p["z"], lo, hi), p["delta_bias"], True,
                   cut(dy, lo, hi), h0=h0, dh_final=dhf, want_dh0=True, **kw)
    whole = piece(0, 25, p["h0"], None)
    _, hm = fwd(cut(p["x"], 0, m), cut(p["delta"], 0, m), p["A"], cut(p["B"], 0, m),
                cut(p["C"], 0, m), p["D"], cut(p["z"], 0, m), p["delta_bias"], True, h0=p["h0"],
                return_final_state=True, **kw)
    second = piece(m, 25, hm, None)
    first = piece(0, m, p["h0"], second["dh0"])
    worst = 0.0
    for k in whole:
        if k in ("dx", "ddelta", "dB", "dC", "dz"):
            ref = np.concatenate([first[k], second[k]], axis=-1)
        elif k == "dh0":
            ref = first[k]
        else:
            ref = first[k] + second[k]
        scale = max(1e-300, float(np.max(np.abs(whole[k]))))
        worst = max(worst, float(np.max(np.abs(whole[k] - ref))) / scale)
    return worst
