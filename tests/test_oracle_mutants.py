"""Planted mistakes in copies of the oracle (built on the CPU) must each fail at least one pin.

Forward mutants edit the forward section of the source (before the backward section's marker)
and must fail a forward pin; backward mutants edit the backward section and must fail a
backward pin (finite differences, torch autograd or the transposed-matrix closed form); complex
mutants edit the complex-A section and must fail a complex pin."""
import os
import subprocess

import pytest

import oracle
import oracle_bwd_pins as BP
import oracle_complex_pins as CP
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")
BWD_MARK = "Gradients of the scan above"
COMPLEX_MARK = "Complex diagonal A."

MUTANTS = {
    "drop_D": ("double yt = acc + Dd * xt;", "double yt = acc;"),
    "swap_B_C": ("const double Bt = Bg[n * L + t], Ct = Cg[n * L + t];",
                 "const double Bt = Cg[n * L + t], Ct = Bg[n * L + t];"),
    "bias_after_softplus": ("const double v = dr[t] + bias;\n    const double delta = p->delta_softplus ? softplus(v) : v;",
                            "const double v = dr[t];\n    const double delta = (p->delta_softplus ? softplus(v) : v) + bias;"),
    "exp_sign": ("const double Abar = exp(delta * a);", "const double Abar = exp(-delta * a);"),
    "readout_before_update": ("h[n] = Abar * h[n] + Bbar * xt;\n      acc += Ct * h[n];",
                              "acc += Ct * h[n];\n      h[n] = Abar * h[n] + Bbar * xt;"),
    "group_index": ("const int64_t group = d / (p->dim / p->ngroups);",
                    "const int64_t group = d % p->ngroups;"),
    "head_index": ("const int64_t head = d / p->headdim;", "const int64_t head = d % nheads;"),
    "gate_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "B_time_shift": ("const double Bt = Bg[n * L + t]", "const double Bt = Bg[n * L + (t ? t - 1 : 0)]"),
    "zoh_missing_1_over_a": ("expm1(delta * a) / a * Bt", "expm1(delta * a) * Bt"),
    "softplus_sign": ("log1p(exp(-fabs(v)))", "log1p(exp(fabs(v)))"),
    "ignore_h0": ("h[n] = p->h0 ? p->h0[(b * p->dim + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "x_not_scaled_by_delta": ("else Bbar = delta * Bt;", "else Bbar = Bt;"),
}


BWD_MUTANTS = {
    "bwd_no_decay_of_gh": ("gh[n] *= Abar;", ""),
    "bwd_dC_with_previous_state": ("dCg[n * L + t] += gy * ht[n];", "dCg[n * L + t] += gy * hp[n];"),
    "bwd_softplus_derivative_sign": ("gdelta * sigmoid(v)", "gdelta * sigmoid(-v)"),
    "bwd_silu_derivative": ("s * (1.0 + zr[t] * (1.0 - s))", "s"),
    "bwd_dA_without_delta": ("gh[n] * (delta * Abar * hp[n]", "gh[n] * (Abar * hp[n]"),
    "bwd_dx_without_state_path": ("gx += gh[n] * Bbar;", ""),
    "bwd_zoh_dBbar_ddelta": ("df_ddelta = Abar;", "df_ddelta = 1.0;"),
    "bwd_dB_without_factor": ("dBg[n * L + t] += gh[n] * xt * f;", "dBg[n * L + t] += gh[n] * xt;"),
    "bwd_gate_not_applied": ("gy = gyr[t] * zr[t] * s;", "gy = gyr[t];"),
    "bwd_final_state_gradient_dropped": ("gh[n] = q->dh_final ? q->dh_final[(b * p->dim + d) * N + n] : 0.0;",
                                         "gh[n] = 0.0;"),
}


COMPLEX_MUTANTS = {
    "cplx_conjugated_readout": ("acc += creal(Ct * h[n]);", "acc += creal(conj(Ct) * h[n]);"),
    "cplx_imaginary_readout": ("acc += creal(Ct * h[n]);", "acc += cimag(Ct * h[n]);"),
    "cplx_decay_without_rotation": ("cexp(delta * a)", "exp(delta * creal(a))"),
    "cplx_exp_sign": ("cexp(delta * a)", "cexp(-delta * a)"),
    "cplx_B_real_part_only": ("const double complex Bbar = delta * Bt;",
                              "const double complex Bbar = delta * creal(Bt);"),
    "cplx_A_conjugated": ("p->Ar[d * N + n] + I * p->Ai[d * N + n]",
                          "p->Ar[d * N + n] - I * p->Ai[d * N + n]"),
    "cplx_C_imag_sign": ("p->Cr[goff + n * L + t] + I * p->Ci[goff + n * L + t]",
                         "p->Cr[goff + n * L + t] - I * p->Ci[goff + n * L + t]"),
}


@pytest.fixture(scope="module")
def src():
    return open(SRC).read()


def _build(tmp_path, name, text):
    cpath = tmp_path / f"{name}.c"
    cpath.write_text(text)
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    str(cpath), "-o", str(so), "-lm", "-lpthread"], check=True)
    return oracle.load_library(str(so))


def _mutate(src, old, new, backward):
    cut = src.index(BWD_MARK)
    head, tail = src[:cut], src[cut:]
    part = tail if backward else head
    assert part.count(old) == 1, f"mutation site not found exactly once: {old!r}"
    part = part.replace(old, new)
    return head + part if backward else part + tail


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, src, tmp_path):
    old, new = BWD_MUTANTS[name]
    lib = _build(tmp_path, name, _mutate(src, old, new, backward=True))

    def bwd(*a, **k):
        return oracle.selective_scan_bwd(*a, lib=lib, **k)

    def fwd(*a, **k):
        return oracle.selective_scan(*a, lib=lib, **k)
    errs = [BP.finite_differences(bwd, fwd, head_mode=h, zoh=z, softplus=sp, gate=g)
            for (h, z, sp, g) in [(False, False, True, True), (False, True, True, True),
                                  (True, False, True, True)]]
    errs.append(BP.dx_closed_form(bwd))
    errs.append(BP.final_state_fd(bwd, fwd))
    errs.append(BP.two_pieces(bwd, fwd))
    assert max(errs) > 1e-4, f"backward mutant {name} passed every pin: {errs}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src, tmp_path):
    old, new = MUTANTS[name]
    lib = _build(tmp_path, name, _mutate(src, old, new, backward=False))

    def scan(*a, **k):
        return oracle.selective_scan(*a, lib=lib, **k)
    res = P.run_all(scan)
    failed = [k for k, (_, ok) in res.items() if not ok]
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(COMPLEX_MUTANTS))
def test_complex_mutant_is_caught(name, src, tmp_path):
    old, new = COMPLEX_MUTANTS[name]
    cut = src.index(COMPLEX_MARK)
    head, tail = src[:cut], src[cut:]
    assert tail.count(old) == 1, f"mutation site not found exactly once: {old!r}"
    lib = _build(tmp_path, name, head + tail.replace(old, new))

    def scan(*a, **k):
        return oracle.selective_scan_complex(*a, lib=lib, **k)
    res = CP.run_all(scan)
    failed = [k for k, (_, ok) in res.items() if not ok]
    assert failed, f"complex mutant {name} passed every pin"
