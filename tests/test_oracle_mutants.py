"""Planted mistakes in copies of the oracle (built on the CPU) must each fail at least one pin."""
import os
import subprocess

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")

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


@pytest.fixture(scope="module")
def src():
    return open(SRC).read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src, tmp_path):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    cpath = tmp_path / f"{name}.c"
    cpath.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    str(cpath), "-o", str(so), "-lm", "-lpthread"], check=True)
    lib = oracle.load_library(str(so))

    def scan(*a, **k):
        return oracle.selective_scan(*a, lib=lib, **k)
    res = P.run_all(scan)
    failed = [k for k, (_, ok) in res.items() if not ok]
    assert failed, f"mutant {name} passed every pin"
