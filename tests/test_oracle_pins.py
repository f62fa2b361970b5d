"""The fp64 oracle against closed forms, brute force and invariants (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import oracle_pins as P

scan = oracle.selective_scan


def test_closed_form_geometric_series():
    assert P.closed_form_geometric(scan) < 1e-12


def test_skip_path_is_exact():
    assert P.skip_path(scan) == 0.0


@pytest.mark.parametrize("head_mode,zoh", [(False, False), (True, False), (False, True)])
def test_semiseparable_bruteforce(head_mode, zoh):
    assert P.semiseparable_bruteforce(scan, head_mode=head_mode, zoh=zoh) < 1e-12


def test_lti_convolution():
    assert P.lti_convolution(scan) < 1e-12


@pytest.mark.parametrize("zoh", [True, False])
def test_theorem1_gated_rnn(zoh):
    assert P.theorem1_gate(scan, zoh=zoh) < 1e-13


def test_linearity_in_x():
    assert P.linearity(scan) < 1e-12


def test_causality():
    before, after = P.causality(scan)
    assert before == 0.0 and after > 0.0


def test_segment_composition_bitwise():
    assert P.segment_composition(scan) == (0.0, 0.0)


def test_head_mode_is_broadcast_channel_mode():
    assert P.head_broadcast(scan) == 0.0


def test_limits():
    assert P.limit_A0(scan) < 1e-12
    assert P.limit_fast_decay(scan) < 1e-12


def test_softplus_values():
    # softplus(0) = ln 2; softplus(v) -> v for large v; -> e^v for very negative v
    for v, ref in [(0.0, math.log(2.0)), (50.0, 50.0 + math.exp(-50.0)), (-40.0, math.exp(-40.0)),
                   (1.0, math.log1p(math.e)), (-3.0, math.log1p(math.exp(-3.0)))]:
        y = scan(np.ones((1, 1, 1)), np.array([[[v]]]), np.zeros((1, 1)), np.ones((1, 1, 1, 1)),
                 np.ones((1, 1, 1, 1)), None, None, None, True)
        # A = 0, B = C = x = 1: y_0 = delta = softplus(v)
        assert abs(y[0, 0, 0] - ref) <= 2e-16 * max(1.0, abs(ref))


def test_theorem1_worked_example():
    """Theorem 1 of the memo page with its parameters (one state, A = -1, B = 1, softplus,
    zero-order hold) makes the scan the gated RNN h_t = (1 - sigmoid(v_t)) h_{t-1} +
    sigmoid(v_t) x_t. The fixture holds a worked example computed by hand from that form, with
    steps whose sigmoid is 1/2 or 3/4, so every expected h_t is an exact binary fraction."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "theorem1.json")))
    assert fx["N"] == 1 and fx["A"] == -1.0 and fx["B"] == 1.0 and fx["tau"] == "softplus"
    ex = fx["worked_example"]
    v = np.array([math.log(3.0) if s == "ln3" else float(s) for s in ex["v"]])
    x = np.array(ex["x"])
    L = len(x)
    y = scan(x.reshape(1, 1, L), v.reshape(1, 1, L), np.array([[-1.0]]), np.ones((1, 1, 1, L)),
             np.ones((1, 1, 1, L)), None, None, None, True, zoh=True)
    assert np.max(np.abs(y[0, 0] - np.array(ex["h_zoh"]))) <= 1e-14


def test_golden_values_match_an_independent_forward():
    """Oracle outputs stored by tests/golden/make_golden.py (which calls only the oracle): they
    are still what the oracle computes, and they agree with the forward pass written
    independently in plain torch fp64 ops (tests/oracle_bwd_pins.py)."""
    import os
    import ssmgen
    torch = pytest.importorskip("torch")
    from oracle_bwd_pins import _torch_forward
    path = os.path.join(os.path.dirname(__file__), "golden", "config0_oracle_y.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    cfg = ssmgen.CONFIGS[0]
    inp = ssmgen.make_inputs(cfg)
    y = oracle.scan_inputs(inp, cfg)
    tp = {k: (torch.tensor(oracle.as_f64(inp[k])) if k in inp else None)
          for k in ("x", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    tp["h0"] = None
    yt = _torch_forward(torch, tp, True, 1, False, False).numpy()
    scale = float(np.max(np.abs(yt)))
    for b, d, t, val in rows:
        g = float.fromhex(val)
        assert g == y[int(b), int(d), int(t)]
        assert abs(g - yt[int(b), int(d), int(t)]) <= 1e-12 * scale


def test_empty_and_degenerate_sizes():
    # L = 0 and batch = 0 are valid and produce empty outputs
    y = scan(np.zeros((1, 2, 0)), np.zeros((1, 2, 0)), np.zeros((2, 3)), np.zeros((1, 1, 3, 0)),
             np.zeros((1, 1, 3, 0)))
    assert y.shape == (1, 2, 0)
    y = scan(np.zeros((0, 2, 5)), np.zeros((0, 2, 5)), np.zeros((2, 3)), np.zeros((0, 1, 3, 5)),
             np.zeros((0, 1, 3, 5)))
    assert y.shape == (0, 2, 5)
