"""The oracle's backward pass against finite differences, torch autograd and a closed form (CPU)."""
import pytest

import oracle
from oracle_bwd_pins import (dx_closed_form, final_state_fd, finite_differences,
                             torch_autograd, two_pieces)

FD_TOL = 2e-6      # central differences with eps = 1e-6 relative: O(eps^2) + rounding / eps
AUTOGRAD_TOL = 1e-11
CLOSED_TOL = 1e-12


@pytest.mark.parametrize("head_mode,zoh,softplus,gate", [
    (False, False, True, True), (False, True, True, True), (True, False, True, True),
    (True, True, False, True), (False, False, False, False)])
def test_backward_matches_finite_differences(head_mode, zoh, softplus, gate):
    err = finite_differences(oracle.selective_scan_bwd, oracle.selective_scan, head_mode=head_mode,
                             zoh=zoh, softplus=softplus, gate=gate)
    assert err <= FD_TOL, err


@pytest.mark.parametrize("head_mode,zoh,softplus", [(False, False, True), (True, True, True),
                                                    (False, True, False)])
def test_backward_matches_torch_autograd(head_mode, zoh, softplus):
    pytest.importorskip("torch")
    err = torch_autograd(oracle.selective_scan_bwd, head_mode=head_mode, zoh=zoh, softplus=softplus)
    assert err <= AUTOGRAD_TOL, err


def test_dx_is_the_transposed_semiseparable_matrix():
    assert dx_closed_form(oracle.selective_scan_bwd) <= CLOSED_TOL


def test_backward_does_not_depend_on_thread_count():
    import numpy as np
    from oracle_bwd_pins import problem
    p = problem(4, b=5, d=6, L=30, N=4, G=2)
    dy = np.random.default_rng(0).normal(size=p["x"].shape)
    args = (p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"], True, dy)
    g1 = oracle.selective_scan_bwd(*args, h0=p["h0"], nthreads=1)
    g3 = oracle.selective_scan_bwd(*args, h0=p["h0"], nthreads=3)
    for k in g1:
        assert np.array_equal(g1[k], g3[k]), k


@pytest.mark.parametrize("head_mode,zoh", [(False, False), (True, True)])
def test_final_state_gradient_matches_finite_differences(head_mode, zoh):
    err = final_state_fd(oracle.selective_scan_bwd, oracle.selective_scan, head_mode=head_mode,
                         zoh=zoh)
    assert err <= FD_TOL, err


@pytest.mark.parametrize("head_mode,zoh", [(False, False), (False, True), (True, False)])
def test_two_pieces_reproduce_the_whole_sequence(head_mode, zoh):
    assert two_pieces(oracle.selective_scan_bwd, oracle.selective_scan, head_mode=head_mode,
                      zoh=zoh) <= 1e-12
