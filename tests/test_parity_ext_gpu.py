"""The extended entry point (ssm_selective_scan_fwd_ext) against the fp64 oracle on the GPU:
zero-order-hold B discretisation, initial state, final state, and a scan resumed across calls.

Tolerances as in test_parity_gpu: y within 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O); the fp32 final
state within 1e-4 in every case (it is never rounded to the io dtype).
"""
import sys

import numpy as np
import pytest

import oracle
import ssmgen
from scan_cases import TOL, device_inputs, y_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

STATE_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_24_amd as ssm
    ssm.lib()  # fails loudly if the HIP library is not built


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cfg(batch, dim, L, N, headdim=1, a_mode="diag", io="f32", gate=True, sp=True, seed=7,
         dists=None):
    d = dict(dists or {})
    if not sp:
        d.setdefault("delta", ssmgen.Dist(ssmgen.UNIFORM, 0.0, 0.2))
        d.setdefault("delta_bias", ssmgen.Dist(ssmgen.UNIFORM, 0.001, 0.01))
    return ssmgen.ScanConfig(name="ext", batch=batch, dim=dim, L=L, N=N, headdim=headdim,
                             a_mode=a_mode, io=io, gate=gate, softplus=sp, seed=seed, dists=d)


def _run(cfg, inputs, zoh=False, h0=None, final=False):
    import selective_state_space_24_amd as ssm
    dev = device_inputs(inputs)
    h0_dev = torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).cuda() if h0 is not None else None
    out = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"],
                                 dev.get("D"), dev.get("z"), dev.get("delta_bias"), cfg.softplus,
                                 zoh=zoh, h0=h0_dev, final_state=final)
    torch.cuda.synchronize()
    return out


def _oracle(cfg, inputs, zoh=False, h0=None, final=False):
    return oracle.scan_inputs(inputs, cfg, zoh=zoh, h0=h0, return_final_state=final)


def _h0(cfg, seed=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((cfg.batch, cfg.dim, cfg.N)).astype(np.float32)


ZOH_CASES = [
    # batch, dim, L, N, headdim, a_mode, io, gate, softplus
    (1, 64, 256, 16, 1, "diag", "f32", False, True),
    (2, 100, 300, 16, 1, "diag", "bf16", True, True),
    (1, 64, 130, 5, 1, "diag", "f32", True, False),
    (2, 256, 200, 64, 64, "head", "f32", True, True),
    (1, 128, 97, 128, 64, "head", "bf16", True, True),
    (1, 64, 4096, 16, 1, "diag", "f32", True, True),      # split along L
    (1, 128, 190, 16, 32, "head", "bf16", True, True),
]


@pytest.mark.parametrize("case", ZOH_CASES, ids=lambda c: "-".join(map(str, c)))
def test_zoh_matches_oracle(case):
    batch, dim, L, N, hd, mode, io, gate, sp = case
    cfg = _cfg(batch, dim, L, N, hd, mode, io, gate, sp, seed=100 + L)
    _say(f"[zoh] {case}")
    inputs = ssmgen.make_inputs(cfg)
    y = _run(cfg, inputs, zoh=True)
    yref = _oracle(cfg, inputs, zoh=True)
    err = oracle.rel_err(y_to_f64(y), yref)
    assert err <= TOL[io], f"rel err {err:.3e}"
    # the rule really is different from delta * B on these inputs
    assert oracle.rel_err(_oracle(cfg, inputs, zoh=False), yref) > 10 * TOL[io]


def test_zoh_limits_a_zero_and_underflow():
    """A = 0 (B_bar -> delta * B exactly) and exp(delta A) below the fp32 range (B_bar -> -B/A)."""
    cfg = _cfg(1, 64, 200, 4, io="f32", gate=False, seed=5)
    inputs = ssmgen.make_inputs(cfg)
    A = inputs["A"].copy()
    A[:, 0] = 0.0
    A[:, 1] = -400.0  # delta up to ~0.6: delta * A < -150, exp underflows in fp32
    A[:, 2] = -1e-3
    inputs["A"] = A
    _say("[zoh] limits")
    y = _run(cfg, inputs, zoh=True)
    yref = _oracle(cfg, inputs, zoh=True)
    err = oracle.rel_err(y_to_f64(y), yref)
    assert err <= TOL["f32"], f"rel err {err:.3e}"


STATE_CASES = [
    (2, 64, 300, 16, 1, "diag", "f32", True),
    (1, 130, 77, 8, 1, "diag", "bf16", True),
    (2, 128, 150, 128, 64, "head", "bf16", True),
    (1, 64, 4096, 16, 1, "diag", "bf16", True),       # split along L: h0 enters segment 0 only
    (1, 144, 333, 13, 1, "diag", "bf16", True),
]


@pytest.mark.parametrize("case", STATE_CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("zoh", [False, True])
def test_initial_and_final_state(case, zoh):
    batch, dim, L, N, hd, mode, io, gate = case
    cfg = _cfg(batch, dim, L, N, hd, mode, io, gate, seed=200 + L)
    _say(f"[state] {case} zoh={zoh}")
    inputs = ssmgen.make_inputs(cfg)
    h0 = _h0(cfg)
    y, hT = _run(cfg, inputs, zoh=zoh, h0=h0, final=True)
    yref, hTref = _oracle(cfg, inputs, zoh=zoh, h0=h0.astype(np.float64), final=True)
    err_y = oracle.rel_err(y_to_f64(y), yref)
    err_h = oracle.rel_err(hT.cpu().numpy().astype(np.float64), hTref)
    assert err_y <= TOL[io], f"y rel err {err_y:.3e}"
    assert err_h <= STATE_TOL, f"final state rel err {err_h:.3e}"
    # the initial state matters on these inputs
    assert oracle.rel_err(_oracle(cfg, inputs, zoh=zoh), yref) > 10 * TOL[io]


def test_resume_in_two_pieces():
    """[0, m) then [m, L) carrying the state equals [0, L) (the oracle's segment composition)."""
    cfg = _cfg(2, 96, 500, 16, io="f32", seed=77)
    inputs = ssmgen.make_inputs(cfg)
    m = 173
    first = {k: (v[..., :m] if k in ("x", "delta", "z", "B", "C") else v) for k, v in inputs.items()}
    second = {k: (v[..., m:] if k in ("x", "delta", "z", "B", "C") else v) for k, v in inputs.items()}
    c1 = ssmgen.with_shape(cfg, L=m)
    c2 = ssmgen.with_shape(cfg, L=cfg.L - m)
    _say("[state] resume")
    y1, h1 = _run(c1, {k: np.ascontiguousarray(v) for k, v in first.items()}, final=True)
    y2, h2 = _run(c2, {k: np.ascontiguousarray(v) for k, v in second.items()},
                  h0=h1.cpu().numpy(), final=True)
    yref, href = _oracle(cfg, inputs, final=True)
    y = np.concatenate([y_to_f64(y1), y_to_f64(y2)], axis=-1)
    assert oracle.rel_err(y, yref) <= TOL["f32"]
    assert oracle.rel_err(h2.cpu().numpy().astype(np.float64), href) <= STATE_TOL


def test_no_steps_copies_the_state():
    import selective_state_space_24_amd as ssm
    x = torch.zeros(2, 8, 0, dtype=torch.float32, device="cuda")
    B = torch.zeros(2, 1, 4, 0, dtype=torch.float32, device="cuda")
    A = -torch.ones(8, 4, device="cuda")
    h0 = torch.randn(2, 8, 4, device="cuda")
    y, hT = ssm.selective_scan_fwd(x, x.clone(), A, B, B.clone(), h0=h0, final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)
    hT2 = torch.full((2, 8, 4), 7.0, device="cuda")
    ssm.selective_scan_fwd(x, x.clone(), A, B, B.clone(), final_state=hT2)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hT2).item() == 0
