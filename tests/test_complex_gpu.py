"""The complex-A forward scan (a_mode SSM_A_COMPLEX) against the fp64 oracle on the GPU.

Tolerances: 2e-2 for bf16 I/O, as for the real scan. For fp32 I/O the kernel's phase carries the
fp32 rounding of delta (and of delta Im(A) / 2 pi): a relative error of a few u = 2^-24 in each
step's angle delta Im(A). A state remembers about 1 / (delta |Re A|) steps, so those phase errors
add up to a relative error of about 4 u |Im A| / |Re A| in the state and in y (the same
amplification that the real scan's exp error sees). The fp32 gate is
therefore max(1e-4, 16 u max_n |Im A_n| / |Re A_n|): four times that estimate, for the metric's
pick of the worst element. A CPU emulation of the kernel's fp32 arithmetic with correctly rounded
sin and cos lands at 0.9-3.4 u R on these inputs.
"""
import sys

import numpy as np
import pytest

import oracle
import ssmgen
from scan_cases import TOL, device_inputs, y_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U32 = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_24_amd as ssm
    ssm.lib()  # fails loudly if the HIP library is not built


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cfg(batch, dim, L, N, ngroups=1, io="f32", gate=True, sp=True, seed=11, dists=None):
    d = dict(dists or {})
    if not sp:
        d.setdefault("delta", ssmgen.Dist(ssmgen.UNIFORM, 0.0, 0.2))
        d.setdefault("delta_bias", ssmgen.Dist(ssmgen.UNIFORM, 0.001, 0.01))
    return ssmgen.ScanConfig(name="complex", batch=batch, dim=dim, L=L, N=N, ngroups=ngroups,
                             a_mode="complex", io=io, gate=gate, softplus=sp, seed=seed, dists=d)


def _tol(cfg, A):
    if cfg.io == "bf16":
        return TOL["bf16"]
    ratio = float(np.max(np.abs(A[..., 1]) / np.abs(A[..., 0])))
    return max(TOL["f32"], 16 * U32 * ratio)


def _run(cfg, dev, out=None):
    import selective_state_space_24_amd as ssm
    y = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"],
                               dev.get("D"), dev.get("z"), dev.get("delta_bias"), cfg.softplus,
                               out=out)
    torch.cuda.synchronize()
    return y


CASES = [
    # batch, dim, L, N, ngroups, io, gate, softplus
    (1, 64, 256, 16, 1, "f32", True, True),
    (2, 100, 300, 4, 1, "f32", False, True),     # ragged channels and steps
    (2, 128, 97, 8, 2, "bf16", True, True),      # two groups
    (1, 64, 513, 32, 1, "f32", True, True),      # the largest state
    (1, 192, 200, 5, 3, "bf16", False, False),   # N not a multiple of 4, no softplus
    (2, 64, 1, 16, 1, "f32", True, True),        # one step
    (1, 64, 16, 32, 1, "bf16", True, True),      # exactly one tile
    (3, 130, 77, 12, 1, "bf16", True, True),     # ragged everything
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_complex_matches_oracle(case):
    batch, dim, L, N, G, io, gate, sp = case
    cfg = _cfg(batch, dim, L, N, G, io, gate, sp)
    _say(f"[complex] {case}")
    inputs = ssmgen.make_inputs(cfg)
    y = _run(cfg, device_inputs(inputs))
    yref = oracle.scan_inputs_complex(inputs, cfg)
    err = oracle.rel_err(y_to_f64(y), yref)
    tol = _tol(cfg, inputs["A"])
    _say(f"[complex] {case}: rel err {err:.3e} (tol {tol:.2e})")
    assert err <= tol, f"{case}: rel err {err:.3e}"


def test_complex_slow_decay_tolerance_scales():
    """Re(A) down to -0.05: the state remembers hundreds of steps and the phase error grows with
    |Im A| / |Re A|; the error stays under the derived fp32 gate."""
    cfg = _cfg(1, 64, 1200, 16, dists={"A": ssmgen.Dist(ssmgen.UNIFORM, -0.2, -0.05)}, seed=12)
    inputs = ssmgen.make_inputs(cfg)
    y = _run(cfg, device_inputs(inputs))
    yref = oracle.scan_inputs_complex(inputs, cfg)
    err = oracle.rel_err(y_to_f64(y), yref)
    tol = _tol(cfg, inputs["A"])
    _say(f"[complex] slow decay: rel err {err:.3e} (tol {tol:.2e})")
    assert err <= tol


def test_complex_real_parts_only_equals_real_scan():
    """Imaginary parts of A, B and C zero: the complex kernel gives the real kernel's y (both on
    the GPU, same inputs) to fp32 rounding, and both match the real oracle."""
    import selective_state_space_24_amd as ssm
    cfg = _cfg(2, 128, 300, 16, seed=13)
    inputs = ssmgen.make_inputs(cfg)
    N = cfg.N
    inputs["A"][..., 1] = 0.0
    inputs["B"][:, :, N:] = 0.0
    inputs["C"][:, :, N:] = 0.0
    dev = device_inputs(inputs)
    y = _run(cfg, dev)
    A_real = torch.from_numpy(np.ascontiguousarray(inputs["A"][..., 0])).cuda()
    B_real = dev["B"][:, :, :N].contiguous()
    C_real = dev["C"][:, :, :N].contiguous()
    yr = ssm.selective_scan_fwd(dev["x"], dev["delta"], A_real, B_real, C_real, dev["D"],
                                dev["z"], dev["delta_bias"], True)
    torch.cuda.synchronize()
    err = oracle.rel_err(y_to_f64(y), y_to_f64(yr))
    _say(f"[complex] real parts only vs real kernel: rel err {err:.3e}")
    assert err <= 1e-5
    yref = oracle.selective_scan(inputs["x"], inputs["delta"], inputs["A"][..., 0],
                                 inputs["B"][:, :, :N], inputs["C"][:, :, :N], inputs["D"],
                                 inputs["z"], inputs["delta_bias"], True)
    assert oracle.rel_err(y_to_f64(y), yref) <= TOL["f32"]


def test_complex_strided_and_misaligned():
    """x, delta, z and y as views with a row stride that is not a multiple of 16 bytes, and B, C
    starting one element past a 16-byte boundary: the kernel's element-wise paths."""
    cfg = _cfg(2, 64, 203, 8, io="bf16", seed=14)
    inputs = ssmgen.make_inputs(cfg)
    yref = oracle.scan_inputs_complex(inputs, cfg)
    dev = device_inputs(inputs)

    def widen(t, extra):
        big = torch.zeros(t.shape[:-1] + (t.shape[-1] + extra,), dtype=t.dtype, device=t.device)
        big[..., :t.shape[-1]] = t
        return big[..., :t.shape[-1]]

    for k in ("x", "delta", "z"):
        dev[k] = widen(dev[k], 3)
    for k in ("B", "C"):
        flat = torch.zeros(dev[k].numel() + 1, dtype=dev[k].dtype, device=dev[k].device)
        flat[1:] = dev[k].reshape(-1)
        dev[k] = flat[1:].view(dev[k].shape)
    out = widen(torch.zeros(2, 64, 203, dtype=torch.bfloat16, device="cuda"), 5)
    y = _run(cfg, dev, out=out)
    err = oracle.rel_err(y_to_f64(y), yref)
    _say(f"[complex] strided/misaligned: rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.timeout(600)
def test_complex_layer_size_every_element():
    """The bench workload, a Mamba-130M-sized layer (batch 8, 1536 channels, L 2048, N 16,
    bf16, gate), in one call as bench.py --workload complex runs it; every output against the
    oracle, which runs one batch entry at a time on inputs regenerated from the streams."""
    cfg = ssmgen.COMPLEX_CONFIG
    dev = {}
    for name in cfg.shapes():
        dev.update(device_inputs({name: ssmgen.make_tensor(cfg, name)}))
    y = y_to_f64(_run(cfg, dev))
    del dev
    one = ssmgen.with_shape(cfg, batch=1)
    worst = 0.0
    for b in range(cfg.batch):
        yref = oracle.scan_inputs_complex(ssmgen.make_batch_entry(cfg, b), one)
        err = oracle.rel_err(y[b:b + 1], yref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (b, err)
    _say(f"[complex] layer size: worst rel err {worst:.3e} over {y.size} outputs")


def test_complex_empty_and_rejections():
    import selective_state_space_24_amd as ssm
    cfg = _cfg(1, 64, 0, 8)
    inputs = ssmgen.make_inputs(cfg)
    dev = device_inputs(inputs)
    y = _run(cfg, dev)
    assert y.shape == (1, 64, 0)
    cfg = _cfg(1, 64, 32, 8)
    dev = device_inputs(ssmgen.make_inputs(cfg))
    args = (dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
            dev["delta_bias"], True)
    for kw in ({"zoh": True}, {"final_state": True}, {"algorithm": "chunked"},
               {"h0": torch.zeros(1, 64, 8, device="cuda")}):
        with pytest.raises(ssm.ScanError) as e:
            ssm.selective_scan_fwd(*args, **kw)
        assert e.value.status == -9, kw  # SSM_ERR_UNSUPPORTED
