"""The backward pass (ssm_selective_scan_bwd) against the fp64 oracle's gradients (needs an
MI355X). Every gradient is compared with the parity metric of the forward tests,
max |g - g_ref| / max(|g_ref|, rms(g_ref)): within 1e-4 with fp32 I/O and 2e-2 with bf16 I/O
(fp32 arithmetic in both; the bf16 gradients dx, ddelta, dz are rounded once to bf16).
"""
import sys

import numpy as np
import pytest

import oracle
import ssmgen
from scan_cases import TOL, device_inputs, to_torch, y_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_24_amd as ssm
    ssm.lib()  # fails loudly if the HIP library is not built


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(cfg, inputs, dy, h0=None, zoh=False, dhf=None):
    import selective_state_space_24_amd as ssm
    dev = device_inputs(inputs)
    dyd = to_torch(dy, dy.dtype == np.uint16, "cuda")
    h0d = torch.from_numpy(h0).cuda() if h0 is not None else None
    dhfd = torch.from_numpy(dhf).cuda() if dhf is not None else None
    g = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("D"),
                               dev.get("z"), dev.get("delta_bias"), cfg.softplus, dyd, h0=h0d,
                               want_dh0=h0 is not None or dhf is not None, zoh=zoh,
                               dh_final=dhfd)
    torch.cuda.synchronize()
    return {k: y_to_f64(v) for k, v in g.items()}


def _dy(cfg, seed):
    """dL/dy drawn N(0, 1) with the io dtype (bf16 bit patterns for bf16)."""
    n = cfg.batch * cfg.dim * cfg.L
    return ssmgen.fill(cfg.seed ^ 0xD1, 9, ssmgen.NORMAL, 0.0, 1.0, n, cfg.io_code).reshape(
        cfg.batch, cfg.dim, cfg.L)


def _compare(cfg, inputs, dy, h0=None, tol=None, zoh=False, dhf=None):
    g = _run(cfg, inputs, dy, h0, zoh=zoh, dhf=dhf)
    ref = oracle.scan_inputs_bwd(inputs, dy, cfg, h0=None if h0 is None else h0.astype(np.float64),
                                 zoh=zoh, dh_final=dhf, want_dh0=dhf is not None)
    tol = tol or TOL[cfg.io]
    errs = {}
    for k, v in ref.items():
        assert k in g, k
        assert np.isfinite(g[k]).all(), k
        errs[k] = oracle.rel_err(g[k], v)
    _say(f"[bwd] errors {', '.join(f'{k} {e:.2e}' for k, e in errs.items())}")
    bad = {k: e for k, e in errs.items() if e > tol}
    assert not bad, f"gradients beyond {tol}: {bad}"


CASES = [
    # batch, dim, L, N, io, gate, softplus, D, bias, groups, h0
    (2, 64, 100, 16, "f32", False, True, True, True, 1, False),
    (2, 130, 77, 8, "bf16", True, True, True, True, 1, False),     # ragged dim and L
    (1, 64, 256, 16, "f32", True, True, True, True, 1, True),      # initial state and dh0
    (3, 128, 200, 4, "bf16", True, True, True, True, 2, False),    # two B/C groups
    (1, 70, 130, 16, "f32", True, False, False, False, 1, False),  # no softplus, D, bias
    (2, 64, 65, 1, "f32", True, True, True, True, 1, True),        # one state
    (1, 96, 64, 5, "f32", False, True, True, True, 1, False),      # ragged state count
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_matches_oracle(case):
    batch, dim, L, N, io, gate, sp, hasD, bias, G, h0 = case
    dists = {} if sp else {"delta": ssmgen.Dist(ssmgen.UNIFORM, 0.0, 0.2),
                           "delta_bias": ssmgen.Dist(ssmgen.UNIFORM, 0.001, 0.01)}
    cfg = ssmgen.ScanConfig(name="bwd", batch=batch, dim=dim, L=L, N=N, ngroups=G, io=io,
                            gate=gate, softplus=sp, has_D=hasD, has_bias=bias, seed=400 + L,
                            dists=dists)
    _say(f"[bwd] {case}")
    inputs = ssmgen.make_inputs(cfg)
    hinit = np.random.default_rng(L).standard_normal((batch, dim, N)).astype(np.float32) if h0 else None
    _compare(cfg, inputs, _dy(cfg, L), hinit)


WIDE_CASES = [
    # batch, dim, L, N, headdim, a_mode, io, gate, zoh, h0, dh_final
    (2, 128, 100, 32, 64, "head", "bf16", True, False, False, False),
    (1, 256, 77, 128, 64, "head", "f32", True, False, True, False),     # 8 wavefronts of 16
    (2, 192, 130, 64, 32, "head", "f32", False, False, False, False),   # two rows per head
    (1, 64, 50, 8, 2, "head", "f32", True, False, False, True),         # heads of two channels
    (2, 96, 70, 16, 96, "head", "f32", True, False, True, False),       # a head over two groups
    (2, 64, 90, 16, 1, "diag", "f32", True, True, False, False),        # zero-order hold
    (1, 70, 60, 32, 1, "diag", "f32", True, True, True, True),
    (2, 128, 100, 64, 64, "head", "bf16", True, True, True, False),
    (1, 64, 40, 64, 1, "diag", "f32", False, False, False, False),      # dstate above 16
    (1, 64, 33, 128, 1, "diag", "f32", True, False, False, False),
    (2, 64, 100, 16, 1, "diag", "f32", True, False, True, True),        # four-state kernel
    (1, 64, 2, 128, 64, "head", "f32", True, True, False, True),        # shorter than a block
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_head_mode_zoh_and_wide_states(case):
    """One A per head (dA, ddelta, dbias summed over each head's channels), dstate up to 128,
    the zero-order hold, and the gradient of the final state."""
    batch, dim, L, N, hd, mode, io, gate, zoh, h0, dhf = case
    cfg = ssmgen.ScanConfig(name="bwd-wide", batch=batch, dim=dim, L=L, N=N, headdim=hd,
                            a_mode=mode, io=io, gate=gate, seed=900 + L + N)
    _say(f"[bwd-wide] {case}")
    inputs = ssmgen.make_inputs(cfg)
    r = np.random.default_rng(L + N)
    hinit = r.standard_normal((batch, dim, N)).astype(np.float32) if h0 else None
    dhfin = r.standard_normal((batch, dim, N)).astype(np.float32) if dhf else None
    _compare(cfg, inputs, _dy(cfg, L), hinit, zoh=zoh, dhf=dhfin)


@pytest.mark.parametrize("N,zoh", [(16, False), (32, False), (16, True)],
                         ids=["four-state-kernel", "wide-kernel", "wide-kernel-zoh"])
def test_final_state_gradient_without_softplus(N, zoh):
    """delta taken as given (no softplus), with a bias and a final-state gradient, and L = 100,
    which is not a multiple of either kernel's tile. The padding steps of the last tile are run
    in reverse first, while the gradient is the final-state one; their ddelta term is not zero
    without the softplus factor, and must not reach the bias gradient."""
    dists = {"delta": ssmgen.Dist(ssmgen.UNIFORM, 0.0, 0.2),
             "delta_bias": ssmgen.Dist(ssmgen.UNIFORM, 0.001, 0.01)}
    cfg = ssmgen.ScanConfig(name="bwd-nosp-dhf", batch=2, dim=64, L=100, N=N, io="f32", gate=True,
                            softplus=False, has_D=True, has_bias=True, seed=4711 + N, dists=dists)
    _say(f"[bwd] no softplus, final-state gradient, N={N}, zoh={zoh}")
    inputs = ssmgen.make_inputs(cfg)
    dhfin = np.random.default_rng(N).standard_normal((2, 64, N)).astype(np.float32)
    _compare(cfg, inputs, _dy(cfg, cfg.L), zoh=zoh, dhf=dhfin)


@pytest.mark.parametrize("ci", [0, 1])
def test_backward_configs(ci):
    cfg = ssmgen.CONFIGS[ci]
    _say(f"[bwd] config {ci} {cfg.name}")
    inputs = ssmgen.make_inputs(cfg)
    _compare(cfg, inputs, _dy(cfg, ci))


def test_backward_is_deterministic():
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.ScanConfig(name="bwd-det", batch=2, dim=192, L=300, N=16, seed=5)
    inputs = ssmgen.make_inputs(cfg)
    dy = _dy(cfg, 1)
    a = _run(cfg, inputs, dy)
    b = _run(cfg, inputs, dy)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_full_size_bench_workload():
    """The Mamba-1.4B layer (batch 8, d_inner 4096, N 16, L 4096, bf16) at full size, in the
    launch configuration that bench.py --workload bwd times. The oracle runs one batch entry at a
    time: dx, ddelta, dz, dB and dC of the first and last entries are compared whole, and dA, dD
    and dbias (sums over the batch) against the sum of all eight entries' oracle gradients."""
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.CONFIGS[2]
    _say(f"[bwd] config 2 {cfg.name}: generating inputs")
    dev = {}
    for name in cfg.shapes():
        dev.update(device_inputs({name: ssmgen.make_tensor(cfg, name)}))
    dy = _dy(cfg, 2)
    dyd = to_torch(dy, dy.dtype == np.uint16, "cuda")
    _say("[bwd] config 2: running")
    g = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"],
                               dev["z"], dev["delta_bias"], cfg.softplus, dyd)
    torch.cuda.synchronize()
    del dev, dyd
    summed = {"dA": None, "dD": None, "ddelta_bias": None}
    one = ssmgen.with_shape(cfg, batch=1)
    worst = {}
    for b in range(cfg.batch):
        ref = oracle.scan_inputs_bwd(ssmgen.make_batch_entry(cfg, b), dy[b:b + 1], one)
        for k in summed:
            summed[k] = ref[k] if summed[k] is None else summed[k] + ref[k]
        if b in (0, cfg.batch - 1):
            for k in ("dx", "ddelta", "dz", "dB", "dC"):
                got = y_to_f64(g[k][b:b + 1])
                assert np.isfinite(got).all(), (k, b)
                err = oracle.rel_err(got, ref[k])
                worst[k] = max(worst.get(k, 0.0), err)
                assert err <= TOL[cfg.io], f"{k} of batch entry {b}: rel err {err:.3e}"
        del ref
    for k, v in summed.items():
        err = oracle.rel_err(y_to_f64(g[k]), v)
        worst[k] = err
        assert err <= TOL[cfg.io], f"{k}: rel err {err:.3e}"
    _say(f"[bwd] config 2 errors {', '.join(f'{k} {e:.2e}' for k, e in worst.items())}")
    del g
    torch.cuda.empty_cache()


def _oracle_bwd_entry_by_blocks(cfg, b, dy_b, block):
    """The oracle's gradients of batch entry b, run over channel blocks (whole heads, one B/C
    group each) on the host's threads at once; dB and dC are the sums over the blocks, in block
    order."""
    from concurrent.futures import ThreadPoolExecutor
    starts = list(range(0, cfg.dim, block))

    def one(d0):
        d1 = min(cfg.dim, d0 + block)
        sub = ssmgen.block_config(cfg, d0, d1)
        return oracle.scan_inputs_bwd(ssmgen.make_channel_block(cfg, b, d0, d1, nthreads=1),
                                      dy_b[None, d0:d1], sub, nthreads=1)
    with ThreadPoolExecutor(max_workers=min(16, oracle.cpu_threads())) as ex:
        parts = list(ex.map(one, starts))
    rows = lambda d0, d1: ((d0 // cfg.headdim, d1 // cfg.headdim) if cfg.a_mode == "head"
                           else (d0, d1))
    out = {k: np.concatenate([g[k] for g in parts], axis=1) for k in ("dx", "dz")}
    out["ddelta"] = np.concatenate([g["ddelta"] for g in parts], axis=1)
    for k in ("dA", "dD", "ddelta_bias"):
        out[k] = np.concatenate([g[k] for g in parts], axis=0)
    for k in ("dB", "dC"):
        acc = None
        for g in parts:
            acc = g[k] if acc is None else acc + g[k]
        out[k] = acc
    assert rows(0, cfg.dim)[1] == out["ddelta"].shape[1]
    return out


@pytest.mark.timeout(900)
def test_backward_full_size_scalar_decay_heads():
    """The scalar-decay heads config (batch 4, 64 heads x 64, N 128, L 8192, bf16) at full size:
    every gradient of every batch entry against the oracle run one entry at a time (over blocks
    of one head each, in parallel), and dA, dD and dbias against the sum over the four
    entries."""
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.CONFIGS[4]
    _say(f"[bwd] config 4 {cfg.name}: generating inputs")
    dev = {}
    for name in cfg.shapes():
        dev.update(device_inputs({name: ssmgen.make_tensor(cfg, name)}))
    dy = _dy(cfg, 4)
    dyd = to_torch(dy, dy.dtype == np.uint16, "cuda")
    _say("[bwd] config 4: running")
    g = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"],
                               dev["z"], dev["delta_bias"], cfg.softplus, dyd)
    torch.cuda.synchronize()
    del dev, dyd
    summed = {"dA": None, "dD": None, "ddelta_bias": None}
    worst = {}
    for b in range(cfg.batch):
        ref = _oracle_bwd_entry_by_blocks(cfg, b, dy[b], cfg.headdim)
        for k in summed:
            summed[k] = ref[k] if summed[k] is None else summed[k] + ref[k]
        for k in ("dx", "ddelta", "dz", "dB", "dC"):
            got = y_to_f64(g[k][b:b + 1])
            assert np.isfinite(got).all(), (k, b)
            err = oracle.rel_err(got, ref[k])
            worst[k] = max(worst.get(k, 0.0), err)
            assert err <= TOL[cfg.io], f"{k} of batch entry {b}: rel err {err:.3e}"
        del ref
        _say(f"[bwd] config 4: batch entry {b} done")
    for k, v in summed.items():
        err = oracle.rel_err(y_to_f64(g[k]), v)
        worst[k] = err
        assert err <= TOL[cfg.io], f"{k}: rel err {err:.3e}"
    _say(f"[bwd] config 4 errors {', '.join(f'{k} {e:.2e}' for k, e in worst.items())}")
    del g
    torch.cuda.empty_cache()
