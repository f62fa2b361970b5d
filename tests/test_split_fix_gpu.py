"""The split along L of the independent-wavefront forward kernel (needs an MI355X).

A sequence with too few channels to fill the chip is cut into segments. There are two schemes.
Segments shorter than 32768 steps run a summary pass first: each segment's end state from a zero
start and its sum of delta. The output pass then starts every segment from the summaries of the
earlier ones, composed. Longer segments instead run the output pass over every segment at once:
segment 0 from the initial state, the later ones from a zero state. Each segment writes its
summary and stores its state after every 1024 steps. A correcting pass then reruns segments 1,
2, ... from their true initial states, composed from the summaries. It rewrites y until its state
is bitwise equal to a stored one, because from there on the output pass's y is the true one.

Checked here:
  * batch 1 x 512 channels x L = 2^18 (64 segments of 4096 steps, the summary scheme), every
    output element against the fp64 oracle. Also the same shape with A = 0 for one state of every
    channel in the first 16-channel wavefront, whose state is then a running sum;
  * the million-token config (16 segments of 65536 steps, the correcting scheme) with the same
    A = 0 channels. The two trajectories of that wavefront never meet, so its correcting pass
    runs every segment to its end; the channels are compared with the oracle over all 2^20 steps;
  * the allocation-free entry point on the million-token config. Its 8 MiB array holds the
    summaries but not the stored states (64 MiB), so it runs with the summaries only, and its
    correcting pass runs every segment to its end. Its y and final state (with an initial state
    given) must be bitwise those of the workspace entry point: the stored states only decide
    where the correcting pass may stop. Every other output of the correcting scheme is compared
    with the oracle by the million-token test of test_parity_full_gpu.py.
"""
import sys

import numpy as np
import pytest

import oracle
import ssmgen
from scan_cases import TOL, device_inputs, run_hip, y_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MID = ssmgen.ScanConfig(name="split-summary", batch=1, dim=512, L=1 << 18, N=16, seed=701)
C3 = ssmgen.CONFIGS[3]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_24_amd as ssm
    ssm.lib()  # fails loudly if the HIP library is not built


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ptr(t):
    return None if t is None else int(t.data_ptr())


def test_workspace_of_each_scheme():
    import selective_state_space_24_amd as ssm
    # 64 segments of 4096 steps: summaries only
    mid = ssm.workspace_size(ssm.desc_contiguous(MID.batch, MID.dim, MID.L, MID.N))
    assert mid == MID.dim * 64 * (MID.N + 1) * 4
    # 16 segments of 65536 steps: summaries, slack, 32 stored states of 16 floats
    c3 = ssm.workspace_size(ssm.desc_contiguous(C3.batch, C3.dim, C3.L, C3.N))
    assert c3 == C3.dim * 16 * 17 * 4 + 12 + C3.dim * 16 * 32 * 64
    assert C3.dim * 16 * 17 * 4 <= ssm.NOALLOC_SCRATCH_BYTES < c3


@pytest.mark.timeout(600)
@pytest.mark.parametrize("a_zero", [False, True], ids=["decaying", "one-state-never-decays"])
def test_summary_scheme_matches_oracle(a_zero):
    inputs = ssmgen.make_inputs(MID)
    if a_zero:
        inputs["A"] = inputs["A"].copy()
        inputs["A"][:16, 5] = 0.0
    _say(f"[split] summary scheme, a_zero={a_zero}: running the GPU path")
    y = run_hip(device_inputs(inputs))
    torch.cuda.synchronize()
    ref = oracle.scan_inputs(inputs, MID)
    got = y_to_f64(y)
    assert np.isfinite(got).all()
    err = oracle.rel_err(got, ref)
    _say(f"[split] summary scheme, a_zero={a_zero}: max rel err {err:.3e} over {got.size}")
    assert err <= TOL[MID.io]
    if a_zero:
        # the running-sum channels with their own rms floor
        err16 = oracle.rel_err(got[:, :16], ref[:, :16])
        _say(f"[split] running-sum channels: max rel err {err16:.3e}")
        assert err16 <= TOL[MID.io]


@pytest.fixture(scope="module")
def c3_inputs():
    _say("[split] million-token config: generating inputs")
    dev = {}
    for name in C3.shapes():
        dev.update(device_inputs({name: ssmgen.make_tensor(C3, name)}))
    yield dev
    dev.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_correcting_scheme_running_sum_channels(c3_inputs):
    dev = dict(c3_inputs)
    dev["A"] = dev["A"].clone()
    dev["A"][:16, 5] = 0.0
    _say("[split] correcting scheme with running-sum channels: running the GPU path")
    y = run_hip(dev)
    torch.cuda.synchronize()
    picks = [(0, 16), (16, 18), (C3.dim - 2, C3.dim)]
    for d0, d1 in picks:
        blk = ssmgen.make_channel_block(C3, 0, d0, d1)
        if d0 < 16:
            blk["A"] = blk["A"].copy()
            blk["A"][:, 5] = 0.0
        ref = oracle.scan_inputs(blk, ssmgen.block_config(C3, d0, d1))
        got = y_to_f64(y[:, d0:d1])
        assert np.isfinite(got).all()
        err = oracle.rel_err(got, ref)
        _say(f"[split] channels [{d0}, {d1}): max rel err {err:.3e} over {got.size}")
        assert err <= TOL[C3.io], (d0, d1, err)
    del y
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_noalloc_without_stored_states_is_bitwise_the_same(c3_inputs):
    import selective_state_space_24_amd as ssm
    dev = c3_inputs
    h0 = torch.randn(C3.batch, C3.dim, C3.N, device="cuda",
                     generator=torch.Generator(device="cuda").manual_seed(7))
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for mode in ("workspace", "noalloc"):
        _say(f"[split] million-token config through the {mode} entry point")
        y = torch.full_like(dev["x"], float("nan"))
        hfin = torch.full((C3.batch, C3.dim, C3.N), float("nan"), device="cuda")
        desc = ssm.describe(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("z"), y)
        ext = ssm.ScanExt(ssm.SSM_DISC_DELTA_B, ssm.SSM_ALGO_AUTO, _ptr(h0), _ptr(hfin))
        args = (desc, _ptr(dev["x"]), _ptr(dev["delta"]), _ptr(dev["A"]), _ptr(dev["B"]),
                _ptr(dev["C"]), _ptr(dev.get("D")), _ptr(dev.get("z")),
                _ptr(dev.get("delta_bias")), C3.softplus, _ptr(y))
        if mode == "noalloc":
            rc = ssm.fwd_noalloc_raw(*args, ext, stream)
        else:
            need = ssm.workspace_size(desc)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            rc = ssm.fwd_ext_raw(*args, ext, _ptr(ws), need, stream)
        assert rc == 0, (mode, ssm.status_string(rc))
        torch.cuda.synchronize()
        out[mode] = (y, hfin)
    yw, hw = out["workspace"]
    yn, hn = out["noalloc"]
    assert torch.isfinite(hw).all()
    assert torch.equal(yw.view(torch.int16), yn.view(torch.int16))
    assert torch.equal(hw.view(torch.int32), hn.view(torch.int32))
    # with h0 the first segment starts from it: its first channel against the oracle
    blk = ssmgen.make_channel_block(C3, 0, 0, 2)
    ref, href = oracle.scan_inputs(blk, ssmgen.block_config(C3, 0, 2),
                                   h0=h0[:, :2].double().cpu().numpy(), return_final_state=True)
    err = oracle.rel_err(y_to_f64(yw[:, :2]), ref)
    herr = oracle.rel_err(hw[:, :2].double().cpu().numpy(), href)
    _say(f"[split] with h0, channels [0, 2): max rel err {err:.3e}, final state {herr:.3e}")
    assert err <= TOL[C3.io] and herr <= 1e-4
