"""The C ABI on the host: the library loads, exports what the header declares, and rejects bad
arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import selective_state_space_24_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

if not os.path.exists(ssm.LIB_PATH):  # built by __graft_entry__.build(); build once if missing
    from selective_state_space_24_amd import build as _b
    _b.build()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssm_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"ssm_selective_scan_fwd", "ssm_selective_scan_fwd_ext",
            "ssm_selective_scan_workspace_size", "ssm_status_string", "ssm_abi_version",
            "ssm_scan_desc_init_contiguous"} <= set(names)
    h = ctypes.CDLL(ssm.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n


def test_version_and_status_strings():
    assert ssm.abi_version() == 6
    for code in range(-10, 1):
        s = ssm.status_string(code)
        assert s and s != "unknown status"
    assert ssm.status_string(-100) == "unknown status"


def test_desc_size_matches_header():
    # 6 int64 + 2 int32 + 14 int64 strides
    assert ctypes.sizeof(ssm.ScanDesc) == 6 * 8 + 2 * 4 + 14 * 8
    # 2 int32 + 2 pointers
    assert ctypes.sizeof(ssm.ScanExt) == 2 * 4 + 2 * 8


FAKE = 1 << 40  # never dereferenced: every call below must fail validation first


def _fwd(desc, **over):
    args = dict(x=FAKE, delta=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                C=FAKE + (4 << 30), D=None, z=None, delta_bias=None, y=FAKE + (8 << 30),
                ws=None, wsb=0)
    args.update(over)
    return ssm.fwd_raw(desc, args["x"], args["delta"], args["A"], args["B"], args["C"], args["D"],
                       args["z"], args["delta_bias"], True, args["y"], args["ws"], args["wsb"], None)


def test_validation_errors_are_reported_before_launch():
    d = ssm.desc_contiguous(2, 64, 128, 16)
    assert _fwd(d, x=None) == -1
    assert _fwd(d, y=None) == -1
    assert ssm.fwd_raw(None if False else d, None, None, None, None, None, None, None, None, 1,
                       None, None, 0, None) == -1
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.dstate = 129
    assert _fwd(bad) == -2
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.dim = 0
    assert _fwd(bad) == -2
    bad = ssm.desc_contiguous(2, 64, 128, 16, ngroups=3)
    assert _fwd(bad) == -2
    bad = ssm.desc_contiguous(2, 64, 128, 16, headdim=2, a_mode=ssm.SSM_A_HEAD)
    bad.headdim = 5
    assert _fwd(bad) == -2
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.headdim = 2  # diag mode requires headdim 1
    assert _fwd(bad) == -2
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.io_dtype = 7
    assert _fwd(bad) == -3
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.a_mode = 3
    assert _fwd(bad) == -3
    bad = ssm.desc_contiguous(2, 64, 128, 16, a_mode=ssm.SSM_A_COMPLEX)
    bad.headdim = 2  # complex mode requires headdim 1
    assert _fwd(bad) == -2
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.x_stride_dim = -1
    assert _fwd(bad) == -4
    bad = ssm.desc_contiguous(2, 64, 128, 16)
    bad.y_stride_dim = 100  # output rows would overlap
    assert _fwd(bad) == -4
    assert _fwd(d, x=FAKE + 1) == -5                      # bf16 needs 2-byte alignment
    assert _fwd(d, A=FAKE + (2 << 30) + 2) == -5          # fp32 needs 4-byte alignment
    assert _fwd(d, y=FAKE + 64) == -6                     # y overlaps x
    assert _fwd(d, y=FAKE + (3 << 30)) == -6              # y overlaps B
    big = ssm.desc_contiguous(1, 2048, 1 << 20, 16)
    need = ssm.workspace_size(big)
    assert need > 0
    assert _fwd(big) == -7
    assert _fwd(big, ws=FAKE + (20 << 30), wsb=need - 4) == -7
    g = ssm.desc_contiguous(1, 64, 128, 16, ngroups=8)     # B/C group of 8 channels: unsupported
    assert _fwd(g) == -9


def _fwd_ext(desc, ext, **over):
    args = dict(x=FAKE, delta=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                C=FAKE + (4 << 30), D=None, z=None, delta_bias=None, y=FAKE + (8 << 30),
                ws=None, wsb=0)
    args.update(over)
    return ssm.fwd_ext_raw(desc, args["x"], args["delta"], args["A"], args["B"], args["C"],
                           args["D"], args["z"], args["delta_bias"], True, args["y"], ext,
                           args["ws"], args["wsb"], None)


def test_extended_entry_point_validation():
    d = ssm.desc_contiguous(2, 64, 128, 16)
    H0, HF = FAKE + (12 << 30), FAKE + (13 << 30)
    assert _fwd_ext(d, ssm.ScanExt(2, 0, None, None)) == -3          # unknown discretisation
    assert _fwd_ext(d, ssm.ScanExt(0, 3, None, None)) == -3          # unknown algorithm
    assert _fwd_ext(d, ssm.ScanExt(0, -1, None, None)) == -3
    assert _fwd_ext(d, ssm.ScanExt(0, 2, None, None)) == -9          # chunked: diagonal A
    assert _fwd_ext(d, ssm.ScanExt(1, 0, H0 + 2, None)) == -5        # h0 not fp32-aligned
    assert _fwd_ext(d, ssm.ScanExt(1, 0, None, HF + 1)) == -5        # h_final not aligned
    assert _fwd_ext(d, ssm.ScanExt(0, 0, H0, H0 + 64)) == -6         # h_final overlaps h0
    assert _fwd_ext(d, ssm.ScanExt(0, 0, None, FAKE + 128)) == -6    # h_final overlaps x
    assert _fwd_ext(d, ssm.ScanExt(0, 0, None, FAKE + (8 << 30))) == -6  # h_final overlaps y
    assert _fwd_ext(d, ssm.ScanExt(0, 0, FAKE + (8 << 30) + 256, None)) == -6  # y overlaps h0
    assert _fwd_ext(d, ssm.ScanExt(0, 0, None, None), x=None) == -1
    big = ssm.desc_contiguous(1, 2048, 1 << 20, 16)
    need = ssm.workspace_size(big)
    assert _fwd_ext(big, None) == -7
    assert _fwd_ext(big, None, ws=FAKE + 64, wsb=need) == -6          # workspace overlaps x
    assert _fwd_ext(big, None, ws=FAKE + (20 << 30) + 2, wsb=need) == -5
    # nothing to compute: no pointers needed, and no final state requested
    e = ssm.desc_contiguous(0, 64, 128, 16)
    assert ssm.fwd_ext_raw(e, None, None, None, None, None, None, None, None, 1, None,
                           ssm.ScanExt(1, 0, None, None), None, 0, None) == 0
    e = ssm.desc_contiguous(3, 64, 0, 16)
    assert ssm.fwd_ext_raw(e, None, None, None, None, None, None, None, None, 1, None,
                           ssm.ScanExt(0, 0, None, None), None, 0, None) == 0
    assert ssm.fwd_ext_raw(e, None, None, None, None, None, None, None, None, 1, None,
                           ssm.ScanExt(0, 0, H0, H0 + 64), None, 0, None) == -6


def test_complex_mode_validation():
    """a_mode SSM_A_COMPLEX: B and C extents cover 2N rows, the forward scan takes only the
    delta * B rule without initial or final state, N <= 32, and needs no workspace; the decode
    step and the backward pass reject it."""
    c = ssm.SSM_A_COMPLEX
    d = ssm.desc_contiguous(2, 64, 128, 16, a_mode=c)
    assert d.B_stride_group == 32 * 128 and d.B_stride_batch == 32 * 128
    assert ssm.workspace_size(d) == 0
    H0 = FAKE + (12 << 30)
    assert _fwd_ext(d, ssm.ScanExt(1, 0, None, None)) == -9          # zero-order hold
    assert _fwd_ext(d, ssm.ScanExt(0, 2, None, None)) == -9          # chunked
    assert _fwd_ext(d, ssm.ScanExt(0, 0, H0, None)) == -9            # initial state
    assert _fwd_ext(d, ssm.ScanExt(0, 0, None, H0)) == -9            # final state
    assert _fwd(ssm.desc_contiguous(2, 64, 128, 33, a_mode=c)) == -9  # N > 32
    assert _fwd(ssm.desc_contiguous(1, 256, 128, 16, ngroups=8, a_mode=c)) == -9  # groups of 32
    assert _fwd(d, x=None) == -1
    assert _fwd(d, x=FAKE + 1) == -5
    assert _fwd(d, y=FAKE + (3 << 30) + 64) == -6                    # y overlaps B
    # B's 2N rows: y placed just past N rows of B still overlaps its imaginary parts
    assert _fwd(d, y=FAKE + (3 << 30) + 16 * 128 * 2) == -6
    # nothing to compute: no pointers needed
    e = ssm.desc_contiguous(3, 64, 0, 16, a_mode=c)
    assert ssm.fwd_raw(e, None, None, None, None, None, None, None, None, 1, None, None, 0,
                       None) == 0
    one = ssm.desc_contiguous(4, 64, 1, 16, a_mode=c)
    S = FAKE + (16 << 30)
    assert ssm.state_update_raw(one, S, FAKE, FAKE + (1 << 30), FAKE + (2 << 30),
                                FAKE + (3 << 30), FAKE + (4 << 30), None, None, None, True,
                                FAKE + (8 << 30), None) == -9
    out = ctypes.c_size_t(0)
    assert ssm.lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(out)) == -9


def test_state_update_validation():
    S = FAKE + (16 << 30)
    def call(desc, **over):
        args = dict(state=S, x=FAKE, delta=FAKE + (1 << 30), A=FAKE + (2 << 30),
                    B=FAKE + (3 << 30), C=FAKE + (4 << 30), y=FAKE + (8 << 30))
        args.update(over)
        return ssm.state_update_raw(desc, args["state"], args["x"], args["delta"], args["A"],
                                    args["B"], args["C"], None, None, None, True, args["y"], None)
    d = ssm.desc_contiguous(4, 64, 1, 16)
    assert call(ssm.desc_contiguous(4, 64, 2, 16)) == -2       # one step only
    assert call(d, state=None) == -1
    assert call(d, y=None) == -1
    assert call(d, state=S + 2) == -5
    assert call(d, state=FAKE + 16) == -6                      # state overlaps x
    assert call(d, state=FAKE + (8 << 30)) == -6               # state overlaps y
    assert call(d, y=FAKE + (2 << 30) + 64) == -6              # y overlaps A
    assert call(ssm.desc_contiguous(0, 64, 1, 16), state=None, x=None) == 0


def test_backward_validation():
    def call(desc, **over):
        a = dict(x=FAKE, delta=FAKE + (1 << 30), A=FAKE + (2 << 30), B=FAKE + (3 << 30),
                 C=FAKE + (4 << 30), D=None, z=None, bias=None, h0=None, dy=FAKE + (5 << 30),
                 dx=FAKE + (6 << 30), ddelta=FAKE + (7 << 30), dA=FAKE + (9 << 30),
                 dB=FAKE + (10 << 30), dC=FAKE + (11 << 30), dD=None, dz=None, dbias=None,
                 dh0=None, ws=FAKE + (20 << 30), wsb=1 << 40)
        a.update(over)
        return ssm.bwd_raw(desc, a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                           a["bias"], True, a["h0"], a["dy"], a["dx"], a["ddelta"], a["dA"],
                           a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"], a["dh0"], a["ws"],
                           a["wsb"], None)
    d = ssm.desc_contiguous(2, 64, 128, 16)
    assert ssm.bwd_workspace_size(d) > 0
    assert call(d, dA=None) == -1
    assert call(d, z=FAKE + (12 << 30)) == -1                                  # z without dz
    assert call(d, dx=None) == -1
    assert call(d, ws=None) == -7
    assert call(d, wsb=ssm.bwd_workspace_size(d) - 4) == -7
    assert call(d, dx=FAKE + (6 << 30) + 1) == -5
    assert call(d, dx=FAKE + 64) == -6                                         # dx overlaps x
    assert call(d, dB=FAKE + (11 << 30)) == -6                                 # dB overlaps dC
    assert call(d, ws=FAKE + (10 << 30)) == -6                                 # workspace overlaps dB
    assert ssm.bwd_workspace_size(ssm.desc_contiguous(2, 64, 0, 16)) == 0
    # gradients are written with the input strides, so those must give disjoint rows
    bc = ssm.desc_contiguous(2, 64, 128, 16)
    bc.B_stride_batch = 0                       # B broadcast over the batch: dB rows collide
    assert call(bc) == -4
    bc = ssm.desc_contiguous(2, 64, 128, 16)
    bc.C_stride_state = 64                      # C rows of consecutive states overlap
    assert call(bc) == -4
    ov = ssm.desc_contiguous(2, 64, 128, 16)
    ov.x_stride_dim = 100                       # overlapping x rows: dx rows collide
    assert call(ov) == -4
    ov = ssm.desc_contiguous(2, 64, 128, 16)
    ov.delta_stride_batch = 0                   # delta broadcast over the batch
    assert call(ov) == -4
    ov = ssm.desc_contiguous(2, 64, 128, 16)
    ov.z_stride_dim = 0
    assert call(ov, z=FAKE + (12 << 30), dz=FAKE + (13 << 30)) == -4
    assert call(ov, dx=FAKE + (6 << 30) + 1) == -5  # without z its strides are not checked
    # the forward call may read such inputs: only y's rows must be disjoint. (A NULL y makes the
    # call fail after the stride checks, so nothing is launched.)
    fw = ssm.desc_contiguous(2, 64, 128, 16)
    fw.B_stride_batch = 0
    fw.x_stride_dim = 100
    assert _fwd(fw, y=None) == -1


def test_disjoint_rows_accepts_any_dimension_order():
    """Output rows are checked as a set: a (dim, batch, L) order is as valid as (batch, dim, L),
    and an interleaving that makes two rows meet is rejected."""
    d = ssm.desc_contiguous(2, 64, 128, 16)
    d.y_stride_dim, d.y_stride_batch = 2 * 128, 128      # channel-major rows, disjoint
    assert _fwd(d, y=None) == -1                         # past the stride checks, no launch
    d.y_stride_batch = 100                               # batch rows overlap within a channel
    assert _fwd(d, y=None) == -4
    d.y_stride_batch, d.y_stride_dim = 64 * 128, 128     # (batch, dim, L) as usual
    assert _fwd(d, y=None) == -1
    d.y_stride_batch = 63 * 128 + 127                    # the last row of entry 0 meets entry 1
    assert _fwd(d, y=None) == -4


def test_workspace_size_depends_only_on_shape():
    assert ssm.workspace_size(ssm.desc_contiguous(8, 4096, 4096, 16)) == 0
    # the million-token scan: 16 segments; per (channel, segment) the summary (16 states and the
    # sum of delta, fp32), then 12 bytes of alignment slack, then the 32 states of 16 floats that
    # the output pass stores for the correcting pass (one per 1024 steps of a 65536-step segment)
    c3 = ssm.workspace_size(ssm.desc_contiguous(1, 2048, 1 << 20, 16))
    assert c3 == 2048 * 16 * 17 * 4 + 12 + 2048 * 16 * 32 * 16 * 4
    # fp32 io takes the four-wavefront kernel, whose split needs the summaries only
    f32 = ssm.workspace_size(ssm.desc_contiguous(1, 2048, 1 << 20, 16, io_dtype=ssm.SSM_DTYPE_F32))
    assert f32 > 0 and f32 % (2048 * 17 * 4) == 0
    assert ssm.workspace_size(ssm.desc_contiguous(0, 64, 10, 16)) == 0
    assert ssm.workspace_size(ssm.desc_contiguous(3, 64, 0, 16)) == 0


def test_empty_problem_needs_no_pointers():
    d = ssm.desc_contiguous(0, 64, 128, 16)
    assert ssm.fwd_raw(d, None, None, None, None, None, None, None, None, 1, None, None, 0, None) == 0
    d = ssm.desc_contiguous(4, 64, 0, 16)
    assert ssm.fwd_raw(d, None, None, None, None, None, None, None, None, 1, None, None, 0, None) == 0


def test_torch_front_end_checks_shapes():
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 8, 16, dtype=torch.bfloat16)
    A = torch.zeros(8, 4)
    B = torch.zeros(2, 1, 4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ssm.describe(x, x, torch.zeros(8, 5), B, B)
    with pytest.raises(TypeError):
        ssm.describe(x, x.float(), A, B, B)
    with pytest.raises(ValueError):
        ssm.describe(x, x, A, B, B[..., :8])
    with pytest.raises(ValueError):
        ssm.describe(x.transpose(1, 2).contiguous().transpose(1, 2), x, A, B, B)
    d = ssm.describe(x, torch.zeros(2, 2, 16, dtype=torch.bfloat16), torch.zeros(2), B, B)
    assert d.a_mode == ssm.SSM_A_HEAD and d.headdim == 4


def test_noalloc_rejects_problems_beyond_its_scratch_on_the_host():
    """The allocation-free entry point checks its fixed array's size before touching the GPU:
    512 segments x 64 channels x 129 floats (dstate 128, L = 2^18) exceed its 8 MiB."""
    d = ssm.desc_contiguous(1, 64, 1 << 18, 128, headdim=64, io_dtype=ssm.SSM_DTYPE_F32,
                            a_mode=ssm.SSM_A_HEAD)
    assert ssm.workspace_size(d) > ssm.NOALLOC_SCRATCH_BYTES
    args = (FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30), None,
            None, None, True, FAKE + (8 << 30), None, None)
    assert ssm.fwd_noalloc_raw(d, *args) == -10
    bad = ssm.desc_contiguous(1, 64, 128, 200)      # argument errors come first
    assert ssm.fwd_noalloc_raw(bad, *args) == -2
    # the summaries of every segment plan with dstate <= 32 fit (the million-token scan's stored
    # states, 64 MiB, do not: that call runs with the summaries only)
    for (b, dim, L, N) in [(1, 64, 1 << 22, 32), (3, 64, 1 << 20, 32)]:
        assert ssm.workspace_size(ssm.desc_contiguous(b, dim, L, N)) <= ssm.NOALLOC_SCRATCH_BYTES
    c3 = ssm.workspace_size(ssm.desc_contiguous(1, 2048, 1 << 20, 16))
    assert c3 > ssm.NOALLOC_SCRATCH_BYTES >= 2048 * 16 * 17 * 4
