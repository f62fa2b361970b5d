"""Python binding of the MI355X selective-scan library (``lib/libssm_scan.so``).

Argument marshalling only: every step of the scan runs in the library's HIP kernels. PyTorch
provides device memory and the current stream. There is no fallback: if the library is not
built, every entry point raises.

The C ABI is declared in ``include/ssm_scan.h``; the names here mirror it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libssm_scan.so")

SSM_OK = 0
SSM_DTYPE_F32, SSM_DTYPE_BF16 = 0, 1
SSM_A_DIAG, SSM_A_HEAD, SSM_A_COMPLEX = 0, 1, 2
SSM_DISC_DELTA_B, SSM_DISC_ZOH = 0, 1
SSM_ALGO_AUTO, SSM_ALGO_RECURRENT, SSM_ALGO_CHUNKED = 0, 1, 2
ALGORITHMS = {"auto": SSM_ALGO_AUTO, "recurrent": SSM_ALGO_RECURRENT, "chunked": SSM_ALGO_CHUNKED}
SSM_MAX_DSTATE = 128
SSM_MAX_COMPLEX_DSTATE = 32

STATUS_NAMES = {
    0: "SSM_OK", -1: "SSM_ERR_NULL_ARG", -2: "SSM_ERR_BAD_SHAPE", -3: "SSM_ERR_BAD_DTYPE",
    -4: "SSM_ERR_BAD_STRIDE", -5: "SSM_ERR_MISALIGNED", -6: "SSM_ERR_ALIAS",
    -7: "SSM_ERR_WORKSPACE", -8: "SSM_ERR_HIP", -9: "SSM_ERR_UNSUPPORTED",
    -10: "SSM_ERR_SCRATCH_LIMIT",
}
NOALLOC_SCRATCH_BYTES = 8 << 20  # SSM_NOALLOC_SCRATCH_BYTES


class ScanDesc(ctypes.Structure):
    """Mirror of ``ssm_scan_desc``."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("headdim", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32), ("a_mode", ctypes.c_int32),
        ("x_stride_batch", ctypes.c_int64), ("x_stride_dim", ctypes.c_int64),
        ("delta_stride_batch", ctypes.c_int64), ("delta_stride_dim", ctypes.c_int64),
        ("B_stride_batch", ctypes.c_int64), ("B_stride_group", ctypes.c_int64),
        ("B_stride_state", ctypes.c_int64),
        ("C_stride_batch", ctypes.c_int64), ("C_stride_group", ctypes.c_int64),
        ("C_stride_state", ctypes.c_int64),
        ("z_stride_batch", ctypes.c_int64), ("z_stride_dim", ctypes.c_int64),
        ("y_stride_batch", ctypes.c_int64), ("y_stride_dim", ctypes.c_int64),
    ]


class ScanExt(ctypes.Structure):
    """Mirror of ``ssm_scan_ext``."""
    _fields_ = [("discretization", ctypes.c_int32), ("algorithm", ctypes.c_int32),
                ("h0", ctypes.c_void_p), ("h_final", ctypes.c_void_p)]


class BwdExt(ctypes.Structure):
    """Mirror of ``ssm_bwd_ext``."""
    _fields_ = [("discretization", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("dh_final", ctypes.c_void_p)]


class ScanError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def lib():
    """ctypes handle of the built library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(ScanDesc)
        h.ssm_scan_desc_init_contiguous.argtypes = [dp, i64, i64, i64, i64, i64, i64, i32, i32]
        h.ssm_scan_desc_init_contiguous.restype = ctypes.c_int
        h.ssm_selective_scan_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
        h.ssm_selective_scan_workspace_size.restype = ctypes.c_int
        h.ssm_selective_scan_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        h.ssm_selective_scan_fwd.restype = ctypes.c_int
        h.ssm_selective_scan_fwd_ext.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                 ctypes.POINTER(ScanExt), vp, sz, vp]
        h.ssm_selective_scan_fwd_ext.restype = ctypes.c_int
        h.ssm_selective_scan_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                     ctypes.POINTER(ScanExt), vp]
        h.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        h.ssm_selective_state_update.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
        h.ssm_selective_state_update.restype = ctypes.c_int
        h.ssm_selective_scan_bwd_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
        h.ssm_selective_scan_bwd_workspace_size.restype = ctypes.c_int
        h.ssm_selective_scan_bwd.argtypes = [dp] + [vp] * 8 + [i32] + [vp] * 11 + [vp, sz, vp]
        h.ssm_selective_scan_bwd.restype = ctypes.c_int
        h.ssm_selective_scan_bwd_ext.argtypes = ([dp] + [vp] * 8 + [i32] + [vp] * 11 +
                                                 [ctypes.POINTER(BwdExt), vp, sz, vp])
        h.ssm_selective_scan_bwd_ext.restype = ctypes.c_int
        h.ssm_status_string.argtypes = [ctypes.c_int]
        h.ssm_status_string.restype = ctypes.c_char_p
        h.ssm_abi_version.argtypes = []
        h.ssm_wave_simd_ids.restype = ctypes.c_int
        h.ssm_wave_simd_ids.argtypes = [vp, i32, vp]
        h.ssm_abi_version.restype = ctypes.c_int
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().ssm_status_string(int(status)).decode()


def wave_simd_ids_raw(out, nworkgroups: int, stream) -> int:
    """ssm_wave_simd_ids: the SIMD of each wavefront of `nworkgroups` 8-wavefront workgroups into
    the device int32 buffer at address `out` (8 per workgroup); returns the status."""
    return int(lib().ssm_wave_simd_ids(out, int(nworkgroups), stream))


def abi_version() -> int:
    return int(lib().ssm_abi_version())


def desc_contiguous(batch, dim, seqlen, dstate, ngroups=1, headdim=1, io_dtype=SSM_DTYPE_BF16,
                    a_mode=SSM_A_DIAG) -> ScanDesc:
    d = ScanDesc()
    rc = lib().ssm_scan_desc_init_contiguous(ctypes.byref(d), batch, dim, seqlen, dstate, ngroups,
                                             headdim, io_dtype, a_mode)
    if rc != SSM_OK:
        raise ScanError(rc, "ssm_scan_desc_init_contiguous")
    return d


def workspace_size(desc: ScanDesc) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().ssm_selective_scan_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if rc != SSM_OK:
        raise ScanError(rc, "ssm_selective_scan_workspace_size")
    return int(out.value)


def fwd_raw(desc: ScanDesc, x, delta, A, B, C, D, z, delta_bias, delta_softplus: bool, y,
            workspace, workspace_bytes: int, stream) -> int:
    """Direct call of ``ssm_selective_scan_fwd`` with integer device addresses (or None).
    Returns the status code without raising."""
    return int(lib().ssm_selective_scan_fwd(ctypes.byref(desc), x, delta, A, B, C, D, z,
                                            delta_bias, int(bool(delta_softplus)), y, workspace,
                                            int(workspace_bytes), stream))


def fwd_ext_raw(desc: ScanDesc, x, delta, A, B, C, D, z, delta_bias, delta_softplus: bool, y,
                ext: Optional[ScanExt], workspace, workspace_bytes: int, stream) -> int:
    """Direct call of ``ssm_selective_scan_fwd_ext``; returns the status code without raising."""
    return int(lib().ssm_selective_scan_fwd_ext(
        ctypes.byref(desc), x, delta, A, B, C, D, z, delta_bias, int(bool(delta_softplus)), y,
        ctypes.byref(ext) if ext is not None else None, workspace, int(workspace_bytes), stream))


def fwd_noalloc_raw(desc: ScanDesc, x, delta, A, B, C, D, z, delta_bias, delta_softplus: bool,
                    y, ext: Optional[ScanExt], stream) -> int:
    """Direct call of ``ssm_selective_scan_fwd_noalloc`` (the workspace is the library's fixed
    device array); returns the status code without raising."""
    return int(lib().ssm_selective_scan_fwd_noalloc(
        ctypes.byref(desc), x, delta, A, B, C, D, z, delta_bias, int(bool(delta_softplus)), y,
        ctypes.byref(ext) if ext is not None else None, stream))


def bwd_workspace_size(desc: ScanDesc) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if rc != SSM_OK:
        raise ScanError(rc, "ssm_selective_scan_bwd_workspace_size")
    return int(out.value)


def bwd_raw(desc: ScanDesc, x, delta, A, B, C, D, z, delta_bias, delta_softplus: bool, h0, dy,
            dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes: int,
            stream) -> int:
    """Direct call of ``ssm_selective_scan_bwd``; returns the status code without raising."""
    return int(lib().ssm_selective_scan_bwd(
        ctypes.byref(desc), x, delta, A, B, C, D, z, delta_bias, int(bool(delta_softplus)), h0, dy,
        dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, workspace, int(workspace_bytes), stream))


def bwd_ext_raw(desc: ScanDesc, x, delta, A, B, C, D, z, delta_bias, delta_softplus: bool, h0,
                dy, dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, ext: Optional[BwdExt],
                workspace, workspace_bytes: int, stream) -> int:
    """Direct call of ``ssm_selective_scan_bwd_ext``; returns the status code without raising."""
    return int(lib().ssm_selective_scan_bwd_ext(
        ctypes.byref(desc), x, delta, A, B, C, D, z, delta_bias, int(bool(delta_softplus)), h0, dy,
        dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
        ctypes.byref(ext) if ext is not None else None, workspace, int(workspace_bytes), stream))


def state_update_raw(desc: ScanDesc, state, x, delta, A, B, C, D, z, delta_bias,
                     delta_softplus: bool, y, stream) -> int:
    """Direct call of ``ssm_selective_state_update``; returns the status code without raising."""
    return int(lib().ssm_selective_state_update(ctypes.byref(desc), state, x, delta, A, B, C, D, z,
                                                delta_bias, int(bool(delta_softplus)), y, stream))


# ---------------------------------------------------------------------------------------------
# torch front end (device memory and streams only)

def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def describe(x, delta, A, B, C, z=None, y=None) -> ScanDesc:
    """Descriptor of torch tensors: x (batch, dim, L), delta (batch, dim | nheads, L),
    A (dim, N) or (nheads,), B/C (batch, ngroups, N, L), z and y like x.

    A complex A, either a complex64 (dim, N) tensor or a float32 (dim, N, 2) tensor of
    (real, imaginary) pairs, selects SSM_A_COMPLEX: B and C are then real tensors of shape
    (batch, ngroups, 2N, L), the real parts in rows 0..N-1 and the imaginary parts in rows N..2N-1.
    """
    import torch
    if x.dtype == torch.bfloat16:
        io = SSM_DTYPE_BF16
    elif x.dtype == torch.float32:
        io = SSM_DTYPE_F32
    else:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z), ("y", y)):
        if t is not None and t.dtype != x.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {x.dtype}")
    if A.dtype == torch.complex64:
        A = torch.view_as_real(A)
    if A.dtype != torch.float32:
        raise TypeError("A must be float32 (or complex64)")
    if x.dim() != 3 or delta.dim() != 3 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("expected x/delta (batch, rows, L) and B/C (batch, groups, N, L)")
    batch, dim, L = x.shape
    ngroups, N = B.shape[1], B.shape[2]
    bc_rows = N
    if A.dim() == 3:
        a_mode, headdim = SSM_A_COMPLEX, 1
        if B.shape[2] % 2:
            raise ValueError("complex A: B and C need 2N rows (real parts, then imaginary)")
        N = B.shape[2] // 2
        if tuple(A.shape) != (dim, N, 2):
            raise ValueError(f"complex A must be (dim, N) = {(dim, N)}, got {tuple(A.shape[:2])}")
    elif A.dim() == 1:
        a_mode = SSM_A_HEAD
        nheads = A.shape[0]
        if nheads == 0 or dim % nheads:
            raise ValueError("A (nheads,) must divide dim")
        headdim = dim // nheads
    elif A.dim() == 2:
        a_mode, headdim = SSM_A_DIAG, 1
        if tuple(A.shape) != (dim, N):
            raise ValueError(f"A must be (dim, N) = {(dim, N)}, got {tuple(A.shape)}")
    else:
        raise ValueError("A must be (dim, N), (nheads,) or complex (dim, N)")
    rows = dim // headdim
    if tuple(delta.shape) != (batch, rows, L):
        raise ValueError(f"delta must be {(batch, rows, L)}, got {tuple(delta.shape)}")
    if (tuple(B.shape) != (batch, ngroups, bc_rows, L)
            or tuple(C.shape) != (batch, ngroups, bc_rows, L)):
        raise ValueError(f"B and C must both be (batch, ngroups, {bc_rows}, L)")
    for name, t in (("x", x), ("delta", delta), ("B", B), ("C", C), ("z", z), ("y", y)):
        if t is not None and t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have unit stride along L")
    if not A.is_contiguous():
        raise ValueError("A must be contiguous")
    d = ScanDesc()
    d.batch, d.dim, d.seqlen, d.dstate, d.ngroups, d.headdim = batch, dim, L, N, ngroups, headdim
    d.io_dtype, d.a_mode = io, a_mode
    d.x_stride_batch, d.x_stride_dim = x.stride(0), x.stride(1)
    d.delta_stride_batch, d.delta_stride_dim = delta.stride(0), delta.stride(1)
    d.B_stride_batch, d.B_stride_group, d.B_stride_state = B.stride(0), B.stride(1), B.stride(2)
    d.C_stride_batch, d.C_stride_group, d.C_stride_state = C.stride(0), C.stride(1), C.stride(2)
    if z is not None:
        if tuple(z.shape) != (batch, dim, L):
            raise ValueError("z must be shaped like x")
        d.z_stride_batch, d.z_stride_dim = z.stride(0), z.stride(1)
    if y is not None:
        if tuple(y.shape) != (batch, dim, L):
            raise ValueError("y must be shaped like x")
        d.y_stride_batch, d.y_stride_dim = y.stride(0), y.stride(1)
    return d


def selective_scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                       *, zoh: bool = False, h0=None, final_state=None, out=None,
                       algorithm: str = "auto", workspace=None, stream=None):
    """y = selective scan of torch device tensors (see ``include/ssm_scan.h``).

    ``zoh`` selects the zero-order-hold B discretisation. ``h0`` (batch, dim, N) float32 is the
    initial state. ``final_state`` is True (allocate) or a (batch, dim, N) float32 tensor that
    receives the state after the last step; the call then returns ``(y, final_state)``.
    ``algorithm`` is "auto", "recurrent" or "chunked" (``ssm_algorithm``: the chunked matrix
    form needs bf16 io and one A per head, see the header for the full conditions).
    ``out`` receives y if given (shape and dtype of x). ``workspace`` may be a uint8 device
    tensor of at least ``workspace_size`` bytes; otherwise one is allocated. ``stream`` defaults
    to the current torch stream. Raises ScanError with the library's status on failure.
    """
    import torch
    if algorithm not in ALGORITHMS:
        raise ValueError(f"algorithm must be one of {sorted(ALGORITHMS)}, got {algorithm!r}")
    algo = ALGORITHMS[algorithm]
    y = out if out is not None else torch.empty_like(x, memory_format=torch.contiguous_format)
    desc = describe(x, delta, A, B, C, z, y)
    for name, t in (("D", D), ("delta_bias", delta_bias), ("h0", h0)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    state_shape = (desc.batch, desc.dim, desc.dstate)
    if h0 is not None and tuple(h0.shape) != state_shape:
        raise ValueError(f"h0 must be {state_shape}, got {tuple(h0.shape)}")
    hfin = None
    if final_state is True:
        hfin = torch.empty(state_shape, dtype=torch.float32, device=x.device)
    elif final_state is not None and final_state is not False:
        hfin = final_state
        if (hfin.dtype != torch.float32 or not hfin.is_contiguous()
                or tuple(hfin.shape) != state_shape):
            raise TypeError(f"final_state must be a contiguous float32 tensor of shape {state_shape}")
    need = workspace_size(desc)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    args = (desc, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), delta_softplus, _ptr(y))
    tail = (_ptr(workspace) if need else None, need, sp)
    if zoh or h0 is not None or hfin is not None or algo != SSM_ALGO_AUTO:
        ext = ScanExt(SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B, algo, _ptr(h0), _ptr(hfin))
        rc = fwd_ext_raw(*args, ext, *tail)
    else:
        rc = fwd_raw(*args, *tail)
    if rc != SSM_OK:
        raise ScanError(rc, "ssm_selective_scan_fwd")
    return (y, hfin) if hfin is not None else y


def describe_step(state, x, delta, A, B, C, z=None, y=None) -> ScanDesc:
    """Descriptor (seqlen 1) of one decoding step: x, z, y (batch, dim); delta (batch, dim) or
    (batch, nheads); B, C (batch, ngroups, N); state (batch, dim, N) float32."""
    x3, d3 = x.unsqueeze(-1), delta.unsqueeze(-1)
    B4, C4 = B.unsqueeze(-1), C.unsqueeze(-1)
    desc = describe(x3, d3, A, B4, C4, None if z is None else z.unsqueeze(-1),
                    None if y is None else y.unsqueeze(-1))
    if tuple(state.shape) != (desc.batch, desc.dim, desc.dstate):
        raise ValueError(f"state must be {(desc.batch, desc.dim, desc.dstate)}, got {tuple(state.shape)}")
    return desc


def selective_state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                           delta_softplus=True, *, out=None, stream=None):
    """One recurrent step per sequence (see ``ssm_selective_state_update``): updates ``state``
    (batch, dim, N) float32 in place and returns y (batch, dim) in the dtype of x."""
    import torch
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise TypeError("state must be a contiguous float32 tensor")
    for name, t in (("D", D), ("delta_bias", delta_bias)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    y = out if out is not None else torch.empty_like(x, memory_format=torch.contiguous_format)
    desc = describe_step(state, x, delta, A, B, C, z, y)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    rc = state_update_raw(desc, _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                          _ptr(D), _ptr(z), _ptr(delta_bias), delta_softplus, _ptr(y), sp)
    if rc != SSM_OK:
        raise ScanError(rc, "ssm_selective_state_update")
    return y


def selective_scan_bwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                       dy=None, *, h0=None, want_dh0=False, zoh: bool = False, dh_final=None,
                       workspace=None, stream=None) -> dict:
    """Gradients of ``selective_scan_fwd`` for dy, the gradient of y (and ``dh_final``, the
    gradient of its final state, if given). ``zoh`` selects the zero-order-hold rule of the
    forward call. Returns a dict: dx, ddelta, dz (io dtype, like x, delta, z), dA (like A), dB,
    dC, dD, ddelta_bias (float32) and dh0 when ``want_dh0``. See ``ssm_selective_scan_bwd_ext``."""
    import torch
    desc = describe(x, delta, A, B, C, z, dy)
    for name, t in (("D", D), ("delta_bias", delta_bias), ("h0", h0), ("dh_final", dh_final)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    g = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(delta),
         "dA": torch.empty_like(A),
         "dB": torch.empty(B.shape, dtype=torch.float32, device=x.device),
         "dC": torch.empty(C.shape, dtype=torch.float32, device=x.device)}
    if x.stride() != g["dx"].stride() or delta.stride() != g["ddelta"].stride():
        raise ValueError("x and delta must be contiguous (their gradients use their strides)")
    if B.stride() != g["dB"].stride() or C.stride() != g["dC"].stride():
        raise ValueError("B and C must be contiguous (their gradients use their strides)")
    if D is not None:
        g["dD"] = torch.empty_like(D)
    if z is not None:
        g["dz"] = torch.empty_like(z)
        if z.stride() != g["dz"].stride():
            raise ValueError("z must be contiguous (its gradient uses its strides)")
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty_like(delta_bias)
    if want_dh0:
        g["dh0"] = torch.empty((desc.batch, desc.dim, desc.dstate), dtype=torch.float32,
                               device=x.device)
    need = bwd_workspace_size(desc)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    if dh_final is not None and tuple(dh_final.shape) != (desc.batch, desc.dim, desc.dstate):
        raise ValueError("dh_final must be (batch, dim, N)")
    ext = BwdExt(SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B, 0, _ptr(dh_final))
    rc = bwd_ext_raw(desc, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                     _ptr(delta_bias), delta_softplus, _ptr(h0), _ptr(dy), _ptr(g["dx"]),
                     _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                     _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")),
                     _ptr(g.get("dh0")), ext, _ptr(workspace) if need else None, need, sp)
    if rc != SSM_OK:
        raise ScanError(rc, "ssm_selective_scan_bwd")
    return g
