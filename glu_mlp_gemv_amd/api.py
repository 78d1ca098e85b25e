"""Python face of the C ABI in include/glu_gemv.h (argument marshalling only).

Every step of the projection runs in the HIP kernels of ``libglu_gemv.so``;
this module checks tensors, passes their device pointers and torch's current
HIP stream, and turns a non-OK status into an exception.  If the library is
missing or cannot be loaded, calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads torch's HIP runtime first, so the library binds to the same one

from . import build as _build

# another build of the same sources (the host-sanitized one of glu_mlp_gemv_amd/sanitize.py) may be
# named in GLU_GEMV_LIBRARY
LIBRARY_PATH = os.environ.get("GLU_GEMV_LIBRARY") or _build.LIBRARY

# enum values of include/glu_gemv.h
GLU_OK = 0
GLU_ERR_UNSUPPORTED = 6
GLU_ERR_BAD_STRIDE = 7
GLU_ERR_WORKSPACE = 8
GLU_ERR_SCRATCH_LIMIT = 9
NOALLOC_SCRATCH_BYTES = 48 << 20  # the device array glu_dual_gemv_backward_noalloc works in
(KERNEL_NONE, KERNEL_ZERO, KERNEL_VALU, KERNEL_MFMA, KERNEL_GENERIC, KERNEL_GEMM, KERNEL_BACKWARD,
 KERNEL_CEILING) = range(8)
KERNEL_NAMES = {KERNEL_NONE: "none", KERNEL_ZERO: "zero", KERNEL_VALU: "valu",
                KERNEL_MFMA: "mfma", KERNEL_GENERIC: "generic", KERNEL_GEMM: "gemm", KERNEL_BACKWARD: "backward",
                KERNEL_CEILING: "ceiling"}

EXPORTED_SYMBOLS = (
    "glu_dual_gemv",
    "glu_grouped_gemv",
    "glu_grouped_gemv_tuned",
    "glu_grouped_gemv_plan",
    "glu_grouped_gemv_plan_tuned",
    "glu_grouped_gemv_describe",
    "glu_dual_gemv_strided",
    "glu_dual_gemv_strided_tuned",
    "glu_status_string",
    "glu_last_hip_error",
    "glu_version",
    "glu_dual_gemv_plan",
    "glu_dual_gemv_tuned",
    "glu_dual_gemv_plan_tuned",
    "glu_dual_gemv_describe",
    "glu_dual_gemv_backward",
    "glu_dual_gemv_backward_workspace",
    "glu_dual_gemv_backward_plan",
    "glu_read_ceiling",
    "glu_read_ceiling_plan",
    "glu_dual_gemv_backward_noalloc",
    "glu_unit_ceiling",
    "glu_unit_ceiling_work",
    "glu_copy_ceiling",
)


class GluError(RuntimeError):
    """A non-OK glu_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("m_per_launch", ctypes.c_int), ("launches", ctypes.c_int),
                ("grid", ctypes.c_int), ("block", ctypes.c_int), ("accum_depth", ctypes.c_int)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["kernel_name"] = KERNEL_NAMES.get(self.kernel, "?")
        return d


class Tuning(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("rows_per_wave", ctypes.c_int), ("waves_per_block", ctypes.c_int),
                ("grid", ctypes.c_int), ("mfma_segments", ctypes.c_int), ("mfma_hidden", ctypes.c_int),
                ("mfma_depth", ctypes.c_int), ("gemm_tile_n", ctypes.c_int), ("gemm_tile_m", ctypes.c_int),
                ("xcd_bands", ctypes.c_int), ("gemv_dot", ctypes.c_int), ("mfma_order", ctypes.c_int)]


class Projection(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("out", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("ldw", ctypes.c_int64), ("ldo", ctypes.c_int64)]


GROUP_MAX = 8

_LIB: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(f"HIP library {LIBRARY_PATH} is not built; run __graft_entry__.build() "
                           "(or python -m glu_mlp_gemv_amd.build)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    u16p, i64, vp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p
    lib.glu_dual_gemv.argtypes = [u16p, u16p, u16p, u16p, i64, i64, i64, vp]
    lib.glu_dual_gemv.restype = ctypes.c_int
    lib.glu_dual_gemv_tuned.argtypes = [u16p, u16p, u16p, u16p, i64, i64, i64, vp, ctypes.POINTER(Tuning)]
    lib.glu_dual_gemv_tuned.restype = ctypes.c_int
    lib.glu_dual_gemv_strided.argtypes = [u16p, i64, u16p, i64, u16p, i64, u16p, i64, i64, i64, i64, vp]
    lib.glu_dual_gemv_strided.restype = ctypes.c_int
    lib.glu_dual_gemv_strided_tuned.argtypes = [u16p, i64, u16p, i64, u16p, i64, u16p, i64, i64, i64, i64, vp,
                                                ctypes.POINTER(Tuning)]
    lib.glu_dual_gemv_strided_tuned.restype = ctypes.c_int
    projp = ctypes.POINTER(Projection)
    lib.glu_grouped_gemv.argtypes = [u16p, i64, projp, ctypes.c_int, i64, i64, vp]
    lib.glu_grouped_gemv.restype = ctypes.c_int
    lib.glu_grouped_gemv_tuned.argtypes = [u16p, i64, projp, ctypes.c_int, i64, i64, vp, ctypes.POINTER(Tuning)]
    lib.glu_grouped_gemv_tuned.restype = ctypes.c_int
    lib.glu_grouped_gemv_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Plan)]
    lib.glu_grouped_gemv_plan.restype = ctypes.c_int
    lib.glu_grouped_gemv_plan_tuned.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Tuning),
                                                ctypes.POINTER(Plan)]
    lib.glu_grouped_gemv_plan_tuned.restype = ctypes.c_int
    lib.glu_status_string.argtypes = [ctypes.c_int]
    lib.glu_status_string.restype = ctypes.c_char_p
    lib.glu_last_hip_error.argtypes = []
    lib.glu_last_hip_error.restype = ctypes.c_int
    lib.glu_version.argtypes = []
    lib.glu_version.restype = ctypes.c_int
    lib.glu_dual_gemv_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Plan)]
    lib.glu_dual_gemv_plan.restype = ctypes.c_int
    lib.glu_dual_gemv_plan_tuned.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Tuning),
                                             ctypes.POINTER(Plan)]
    lib.glu_dual_gemv_plan_tuned.restype = ctypes.c_int
    lib.glu_dual_gemv_describe.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Tuning), ctypes.c_char_p,
                                           ctypes.c_int]
    lib.glu_dual_gemv_describe.restype = ctypes.c_int
    lib.glu_grouped_gemv_describe.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Tuning), ctypes.c_char_p,
                                              ctypes.c_int]
    lib.glu_grouped_gemv_describe.restype = ctypes.c_int
    lib.glu_dual_gemv_backward.argtypes = [u16p, u16p, u16p, u16p, u16p, u16p, u16p, i64, i64, i64, vp, i64, vp]
    lib.glu_dual_gemv_backward.restype = ctypes.c_int
    lib.glu_dual_gemv_backward_workspace.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.glu_dual_gemv_backward_workspace.restype = ctypes.c_int
    lib.glu_dual_gemv_backward_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    lib.glu_dual_gemv_backward_plan.restype = ctypes.c_int
    lib.glu_dual_gemv_backward_noalloc.argtypes = [u16p, u16p, u16p, u16p, u16p, u16p, u16p, i64, i64, i64, vp]
    lib.glu_dual_gemv_backward_noalloc.restype = ctypes.c_int
    lib.glu_read_ceiling.argtypes = [vp, vp, i64, i64, vp, ctypes.POINTER(Tuning), vp]
    lib.glu_read_ceiling.restype = ctypes.c_int
    lib.glu_read_ceiling_plan.argtypes = [i64, i64, ctypes.POINTER(Tuning), ctypes.POINTER(Plan)]
    lib.glu_read_ceiling_plan.restype = ctypes.c_int
    lib.glu_unit_ceiling.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, vp, vp]
    lib.glu_unit_ceiling.restype = ctypes.c_int
    lib.glu_unit_ceiling_work.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, ctypes.POINTER(ctypes.c_double)]
    lib.glu_unit_ceiling_work.restype = ctypes.c_int
    lib.glu_copy_ceiling.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.POINTER(Tuning), vp]
    lib.glu_copy_ceiling.restype = ctypes.c_int
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return library().glu_status_string(int(status)).decode()


def _raise_for(status: int):
    if status != GLU_OK:
        msg = status_string(status)
        hip = library().glu_last_hip_error()
        if hip:
            msg += f" (hipError {hip})"
        raise GluError(status, msg)


def make_tuning(**kw) -> Tuning:
    t = Tuning()
    for k, v in kw.items():
        if not hasattr(t, k):
            raise TypeError(f"unknown tuning field {k}")
        setattr(t, k, int(v))
    return t


def plan(M: int, N: int, K: int, aligned16: bool = True, tuning: Optional[Tuning] = None) -> dict:
    """The launch the library would make for a shape (host only, no GPU needed)."""
    p = Plan()
    lib = library()
    if tuning is None:
        st = lib.glu_dual_gemv_plan(M, N, K, int(aligned16), ctypes.byref(p))
    else:
        st = lib.glu_dual_gemv_plan_tuned(M, N, K, int(aligned16), ctypes.byref(tuning), ctypes.byref(p))
    _raise_for(st)
    d = p.as_dict()
    buf = ctypes.create_string_buffer(256)
    st = lib.glu_dual_gemv_describe(M, N, K, int(aligned16), ctypes.byref(tuning) if tuning is not None else None,
                                    buf, 256)
    _raise_for(st)
    d["kernel_symbol"] = buf.value.decode()
    return d


def _check(name: str, t: torch.Tensor, ndims):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dim() not in ndims:
        raise ValueError(f"{name} must have {' or '.join(map(str, ndims))} dims, got {t.dim()}")


def _row_stride(name: str, t: torch.Tensor) -> int:
    """Element stride between rows of a 2-D view whose rows are contiguous; refuses any other layout."""
    if t.dim() == 1:
        if t.shape[0] > 1 and t.stride(0) != 1:
            raise ValueError(f"{name}: elements must be contiguous, got stride {t.stride(0)}")
        return t.shape[0]
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: the elements of a row must be contiguous, got strides {tuple(t.stride())}")
    if rows <= 1:
        return cols  # a single row: its stride is never used
    if t.stride(0) < cols:
        raise ValueError(f"{name}: rows overlap (row stride {t.stride(0)} < row length {cols})")
    return t.stride(0)


def dual_gemv(hidden: torch.Tensor, gate_w: torch.Tensor, up_w: torch.Tensor,
              out: Optional[torch.Tensor] = None, tuning: Optional[Tuning] = None,
              stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """out = bf16(bf16(silu(bf16(hidden @ gate_w.T))) * bf16(hidden @ up_w.T)).

    hidden [M, K] (or [K], then the result is [N]), gate_w and up_w [N, K], all
    bf16 on one GPU.  Each may be a row-strided view (rows contiguous, any row
    stride at least the row length, e.g. a slice of a wider fused block): the
    stride the tensor reports is what the kernel uses, and any other layout is
    refused.  ``out`` [M, N] (or [N]), written in place if given, may be
    row-strided too.  Runs asynchronously on ``stream`` (default: torch's
    current stream).
    """
    _check("hidden", hidden, (1, 2))
    _check("gate_w", gate_w, (2,))
    _check("up_w", up_w, (2,))
    vec = hidden.dim() == 1
    M = 1 if vec else hidden.shape[0]
    K = hidden.shape[-1]
    N = gate_w.shape[0]
    if tuple(gate_w.shape) != (N, K) or tuple(up_w.shape) != (N, K):
        raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, gate_w {tuple(gate_w.shape)}, "
                         f"up_w {tuple(up_w.shape)}")
    dev = hidden.device
    if gate_w.device != dev or up_w.device != dev:
        raise ValueError("hidden, gate_w and up_w must be on the same device")
    want = (N,) if vec else (M, N)
    if out is None:
        out = torch.empty(want, dtype=torch.bfloat16, device=dev)
    else:
        _check("out", out, (len(want),))
        if tuple(out.shape) != want or out.device != dev:
            raise ValueError(f"out must be {want} on {dev}, got {tuple(out.shape)} on {out.device}")
    ldh = _row_stride("hidden", hidden)
    ldg = _row_stride("gate_w", gate_w)
    ldu = _row_stride("up_w", up_w)
    ldo = _row_stride("out", out)
    lib = library()
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        if tuning is None:
            st = lib.glu_dual_gemv_strided(hidden.data_ptr(), ldh, gate_w.data_ptr(), ldg, up_w.data_ptr(), ldu,
                                           out.data_ptr(), ldo, M, N, K, s.cuda_stream)
        else:
            st = lib.glu_dual_gemv_strided_tuned(hidden.data_ptr(), ldh, gate_w.data_ptr(), ldg, up_w.data_ptr(),
                                                 ldu, out.data_ptr(), ldo, M, N, K, s.cuda_stream,
                                                 ctypes.byref(tuning))
    _raise_for(st)
    return out


def backward_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes glu_dual_gemv_backward needs (host only)."""
    b = ctypes.c_int64(0)
    _raise_for(library().glu_dual_gemv_backward_workspace(M, N, K, ctypes.byref(b)))
    return int(b.value)


def backward_plan(M: int, N: int, K: int) -> dict:
    """The backward's launch for a shape (host only)."""
    p = Plan()
    _raise_for(library().glu_dual_gemv_backward_plan(M, N, K, ctypes.byref(p)))
    return p.as_dict()


def _backward_args(hidden, gate_w, up_w, dout, dhidden, dgate_w, dup_w):
    """Checked shapes of a backward call and its output tensors (allocated unless given)."""
    _check("hidden", hidden, (1, 2))
    _check("gate_w", gate_w, (2,))
    _check("up_w", up_w, (2,))
    _check("dout", dout, (1, 2))
    vec = hidden.dim() == 1
    M = 1 if vec else hidden.shape[0]
    K = hidden.shape[-1]
    N = gate_w.shape[0]
    dev = hidden.device
    if tuple(gate_w.shape) != (N, K) or tuple(up_w.shape) != (N, K):
        raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, gate_w {tuple(gate_w.shape)}, "
                         f"up_w {tuple(up_w.shape)}")
    if tuple(dout.shape) != ((N,) if vec else (M, N)):
        raise ValueError(f"dout must be {(N,) if vec else (M, N)}, got {tuple(dout.shape)}")
    for name, t in (("gate_w", gate_w), ("up_w", up_w), ("hidden", hidden), ("dout", dout)):
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def out_tensor(name, t, shape):
        if t is None:
            return torch.empty(shape, dtype=torch.bfloat16, device=dev)
        _check(name, t, (len(shape),))
        if tuple(t.shape) != tuple(shape) or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {tuple(shape)} tensor on {dev}")
        return t
    dhidden = out_tensor("dhidden", dhidden, tuple(hidden.shape))
    dgate_w = out_tensor("dgate_w", dgate_w, (N, K))
    dup_w = out_tensor("dup_w", dup_w, (N, K))
    return M, N, K, dev, dhidden, dgate_w, dup_w


def dual_gemv_backward(hidden: torch.Tensor, gate_w: torch.Tensor, up_w: torch.Tensor, dout: torch.Tensor,
                       dhidden: Optional[torch.Tensor] = None, dgate_w: Optional[torch.Tensor] = None,
                       dup_w: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None):
    """Gradients (dhidden, dgate_w, dup_w) of dual_gemv for the upstream gradient ``dout``.

    hidden [M, K] (or [K], then dout is [N] and dhidden [K]), gate_w and up_w
    [N, K], dout [M, N]; all bf16, contiguous, on one GPU; M <= 65536.  Outputs are
    allocated unless given (contiguous, overwritten).  ``workspace``: a uint8
    device tensor of at least backward_workspace_bytes(M, N, K) bytes, else one
    is allocated; on return it begins with dg and du, the bf16 gradients of the
    gate and up pre-activations ([2, M, N]).
    """
    M, N, K, dev, dhidden, dgate_w, dup_w = _backward_args(hidden, gate_w, up_w, dout, dhidden, dgate_w, dup_w)
    need = backward_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    lib = library()
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = lib.glu_dual_gemv_backward(hidden.data_ptr(), gate_w.data_ptr(), up_w.data_ptr(), dout.data_ptr(),
                                        dhidden.data_ptr(), dgate_w.data_ptr(), dup_w.data_ptr(), M, N, K,
                                        workspace.data_ptr(), workspace.numel(), s.cuda_stream)
    _raise_for(st)
    return dhidden, dgate_w, dup_w


def dual_gemv_backward_noalloc(hidden: torch.Tensor, gate_w: torch.Tensor, up_w: torch.Tensor,
                               dout: torch.Tensor, dhidden: Optional[torch.Tensor] = None,
                               dgate_w: Optional[torch.Tensor] = None, dup_w: Optional[torch.Tensor] = None,
                               stream: Optional[torch.cuda.Stream] = None):
    """dual_gemv_backward through glu_dual_gemv_backward_noalloc: the library works in its own fixed
    device array (NOALLOC_SCRATCH_BYTES per GPU) instead of a workspace, so with all three outputs
    given nothing is allocated at all.  Calls that overlap on one GPU race on that array."""
    M, N, K, dev, dhidden, dgate_w, dup_w = _backward_args(hidden, gate_w, up_w, dout, dhidden, dgate_w, dup_w)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = library().glu_dual_gemv_backward_noalloc(hidden.data_ptr(), gate_w.data_ptr(), up_w.data_ptr(),
                                                      dout.data_ptr(), dhidden.data_ptr(), dgate_w.data_ptr(),
                                                      dup_w.data_ptr(), M, N, K, s.cuda_stream)
    _raise_for(st)
    return dhidden, dgate_w, dup_w


def dual_gemv_backward_raw(hidden_ptr: int, gate_ptr: int, up_ptr: int, dout_ptr: int, dh_ptr: int, dwg_ptr: int,
                           dwu_ptr: int, M: int, N: int, K: int, ws_ptr: int, ws_bytes: int,
                           stream_handle: int = 0) -> int:
    """The C call on raw device addresses; returns the glu_status (used by boundary tests)."""
    return library().glu_dual_gemv_backward(hidden_ptr, gate_ptr, up_ptr, dout_ptr, dh_ptr, dwg_ptr, dwu_ptr,
                                            M, N, K, ws_ptr, ws_bytes, stream_handle)


def dual_gemv_raw(hidden_ptr: int, gate_ptr: int, up_ptr: int, out_ptr: int, M: int, N: int, K: int,
                  stream_handle: int = 0, tuning: Optional[Tuning] = None) -> int:
    """The C call on raw device addresses; returns the glu_status (used by boundary tests)."""
    lib = library()
    if tuning is None:
        return lib.glu_dual_gemv(hidden_ptr, gate_ptr, up_ptr, out_ptr, M, N, K, stream_handle)
    return lib.glu_dual_gemv_tuned(hidden_ptr, gate_ptr, up_ptr, out_ptr, M, N, K, stream_handle,
                                   ctypes.byref(tuning))


def dual_gemv_strided_raw(hidden_ptr: int, ldh: int, gate_ptr: int, ldg: int, up_ptr: int, ldu: int, out_ptr: int,
                          ldo: int, M: int, N: int, K: int, stream_handle: int = 0,
                          tuning: Optional[Tuning] = None) -> int:
    """The strided C call on raw device addresses; returns the glu_status (used by boundary tests)."""
    lib = library()
    if tuning is None:
        return lib.glu_dual_gemv_strided(hidden_ptr, ldh, gate_ptr, ldg, up_ptr, ldu, out_ptr, ldo, M, N, K,
                                         stream_handle)
    return lib.glu_dual_gemv_strided_tuned(hidden_ptr, ldh, gate_ptr, ldg, up_ptr, ldu, out_ptr, ldo, M, N, K,
                                           stream_handle, ctypes.byref(tuning))


def grouped_plan(M: int, K: int, rows: int, fast: bool = True, tuning: Optional[Tuning] = None,
                 mult4: bool = True, mult8: bool = False) -> dict:
    """The launch glu_grouped_gemv would make (host only): rows = sum of N over the projections,
    ``fast`` whether the layout is a fast one, ``mult4`` / ``mult8`` whether every N is a multiple
    of 4 / of 8."""
    p = Plan()
    lib = library()
    flags = int(fast) | (2 if mult4 else 0) | (4 if mult8 and mult4 else 0)
    if tuning is None:
        st = lib.glu_grouped_gemv_plan(M, K, rows, flags, ctypes.byref(p))
    else:
        st = lib.glu_grouped_gemv_plan_tuned(M, K, rows, flags, ctypes.byref(tuning), ctypes.byref(p))
    _raise_for(st)
    d = p.as_dict()
    buf = ctypes.create_string_buffer(256)
    st = lib.glu_grouped_gemv_describe(M, K, rows, flags, ctypes.byref(tuning) if tuning is not None else None,
                                       buf, 256)
    _raise_for(st)
    d["kernel_symbol"] = buf.value.decode()
    return d


def grouped_gemv(hidden: torch.Tensor, weights, outs=None, tuning: Optional[Tuning] = None,
                 stream: Optional[torch.cuda.Stream] = None):
    """[bf16(hidden @ W.T) for W in weights], each W [N_i, K] read in place (no concatenation).

    hidden [M, K] (or [K]: each result is then [N_i]); 1 to 8 weights, all bf16
    on one GPU; row-strided views are read at the stride they report (rows must
    be contiguous).  ``outs`` (same count, [M, N_i] each) are written in place
    if given.  Runs asynchronously on ``stream`` (default: torch's current one).
    """
    weights = list(weights)
    if not 1 <= len(weights) <= GROUP_MAX:
        raise ValueError(f"1 to {GROUP_MAX} weights, got {len(weights)}")
    _check("hidden", hidden, (1, 2))
    vec = hidden.dim() == 1
    M = 1 if vec else hidden.shape[0]
    K = hidden.shape[-1]
    dev = hidden.device
    for i, w in enumerate(weights):
        _check(f"weights[{i}]", w, (2,))
        if w.shape[1] != K or w.device != dev:
            raise ValueError(f"weights[{i}] must be [N, {K}] on {dev}, got {tuple(w.shape)} on {w.device}")
    if outs is None:
        outs = [torch.empty((w.shape[0],) if vec else (M, w.shape[0]), dtype=torch.bfloat16, device=dev)
                for w in weights]
    else:
        outs = list(outs)
        if len(outs) != len(weights):
            raise ValueError("one output per weight")
        for i, (o, w) in enumerate(zip(outs, weights)):
            want = (w.shape[0],) if vec else (M, w.shape[0])
            _check(f"outs[{i}]", o, (len(want),))
            if tuple(o.shape) != want or o.device != dev:
                raise ValueError(f"outs[{i}] must be {want} on {dev}, got {tuple(o.shape)} on {o.device}")
    projs = (Projection * len(weights))()
    for i, (w, o) in enumerate(zip(weights, outs)):
        projs[i] = Projection(w.data_ptr(), o.data_ptr(), w.shape[0], _row_stride(f"weights[{i}]", w),
                              _row_stride(f"outs[{i}]", o))
    ldh = _row_stride("hidden", hidden)
    lib = library()
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        if tuning is None:
            st = lib.glu_grouped_gemv(hidden.data_ptr(), ldh, projs, len(weights), M, K, s.cuda_stream)
        else:
            st = lib.glu_grouped_gemv_tuned(hidden.data_ptr(), ldh, projs, len(weights), M, K, s.cuda_stream,
                                            ctypes.byref(tuning))
    _raise_for(st)
    return outs


def grouped_gemv_raw(hidden_ptr: int, ldh: int, projections, M: int, K: int, stream_handle: int = 0,
                     n: Optional[int] = None) -> int:
    """The grouped C call on raw addresses: projections is a list of (weight, out, N, ldw, ldo) tuples
    (or None for a NULL array); returns the glu_status (used by boundary tests)."""
    lib = library()
    if projections is None:
        return lib.glu_grouped_gemv(hidden_ptr, ldh, None, n or 0, M, K, stream_handle)
    arr = (Projection * max(1, len(projections)))()
    for i, p in enumerate(projections):
        arr[i] = Projection(*p)
    return lib.glu_grouped_gemv(hidden_ptr, ldh, arr, len(projections) if n is None else n, M, K, stream_handle)


UNIT_MFMA_16X16X32_BF16 = 1
UNIT_MFMA_32X32X16_BF16 = 2
UNIT_LDS_READ_B128 = 3


def unit_ceiling_work(unit: int, waves_per_cu: int, workgroups: int, iterations: int) -> float:
    """Flops (MFMA units) or LDS bytes (LDS unit) of one glu_unit_ceiling launch (host only)."""
    w = ctypes.c_double()
    _raise_for(library().glu_unit_ceiling_work(unit, waves_per_cu, workgroups, iterations, ctypes.byref(w)))
    return w.value


def unit_ceiling(unit: int, waves_per_cu: int, workgroups: int, iterations: int, sink: torch.Tensor) -> None:
    """One launch of a unit-throughput yardstick (MFMA shape or LDS reads) on the current stream of sink's
    device.  sink: >= 64 int32 of device memory."""
    if not sink.is_contiguous() or sink.numel() * sink.element_size() < 256 or sink.device.type != "cuda":
        raise ValueError("sink must hold 64 contiguous 32-bit words of device memory")
    st = library().glu_unit_ceiling(unit, waves_per_cu, workgroups, iterations, sink.data_ptr(),
                                    torch.cuda.current_stream(sink.device).cuda_stream)
    _raise_for(st)


def copy_ceiling(a: torch.Tensor, b: torch.Tensor, ca: torch.Tensor, cb: torch.Tensor,
                 tuning: Optional[Tuning] = None) -> None:
    """Read/write yardstick: ca[:] = a, cb[:] = b with the M = 1 GEMV's streaming pattern and nontemporal
    stores (four equal 2-D contiguous device tensors, rows of a multiple of 1 KiB)."""
    ts = (a, b, ca, cb)
    if a.dim() != 2 or any(t.shape != a.shape or t.dtype != a.dtype for t in ts):
        raise ValueError("a, b, ca and cb must be 2-D tensors of one shape and dtype")
    if not all(t.is_contiguous() and t.device == a.device for t in ts) or a.device.type != "cuda":
        raise ValueError("a, b, ca and cb must be contiguous and on one GPU")
    st = library().glu_copy_ceiling(a.data_ptr(), b.data_ptr(), ca.data_ptr(), cb.data_ptr(), a.shape[0],
                                    a.shape[1] * a.element_size(), ctypes.byref(tuning) if tuning is not None else None,
                                    torch.cuda.current_stream(a.device).cuda_stream)
    _raise_for(st)


def read_ceiling_plan(rows: int, row_bytes: int, tuning: Optional[Tuning] = None) -> dict:
    """Launch shape of the streaming-read yardstick (host only)."""
    p = Plan()
    st = library().glu_read_ceiling_plan(rows, row_bytes, ctypes.byref(tuning) if tuning is not None else None,
                                         ctypes.byref(p))
    _raise_for(st)
    d = p.as_dict()
    d["kernel_symbol"] = "glu::(anonymous namespace)::read_ceiling_kernel"
    return d


def read_ceiling(a: torch.Tensor, b: torch.Tensor, sink: torch.Tensor, tuning: Optional[Tuning] = None) -> None:
    """Streaming-read yardstick over two equal 2-D device tensors (rows of a multiple of 1 KiB): reads them
    as the M = 1 GEMV reads its weights.  sink: >= 64 int32 on the same device."""
    if a.dim() != 2 or a.shape != b.shape or a.dtype != b.dtype:
        raise ValueError("a and b must be 2-D tensors of one shape and dtype")
    if not (a.is_contiguous() and b.is_contiguous() and sink.is_contiguous()):
        raise ValueError("a, b and sink must be contiguous")
    if sink.numel() * sink.element_size() < 256 or not (a.device == b.device == sink.device) or a.device.type != "cuda":
        raise ValueError("sink must hold 64 32-bit words on the device of a and b")
    st = library().glu_read_ceiling(a.data_ptr(), b.data_ptr(), a.shape[0], a.shape[1] * a.element_size(),
                                    sink.data_ptr(), ctypes.byref(tuning) if tuning is not None else None,
                                    torch.cuda.current_stream(a.device).cuda_stream)
    _raise_for(st)
