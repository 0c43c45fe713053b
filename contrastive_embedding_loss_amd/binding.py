"""ctypes binding of ``libuform_contrastive.so`` (argument marshalling only).

Every step of the loss runs in the library's HIP kernels; this module only
allocates outputs with torch on the inputs' device and passes raw pointers
plus torch's current HIP stream.  It raises if the library is missing: there
is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch  # imported before the library so both share one HIP runtime

INFONCE = 0
SIGLIP = 1
INFONCE_ROWS = 2
ONESET_SIGLIP = 3  # one set scored against itself: q = k[row_offset:row_offset + R], no dk
ONESET_SIGLIP_EDGES = 4  # the same, every positive listed as a relation (``positives``), no implicit pairs
ACCUMULATE = 1
PROFILE = 2
ONE_SPLIT = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuform_contrastive.so")

STATUS_NAMES = {0: "success", 1: "invalid-argument", 2: "unsupported", 3: "out-of-memory", 4: "device-error"}


class UformError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, 'unknown')}: {message}")
        self.status = status
        self.message = message


class Options(ctypes.Structure):
    _fields_ = [
        ("prefix_weights", ctypes.POINTER(ctypes.c_float)),
        ("row_offset", ctypes.c_int64),
        ("prefix_losses_out", ctypes.c_void_p),
        ("col_lse_out", ctypes.c_void_p),
        ("row_lse_out", ctypes.c_void_p),
        ("pos_logit_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("flags", ctypes.c_uint32),
        ("dscale_out", ctypes.c_void_p),
        ("dbias_out", ctypes.c_void_p),
        ("pos_row_ptr", ctypes.POINTER(ctypes.c_int64)),
        ("pos_col", ctypes.POINTER(ctypes.c_int32)),
    ]


_lib = None


def library() -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    args = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.uform_contrastive_fwd_bwd.argtypes = args
    lib.uform_contrastive_fwd_bwd.restype = ctypes.c_int
    lib.uform_contrastive_fwd_bwd_ex.argtypes = args + [ctypes.POINTER(Options)]
    lib.uform_contrastive_fwd_bwd_ex.restype = ctypes.c_int
    lib.uform_contrastive_fwd_bwd_noalloc.argtypes = args + [ctypes.POINTER(Options)]
    lib.uform_contrastive_fwd_bwd_noalloc.restype = ctypes.c_int
    lib.uform_contrastive_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                      ctypes.c_int32, ctypes.c_int32]
    lib.uform_contrastive_workspace_bytes.restype = ctypes.c_size_t
    lib.uform_contrastive_workspace_bytes_ex.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    lib.uform_contrastive_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.uform_contrastive_supported.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32]
    lib.uform_contrastive_supported.restype = ctypes.c_int
    lib.uform_status_name.argtypes = [ctypes.c_int]
    lib.uform_status_name.restype = ctypes.c_char_p
    lib.uform_contrastive_last_error.argtypes = []
    lib.uform_contrastive_last_error.restype = ctypes.c_char_p
    lib.uform_contrastive_profile.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                              ctypes.c_int32]
    lib.uform_contrastive_profile.restype = ctypes.c_int32
    lib.uform_contrastive_release.argtypes = []
    lib.uform_contrastive_release.restype = None
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return library().uform_status_name(status).decode()


def last_error() -> str:
    return library().uform_contrastive_last_error().decode()


def supported(D: int, prefixes, kind: int, with_gradients: bool = True) -> int:
    """Status a call with this width, ladder and kind would get from its checks (0 = runs)."""
    pw = (ctypes.c_int32 * len(prefixes))(*[int(p) for p in prefixes])
    return int(library().uform_contrastive_supported(D, pw, len(prefixes), kind, int(with_gradients)))


def workspace_bytes(R: int, N: int, D: int, n_prefixes: int, kind: int, n_positives: int | None = None) -> int:
    if n_positives is None:
        return int(library().uform_contrastive_workspace_bytes(R, N, D, n_prefixes, kind))
    return int(library().uform_contrastive_workspace_bytes_ex(R, N, D, n_prefixes, kind, int(n_positives)))


def profile() -> dict:
    """Summed milliseconds per kernel over the profiled calls since the last read."""
    cap = 64
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = min(library().uform_contrastive_profile(names, ms, cap), cap)
    return {names[i].decode(): float(ms[i]) for i in range(n)}


def release() -> None:
    library().uform_contrastive_release()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_grad_buffer(name, t, shape, dev) -> None:
    """A caller-given gradient buffer must be exactly what the kernels write: contiguous
    float32 of the given shape on q's device (anything else would be written past its end)."""
    if t is None:
        return
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on q's device")


def _check(status: int) -> None:
    if status != 0:
        raise UformError(status, last_error())


def fwd_bwd(q: torch.Tensor, k: torch.Tensor, prefixes, scale: float, bias: float, kind: int, weights=None,
            row_offset: int = 0, want_dq: bool = True, want_dk: bool = True, extras: bool = False,
            dq: torch.Tensor | None = None, dk: torch.Tensor | None = None, accumulate: bool = False,
            workspace: torch.Tensor | None = None, profile: bool = False, one_split: bool = False,
            positives=None, noalloc: bool = False):
    """Loss and gradients of the Matryoshka contrastive loss on q's device.

    q [R, D] and k [N, D] are contiguous bfloat16 device tensors.  Returns
    ``(loss, dq, dk)`` (float32 tensors; dq/dk None when not wanted), plus a
    dict of ``prefix_losses``, ``row_lse``, ``col_lse`` and ``pos_logit`` when
    ``extras`` (and ``dscale``, ``dbias``: dL/dscale and dL/dbias, when a
    gradient is wanted).  Everything is enqueued on torch's current stream.  ``one_split`` runs each backward pass as
    one inner split (a diagnostic: the in-place finish that large problems take).
    ``noalloc`` calls the allocation-free entry point (the library's fixed per-GPU
    scratch instead of a workspace; outputs are still allocated here unless given).
    ``positives`` = (row_ptr, col), host integer arrays in CSR form, lists extra
    positive cells of the sigmoid kinds (row i: columns col[row_ptr[i]:row_ptr[i + 1]]).
    """
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TypeError("q and k must be bfloat16")
    if not (q.is_cuda and k.is_cuda):
        raise TypeError("q and k must be device tensors")
    if q.dim() != 2 or k.dim() != 2 or q.shape[1] != k.shape[1]:
        raise ValueError("q and k must be [R, D] and [N, D]")
    if q.device != k.device:
        raise ValueError("q and k must be on one device")
    q = q.contiguous()
    k = k.contiguous()
    R, D = q.shape
    N = k.shape[0]
    dev = q.device
    _check_grad_buffer("dq", dq, (R, D), dev)
    _check_grad_buffer("dk", dk, (N, D), dev)
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    P = len(prefixes)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32)
    if want_dq and dq is None:
        dq = torch.zeros(R, D, **f32) if accumulate else torch.empty(R, D, **f32)
    if kind in (ONESET_SIGLIP, ONESET_SIGLIP_EDGES):
        want_dk = False  # the one-set forms' only gradient is dq
    if want_dk and dk is None:
        dk = torch.zeros(N, D, **f32) if accumulate else torch.empty(N, D, **f32)
    if not want_dq:
        dq = None
    if not want_dk:
        dk = None
    pw = (ctypes.c_int32 * P)(*[int(p) for p in prefixes])
    opt = Options()
    opt.row_offset = int(row_offset)
    wbuf = None
    if weights is not None:
        wbuf = (ctypes.c_float * P)(*[float(w) for w in weights])
        opt.prefix_weights = ctypes.cast(wbuf, ctypes.POINTER(ctypes.c_float))
    ex = None
    if extras:
        softmax = kind not in (SIGLIP, ONESET_SIGLIP, ONESET_SIGLIP_EDGES)
        ex = {"prefix_losses": torch.empty(P, **f32)}
        opt.prefix_losses_out = ex["prefix_losses"].data_ptr()
        if kind != ONESET_SIGLIP_EDGES:  # every other kind has one positive per row
            ex["pos_logit"] = torch.empty(P, R, **f32)
            opt.pos_logit_out = ex["pos_logit"].data_ptr()
        if softmax:
            ex["row_lse"] = torch.empty(P, R, **f32)
            ex["col_lse"] = torch.empty(P, N, **f32)
        if softmax:
            opt.row_lse_out = ex["row_lse"].data_ptr()
            opt.col_lse_out = ex["col_lse"].data_ptr()
        if dq is not None or dk is not None:
            ex["dscale"] = torch.empty(1, **f32)
            ex["dbias"] = torch.empty(1, **f32)
            opt.dscale_out = ex["dscale"].data_ptr()
            opt.dbias_out = ex["dbias"].data_ptr()
    pos_keep = None
    if positives is not None:
        import numpy as np
        rp = np.ascontiguousarray(np.asarray(positives[0]), dtype=np.int64)
        pc_in = np.asarray(positives[1])
        if pc_in.size and (pc_in.min() < -2**31 or pc_in.max() >= 2**31):
            raise ValueError("positives: column indices must fit int32")
        pc = np.ascontiguousarray(pc_in, dtype=np.int32)
        if rp.shape != (R + 1,):
            raise ValueError("positives: row_ptr must have R + 1 entries")
        if rp[-1] > pc.size:
            raise ValueError("positives: col is shorter than row_ptr[R]")
        pos_keep = (rp, pc)
        opt.pos_row_ptr = rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        opt.pos_col = pc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if workspace is not None:
        opt.workspace = workspace.data_ptr()
        opt.workspace_bytes = workspace.numel() * workspace.element_size()
    opt.flags = (ACCUMULATE if accumulate else 0) | (PROFILE if profile else 0) | (ONE_SPLIT if one_split else 0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    entry = library().uform_contrastive_fwd_bwd_noalloc if noalloc else library().uform_contrastive_fwd_bwd_ex
    status = entry(
        _ptr(q), _ptr(k), R, N, D, pw, P, float(scale), float(bias), int(kind), _ptr(loss), _ptr(dq), _ptr(dk),
        ctypes.c_void_p(stream), ctypes.byref(opt))
    _check(status)
    del wbuf, pos_keep
    if extras:
        return loss, dq, dk, ex
    return loss, dq, dk
