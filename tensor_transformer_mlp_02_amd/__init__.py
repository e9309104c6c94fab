"""Python binding of libtpmlp.so, the tensor-parallel MLP shard library.

Argument marshalling only: each function has the name of the C entry point
it calls (declared in include/tpmlp.h), takes device tensors (or raw
integer device addresses) and passes their pointers and the current HIP
stream.  No arithmetic of the method happens here: every step runs in the
library's HIP kernels.  A nonzero status raises ``TpError``.  When the
library has not been built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "TP_F32", "TP_BF16", "TP_ACT_GELU_TANH", "TP_ACT_SWIGLU", "TpError",
    "tp_mlp_desc", "tp_expert_desc", "lib", "library_path",
    "tp_mlp_shard_fwd", "tp_mlp_shard_bwd", "tp_mlp_shard_bwd_accum", "tp_mlp_shard_bwd_workspace",
    "tp_mlp_shard_bwd_noalloc", "tp_mlp_shard_bwd_dact_prologue",
    "tp_partial_sum", "tp_partial_sum_capped", "tp_partial_sum_scatter", "tp_grouped_expert_fwd", "tp_grouped_expert_bwd",
    "tp_grouped_expert_bwd_workspace", "tp_grouped_expert_bwd_accum",
    "tp_grouped_expert_fwd_devoff", "tp_grouped_expert_bwd_devoff",
    "tp_grouped_expert_devoff_workspace",
    "tp_moe_permute", "tp_moe_combine", "tp_moe_combine_bwd",
    "tp_fp8_quantize", "tp_mlp_shard_fwd_fp8", "tp_fp8_transpose", "tp_fp8_scale_update", "tp_mlp_shard_bwd_fp8", "TP_FP8_E4M3", "TP_FP8_E5M2", "tp_last_error", "tp_status_string",
    "tp_launch_events", "tp_launch_events_used",
]

TP_F32, TP_BF16 = 0, 1
TP_FP8_E4M3, TP_FP8_E5M2 = 0, 1
TP_ACT_GELU_TANH, TP_ACT_SWIGLU = 0, 1
STATUS_NAMES = {0: "TP_OK", 1: "TP_ERR_NULL", 2: "TP_ERR_SHAPE", 3: "TP_ERR_DTYPE",
                4: "TP_ERR_ALIGN", 5: "TP_ERR_WORKSPACE", 6: "TP_ERR_DEVICE",
                7: "TP_ERR_HIP", 8: "TP_ERR_ALIAS"}

_HERE = os.path.dirname(os.path.abspath(__file__))
# TPMLP_LIBRARY selects another build of the library (a build-option variant)
library_path = os.environ.get("TPMLP_LIBRARY") or os.path.join(_HERE, "libtpmlp.so")


class TpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class tp_mlp_desc(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int64), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("F_shard", ctypes.c_int64), ("T", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class tp_expert_desc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int64), ("F", ctypes.c_int64), ("E", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_vp = ctypes.c_void_p
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it with __graft_entry__.build() "
            "(python tensor_transformer_mlp_02_amd/build.py)")
    L = ctypes.CDLL(library_path)
    D = ctypes.POINTER(tp_mlp_desc)
    ED = ctypes.POINTER(tp_expert_desc)
    I64P = ctypes.POINTER(ctypes.c_int64)
    L.tp_mlp_shard_fwd.argtypes = [D] + [_vp] * 8
    L.tp_mlp_shard_fwd.restype = ctypes.c_int
    L.tp_mlp_shard_bwd_workspace.argtypes = [D]
    L.tp_mlp_shard_bwd_workspace.restype = ctypes.c_size_t
    L.tp_mlp_shard_bwd.argtypes = [D] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    L.tp_mlp_shard_bwd.restype = ctypes.c_int
    L.tp_mlp_shard_bwd_noalloc.argtypes = [D] + [_vp] * 12
    L.tp_mlp_shard_bwd_noalloc.restype = ctypes.c_int
    L.tp_mlp_shard_bwd_accum.argtypes = [D] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    L.tp_mlp_shard_bwd_accum.restype = ctypes.c_int
    L.tp_mlp_shard_bwd_dact_prologue.argtypes = [D] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    L.tp_mlp_shard_bwd_dact_prologue.restype = ctypes.c_int
    L.tp_partial_sum.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_vp),
                                 ctypes.c_int64, _vp, _vp]
    L.tp_partial_sum.restype = ctypes.c_int
    L.tp_partial_sum_capped.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_vp),
                                        ctypes.c_int64, _vp, ctypes.c_int32, _vp]
    L.tp_partial_sum_capped.restype = ctypes.c_int
    L.tp_partial_sum_scatter.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_vp),
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int32, _vp, _vp]
    L.tp_partial_sum_scatter.restype = ctypes.c_int
    L.tp_grouped_expert_fwd.argtypes = [ED, I64P] + [_vp] * 8
    L.tp_grouped_expert_fwd.restype = ctypes.c_int
    L.tp_grouped_expert_bwd_workspace.argtypes = [ED, I64P]
    L.tp_grouped_expert_bwd_workspace.restype = ctypes.c_size_t
    L.tp_grouped_expert_bwd.argtypes = [ED, I64P] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    L.tp_grouped_expert_bwd.restype = ctypes.c_int
    L.tp_grouped_expert_bwd_accum.argtypes = [ED, I64P] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    L.tp_grouped_expert_bwd_accum.restype = ctypes.c_int
    L.tp_grouped_expert_fwd_devoff.argtypes = [ED, ctypes.c_int64] + [_vp] * 9
    L.tp_grouped_expert_fwd_devoff.restype = ctypes.c_int
    L.tp_grouped_expert_devoff_workspace.argtypes = [ED, ctypes.c_int64]
    L.tp_grouped_expert_devoff_workspace.restype = ctypes.c_size_t
    L.tp_grouped_expert_bwd_devoff.argtypes = ([ED, ctypes.c_int64] + [_vp] * 13 +
                                               [ctypes.c_size_t, ctypes.c_int32, _vp])
    L.tp_grouped_expert_bwd_devoff.restype = ctypes.c_int
    L.tp_moe_permute.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 _vp, _vp, _vp, _vp]
    L.tp_moe_permute.restype = ctypes.c_int
    L.tp_moe_combine.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 _vp, _vp, _vp, _vp, _vp, _vp]
    L.tp_moe_combine.restype = ctypes.c_int
    L.tp_moe_combine_bwd.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.tp_moe_combine_bwd.restype = ctypes.c_int
    L.tp_fp8_quantize.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                  _vp, _vp, _vp, _vp, _vp]
    L.tp_fp8_quantize.restype = ctypes.c_int
    L.tp_mlp_shard_fwd_fp8.argtypes = [D] + [_vp] * 11
    L.tp_mlp_shard_fwd_fp8.restype = ctypes.c_int
    L.tp_fp8_transpose.argtypes = [ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]
    L.tp_fp8_transpose.restype = ctypes.c_int
    L.tp_fp8_scale_update.argtypes = ([ctypes.c_int32] * 3 + [_vp] * 4 +
                                      [ctypes.c_int32, _vp])
    L.tp_fp8_scale_update.restype = ctypes.c_int
    L.tp_mlp_shard_bwd_fp8.argtypes = [D] + [_vp] * 17
    L.tp_mlp_shard_bwd_fp8.restype = ctypes.c_int
    L.tp_launch_events.argtypes = [ctypes.POINTER(_vp), ctypes.c_int32]
    L.tp_launch_events.restype = ctypes.c_int
    L.tp_launch_events_used.argtypes = []
    L.tp_launch_events_used.restype = ctypes.c_int32
    L.tp_last_error.argtypes = []
    L.tp_last_error.restype = ctypes.c_char_p
    L.tp_status_string.argtypes = [ctypes.c_int]
    L.tp_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(t, nbytes: Optional[int] = None, name: str = "tensor",
         dtype: Optional[str] = None) -> Optional[int]:
    """Device address of a tensor, an int (a raw device address, passed as
    given), or None.  A tensor must be contiguous, live on the current GPU
    (a host tensor's address would reach a kernel as a device address) and,
    when nbytes is given, hold at least that many bytes; tables and scale
    buffers (dtype "int32" / "float32") must hold that element type, since
    the library reads their bytes as such."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if dtype is not None and str(getattr(t, "dtype", "")) != f"torch.{dtype}":
        raise ValueError(f"{name} must be a torch.{dtype} tensor, got {getattr(t, 'dtype', None)}")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
    import torch
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, "
                         f"{nbytes} needed")
    return t.data_ptr()


def _sized(items):
    """_ptr of each (tensor, bytes, name) or (tensor, bytes, name, dtype)."""
    return [_ptr(*it) for it in items]


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(rc: int) -> int:
    if rc != 0:
        raise TpError(rc, tp_last_error())
    return rc


def tp_last_error() -> str:
    return lib().tp_last_error().decode()


def tp_status_string(status: int) -> str:
    return lib().tp_status_string(int(status)).decode()


def tp_launch_events(events) -> int:
    """Time this thread's next calls: ``events`` is a sequence of raw
    hipEvent_t handles (ints), two per timed unit, or None / [] to stop."""
    evs = [int(e) for e in (events or [])]
    arr = (_vp * len(evs))(*evs) if evs else None
    return _check(lib().tp_launch_events(arr, len(evs)))


def tp_launch_events_used() -> int:
    return int(lib().tp_launch_events_used())


def _desc(desc) -> tp_mlp_desc:
    if isinstance(desc, tp_mlp_desc):
        return desc
    return tp_mlp_desc(**desc)


def _edesc(desc) -> tp_expert_desc:
    if isinstance(desc, tp_expert_desc):
        return desc
    return tp_expert_desc(**desc)


def _offsets(offsets: Sequence[int], E: int):
    """Host array of the E+1 row offsets (the library reads exactly E+1)."""
    vals = [int(v) for v in offsets]
    if len(vals) != E + 1:
        raise ValueError(f"offsets has {len(vals)} entries, E + 1 = {E + 1} needed")
    return (ctypes.c_int64 * len(vals))(*vals)


def _partials(partials, T: int, nbytes: Optional[int]):
    """Host array of the T partial pointers (the library reads exactly T)."""
    if partials is None:
        return None
    if len(partials) != T:
        raise ValueError(f"{len(partials)} partials given, T = {T}")
    return (_vp * T)(*[_ptr(p, nbytes, f"partials[{i}]") for i, p in enumerate(partials)])


def _elt(dtype: int) -> int:
    return 2 if dtype == TP_BF16 else 4


def _shard_sizes(d: tp_mlp_desc):
    """Bytes of each shard tensor the descriptor implies (0 for an invalid
    descriptor: the library's own checks then report it)."""
    N, H, Ft = max(d.S, 0) * max(d.B, 0), max(d.H, 0), max(d.F_shard, 0)
    e = _elt(d.dtype)
    zw = 2 * Ft if d.act == TP_ACT_SWIGLU else Ft
    return dict(X=N * H * e, A=H * Ft * e, B=Ft * H * e, Z=N * zw * e, H=N * Ft * e,
                Y=N * H * e, dA=H * Ft * 4, dB=Ft * H * 4)


def _expert_sizes(d: tp_expert_desc, R: int):
    E, H, F = max(d.E, 0), max(d.H, 0), max(d.F, 0)
    return dict(X=R * H * 2, W=E * H * F * 2, Z=R * 2 * F * 2, H=R * F * 2, Y=R * H * 2,
                dW=E * H * F * 4)


def tp_mlp_shard_fwd(desc, X, A, A_up, B, Z_save, H_act, Y_partial, stream=None) -> int:
    d = _desc(desc)
    n = _shard_sizes(d)
    p = _sized([(X, n["X"], "X"), (A, n["A"], "A"), (A_up, n["A"], "A_up"), (B, n["B"], "B"),
                (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"),
                (Y_partial, n["Y"], "Y_partial")])
    return _check(lib().tp_mlp_shard_fwd(ctypes.byref(d), *p, _stream(stream)))


def tp_mlp_shard_bwd_workspace(desc) -> int:
    d = _desc(desc)
    return int(lib().tp_mlp_shard_bwd_workspace(ctypes.byref(d)))


def tp_mlp_shard_bwd(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA, dA_up, dB,
                     workspace, ws_bytes: int, stream=None, accumulate: bool = False) -> int:
    """accumulate=True calls tp_mlp_shard_bwd_accum (dA, dA_up, dB += ...)."""
    d = _desc(desc)
    n = _shard_sizes(d)
    fn = lib().tp_mlp_shard_bwd_accum if accumulate else lib().tp_mlp_shard_bwd
    p = _sized([(X, n["X"], "X"), (A, n["A"], "A"), (A_up, n["A"], "A_up"), (B, n["B"], "B"),
                (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"), (dY, n["Y"], "dY"),
                (dX_partial, n["X"], "dX_partial"), (dA, n["dA"], "dA"),
                (dA_up, n["dA"], "dA_up"), (dB, n["dB"], "dB"),
                (workspace, int(ws_bytes), "workspace")])
    return _check(fn(ctypes.byref(d), *p, int(ws_bytes), _stream(stream)))


def tp_mlp_shard_bwd_dact_prologue(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA,
                                   dA_up, dB, workspace, ws_bytes: int, stream=None) -> int:
    """The backward with the activation derivative formed by the dA and dX
    GEMMs as they load dZ; the workspace (N * F_shard elements) ends up
    holding dH."""
    d = _desc(desc)
    n = _shard_sizes(d)
    p = _sized([(X, n["X"], "X"), (A, n["A"], "A"), (A_up, n["A"], "A_up"), (B, n["B"], "B"),
                (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"), (dY, n["Y"], "dY"),
                (dX_partial, n["X"], "dX_partial"), (dA, n["dA"], "dA"),
                (dA_up, n["dA"], "dA_up"), (dB, n["dB"], "dB"),
                (workspace, int(ws_bytes), "workspace")])
    return _check(lib().tp_mlp_shard_bwd_dact_prologue(ctypes.byref(d), *p, int(ws_bytes),
                                                       _stream(stream)))


def tp_mlp_shard_bwd_noalloc(desc, X, A, A_up, B, Z_save, H_act, dY, dX_partial, dA, dA_up,
                             dB, stream=None) -> int:
    """tp_mlp_shard_bwd without a workspace: dZ goes to the library's own
    per-GPU scratch array (calls on one GPU must not overlap)."""
    d = _desc(desc)
    n = _shard_sizes(d)
    p = _sized([(X, n["X"], "X"), (A, n["A"], "A"), (A_up, n["A"], "A_up"), (B, n["B"], "B"),
                (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"), (dY, n["Y"], "dY"),
                (dX_partial, n["X"], "dX_partial"), (dA, n["dA"], "dA"),
                (dA_up, n["dA"], "dA_up"), (dB, n["dB"], "dB")])
    return _check(lib().tp_mlp_shard_bwd_noalloc(ctypes.byref(d), *p, _stream(stream)))


def tp_partial_sum(dtype: int, T: int, partials, count: int, out, stream=None) -> int:
    nb = max(int(count), 0) * _elt(dtype)
    arr = _partials(partials, int(T), nb)
    return _check(lib().tp_partial_sum(int(dtype), int(T), arr, int(count),
                                       _ptr(out, nb, "out"), _stream(stream)))


def tp_partial_sum_capped(dtype: int, T: int, partials, count: int, out, max_workgroups: int,
                          stream=None) -> int:
    nb = max(int(count), 0) * _elt(dtype)
    arr = _partials(partials, int(T), nb)
    return _check(lib().tp_partial_sum_capped(int(dtype), int(T), arr, int(count),
                                              _ptr(out, nb, "out"), int(max_workgroups),
                                              _stream(stream)))


def tp_partial_sum_scatter(dtype: int, T: int, partials, S: int, B: int, H: int, rank: int,
                           out, stream=None) -> int:
    full = max(int(S), 0) * max(int(B), 0) * max(int(H), 0) * _elt(dtype)
    arr = _partials(partials, int(T), full)
    sl = full // int(T) if int(T) > 0 and int(S) % int(T) == 0 else None
    return _check(lib().tp_partial_sum_scatter(int(dtype), int(T), arr, int(S), int(B), int(H),
                                               int(rank), _ptr(out, sl, "out"), _stream(stream)))


def tp_grouped_expert_fwd(desc, offsets, X_perm, Wg, Wu, Wd, Z_save, H_act, Y_perm,
                          stream=None) -> int:
    d = _edesc(desc)
    off = _offsets(offsets, d.E)
    n = _expert_sizes(d, int(off[d.E]))
    p = _sized([(X_perm, n["X"], "X_perm"), (Wg, n["W"], "Wg"), (Wu, n["W"], "Wu"),
                (Wd, n["W"], "Wd"), (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"),
                (Y_perm, n["Y"], "Y_perm")])
    return _check(lib().tp_grouped_expert_fwd(ctypes.byref(d), off, *p, _stream(stream)))


def tp_grouped_expert_bwd_workspace(desc, offsets) -> int:
    d = _edesc(desc)
    return int(lib().tp_grouped_expert_bwd_workspace(ctypes.byref(d), _offsets(offsets, d.E)))


def tp_grouped_expert_bwd(desc, offsets, X_perm, Wg, Wu, Wd, Z_save, H_act, dY_perm,
                          dX_perm, dWg, dWu, dWd, workspace, ws_bytes: int,
                          stream=None, accumulate: bool = False) -> int:
    """accumulate=True calls tp_grouped_expert_bwd_accum (dW* += ...)."""
    d = _edesc(desc)
    off = _offsets(offsets, d.E)
    n = _expert_sizes(d, int(off[d.E]))
    fn = lib().tp_grouped_expert_bwd_accum if accumulate else lib().tp_grouped_expert_bwd
    p = _sized([(X_perm, n["X"], "X_perm"), (Wg, n["W"], "Wg"), (Wu, n["W"], "Wu"),
                (Wd, n["W"], "Wd"), (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"),
                (dY_perm, n["Y"], "dY_perm"), (dX_perm, n["X"], "dX_perm"),
                (dWg, n["dW"], "dWg"), (dWu, n["dW"], "dWu"), (dWd, n["dW"], "dWd"),
                (workspace, int(ws_bytes), "workspace")])
    return _check(fn(ctypes.byref(d), off, *p, int(ws_bytes), _stream(stream)))


def tp_grouped_expert_fwd_devoff(desc, R: int, offsets, X_perm, Wg, Wu, Wd, Z_save, H_act,
                                 Y_perm, stream=None) -> int:
    """tp_grouped_expert_fwd with the E+1 row offsets an int32 GPU tensor
    (read by the kernels, clamped into [0, R]); R is the rows the buffers
    hold."""
    d = _edesc(desc)
    n = _expert_sizes(d, max(int(R), 0))
    p = _sized([(offsets, 4 * (max(d.E, 0) + 1), "offsets", "int32"), (X_perm, n["X"], "X_perm"),
                (Wg, n["W"], "Wg"), (Wu, n["W"], "Wu"), (Wd, n["W"], "Wd"),
                (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"), (Y_perm, n["Y"], "Y_perm")])
    return _check(lib().tp_grouped_expert_fwd_devoff(ctypes.byref(d), int(R), *p,
                                                      _stream(stream)))


def tp_grouped_expert_devoff_workspace(desc, R: int) -> int:
    d = _edesc(desc)
    return int(lib().tp_grouped_expert_devoff_workspace(ctypes.byref(d), int(R)))


def tp_grouped_expert_bwd_devoff(desc, R: int, offsets, X_perm, Wg, Wu, Wd, Z_save, H_act,
                                 dY_perm, dX_perm, dWg, dWu, dWd, workspace, ws_bytes: int,
                                 accumulate: bool = False, stream=None) -> int:
    """tp_grouped_expert_bwd (accumulate=True: _bwd_accum) with device-resident
    int32 offsets, as tp_grouped_expert_fwd_devoff."""
    d = _edesc(desc)
    n = _expert_sizes(d, max(int(R), 0))
    p = _sized([(offsets, 4 * (max(d.E, 0) + 1), "offsets", "int32"), (X_perm, n["X"], "X_perm"),
                (Wg, n["W"], "Wg"), (Wu, n["W"], "Wu"), (Wd, n["W"], "Wd"),
                (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"),
                (dY_perm, n["Y"], "dY_perm"), (dX_perm, n["X"], "dX_perm"),
                (dWg, n["dW"], "dWg"), (dWu, n["dW"], "dWu"), (dWd, n["dW"], "dWd"),
                (workspace, int(ws_bytes), "workspace")])
    return _check(lib().tp_grouped_expert_bwd_devoff(ctypes.byref(d), int(R), *p, int(ws_bytes),
                                                      1 if accumulate else 0, _stream(stream)))


def tp_mlp_shard_bwd_accum(*args, **kw) -> int:
    return tp_mlp_shard_bwd(*args, accumulate=True, **kw)


def tp_grouped_expert_bwd_accum(*args, **kw) -> int:
    return tp_grouped_expert_bwd(*args, accumulate=True, **kw)


def tp_moe_permute(dtype: int, N: int, H: int, R: int, row_token, X, X_perm, stream=None) -> int:
    e, n, h, r = _elt(dtype), max(int(N), 0), max(int(H), 0), max(int(R), 0)
    p = _sized([(row_token, r * 4, "row_token", "int32"), (X, n * h * e, "X"),
                (X_perm, r * h * e, "X_perm")])
    return _check(lib().tp_moe_permute(int(dtype), int(N), int(H), int(R), *p, _stream(stream)))


def tp_moe_combine(dtype: int, N: int, H: int, R: int, tok_ptr, tok_rows, row_weight, Y_perm, Y,
                   stream=None) -> int:
    e, n, h, r = _elt(dtype), max(int(N), 0), max(int(H), 0), max(int(R), 0)
    p = _sized([(tok_ptr, (n + 1) * 4, "tok_ptr", "int32"), (tok_rows, r * 4, "tok_rows", "int32"),
                (row_weight, r * 4, "row_weight", "float32"), (Y_perm, r * h * e, "Y_perm"),
                (Y, n * h * e, "Y")])
    return _check(lib().tp_moe_combine(int(dtype), int(N), int(H), int(R), *p, _stream(stream)))


def tp_moe_combine_bwd(dtype: int, N: int, H: int, R: int, row_token, row_weight, dY, Y_perm,
                       dY_perm, d_weight, stream=None) -> int:
    e, n, h, r = _elt(dtype), max(int(N), 0), max(int(H), 0), max(int(R), 0)
    p = _sized([(row_token, r * 4, "row_token", "int32"), (row_weight, r * 4, "row_weight", "float32"),
                (dY, n * h * e, "dY"), (Y_perm, r * h * e, "Y_perm"),
                (dY_perm, r * h * e, "dY_perm"), (d_weight, r * 4, "d_weight", "float32")])
    return _check(lib().tp_moe_combine_bwd(int(dtype), int(N), int(H), int(R), *p,
                                           _stream(stream)))


def tp_fp8_quantize(fmt: int, transpose: bool, rows: int, cols: int, x, scale, q, amax=None,
                    stream=None) -> int:
    n = max(int(rows), 0) * max(int(cols), 0)
    p = _sized([(x, n * 2, "x"), (scale, 4, "scale", "float32"), (q, n, "q"), (amax, 4, "amax", "float32")])
    return _check(lib().tp_fp8_quantize(int(fmt), int(bool(transpose)), int(rows), int(cols),
                                        *p, _stream(stream)))


def tp_mlp_shard_fwd_fp8(desc, Xq, Aq_t, Auq_t, Bq_t, scales, Z_save, H_act, H_q, h_amax,
                         Y_partial, stream=None) -> int:
    d = _desc(desc)
    n = _shard_sizes(d)
    p = _sized([(Xq, n["X"] // 2, "Xq"), (Aq_t, n["A"] // 2, "Aq_t"),
                (Auq_t, n["A"] // 2, "Auq_t"), (Bq_t, n["B"] // 2, "Bq_t"),
                (scales, 5 * 4, "scales", "float32"), (Z_save, n["Z"], "Z_save"), (H_act, n["H"], "H_act"),
                (H_q, n["H"] // 2, "H_q"), (h_amax, 4, "h_amax", "float32"),
                (Y_partial, n["Y"], "Y_partial")])
    return _check(lib().tp_mlp_shard_fwd_fp8(ctypes.byref(d), *p, _stream(stream)))


def tp_fp8_transpose(rows: int, cols: int, q, q_t, stream=None) -> int:
    n = max(int(rows), 0) * max(int(cols), 0)
    return _check(lib().tp_fp8_transpose(int(rows), int(cols), _ptr(q, n, "q"),
                                         _ptr(q_t, n, "q_t"), _stream(stream)))


def tp_fp8_scale_update(fmt: int, n: int, length: int, history, amax, scale, scale_inv=None,
                        margin: int = 0, stream=None) -> int:
    nb = max(int(n), 0) * 4
    return _check(lib().tp_fp8_scale_update(int(fmt), int(n), int(length),
                                            _ptr(history, nb * max(int(length), 0), "history",
                                                 "float32"),
                                            _ptr(amax, nb, "amax", "float32"),
                                            _ptr(scale, nb, "scale", "float32"),
                                            _ptr(scale_inv, nb, "scale_inv", "float32"),
                                            int(margin),
                                            _stream(stream)))


def tp_mlp_shard_bwd_fp8(desc, dYq, dYq_t, Xq_t, Hq_t, Aq, Auq, Bq, Z_save, scales, dX_partial,
                         dA, dA_up, dB, dZq, dZq_t, dz_amax, stream=None) -> int:
    d = _desc(desc)
    n = _shard_sizes(d)
    zq = n["Z"] // 2
    p = _sized([(dYq, n["Y"] // 2, "dYq"), (dYq_t, n["Y"] // 2, "dYq_t"),
                (Xq_t, n["X"] // 2, "Xq_t"), (Hq_t, n["H"] // 2, "Hq_t"),
                (Aq, n["A"] // 2, "Aq"), (Auq, n["A"] // 2, "Auq"), (Bq, n["B"] // 2, "Bq"),
                (Z_save, n["Z"], "Z_save"), (scales, 7 * 4, "scales", "float32"),
                (dX_partial, n["X"], "dX_partial"), (dA, n["dA"], "dA"),
                (dA_up, n["dA"], "dA_up"), (dB, n["dB"], "dB"), (dZq, zq, "dZq"),
                (dZq_t, zq, "dZq_t"), (dz_amax, 4, "dz_amax", "float32")])
    return _check(lib().tp_mlp_shard_bwd_fp8(ctypes.byref(d), *p, _stream(stream)))
