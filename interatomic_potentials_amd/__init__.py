"""interatomic_potentials_amd -- E2Former-V2 on-the-fly equivariant attention on MI355X.

A thin ctypes binding over ``libe2f.so`` (include/e2f.h).  Every step of the
path runs in the library's HIP kernels; this module only checks tensor
metadata, picks the stream, and passes device pointers.  PyTorch provides the
device memory and the current stream.

Importing the package loads the library and fails loudly if it has not been
built (``python interatomic_potentials_amd/build.py``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = [
    "E2FError", "lib", "status_string", "path_count", "eaas_couple", "dense_couple",
    "attn_workspace_bytes",
    "attn_precouple", "attn_aggregate", "attn_forward", "attn_backward",
    "attn_backward_workspace_bytes", "neighbour_workspace_bytes", "neighbour_list", "frames",
    "attn_forward_noalloc", "attn_noalloc_max_bytes",
    "F32", "BF16",
    "VALIDATE_INDICES", "TARGETS_IN_ORDER", "MSG_F32",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libe2f.so")

F32 = 0
BF16 = 1
VALIDATE_INDICES = 1
TARGETS_IN_ORDER = 2
MSG_F32 = 4
SHARED_ROWS = 8
MATRIX_TILES = 16

_STATUS = {
    0: "E2F_OK", -1: "E2F_ERR_NULL", -2: "E2F_ERR_SHAPE", -3: "E2F_ERR_DTYPE",
    -4: "E2F_ERR_ALIGN", -5: "E2F_ERR_WORKSPACE", -6: "E2F_ERR_ALIAS", -7: "E2F_ERR_HIP",
    -8: "E2F_ERR_INDEX", -9: "E2F_ERR_UNSUPPORTED", -10: "E2F_ERR_RUNTIME",
}
STATUS_CODES = {v: k for k, v in _STATUS.items()}

# exported symbols and their C signatures (mirrors include/e2f.h)
_vp, _i32, _i64, _u32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32,
                                    ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "e2f_status_string": (ctypes.c_char_p, [_i32]),
    "e2f_path_count": (_i32, [_i32]),
    "e2f_last_hip_error": (_i32, []),
    "e2f_last_hip_error_name": (ctypes.c_char_p, []),
    "e2f_eaas_couple": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "e2f_dense_couple": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "e2f_attn_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "e2f_attn_precouple": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz]),
    "e2f_attn_precouple_proj": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _sz]),
    "e2f_attn_forward_proj": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _f32, _f32, _vp, _vp, _sz, _vp, _vp, _vp,
                                     _u32]),
    "e2f_attn_aggregate": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _f32,
                                  _f32, _vp, _vp, _sz, _vp, _vp, _vp, _u32]),
    "e2f_attn_forward": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                _f32, _f32, _vp, _vp, _sz, _vp, _vp, _vp, _u32]),
    "e2f_attn_forward_noalloc": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                        _vp, _f32, _f32, _vp, _vp, _vp, _vp, _u32]),
    "e2f_attn_noalloc_max_bytes": (_sz, []),
    "e2f_attn_backward_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32]),
    "e2f_attn_backward": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _f32, _f32, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                 _u32]),
    "e2f_attn_backward_proj_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32]),
    "e2f_attn_backward_proj": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _f32, _f32, _vp, _vp, _sz, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _u32]),
    "e2f_neighbour_workspace_bytes": (_sz, [_i64]),
    "e2f_neighbour_list": (_i32, [_vp, _i64, _i32, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _sz]),
    "e2f_frames": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
}


def hip_runtimes_mapped(maps_text: Optional[str] = None) -> list:
    """Distinct HIP runtime files (libamdhip64*) mapped into this process.

    Read from /proc/self/maps (or the given text in that format); files are
    compared after resolving symbolic links.
    """
    if maps_text is None:
        with open("/proc/self/maps") as f:
            maps_text = f.read()
    found = set()
    for line in maps_text.splitlines():
        parts = line.split(None, 5)
        if len(parts) == 6:
            path = parts[5].strip()
            if os.path.basename(path).startswith("libamdhip64"):
                found.add(os.path.realpath(path) if os.path.exists(path) else path)
    return sorted(found)


def _check_one_runtime(maps_text: Optional[str] = None) -> None:
    found = hip_runtimes_mapped(maps_text)
    if len(found) > 1:
        raise ImportError(
            "two HIP runtimes are mapped into this process (" + ", ".join(found) + "): "
            "libe2f.so was loaded before torch.  Device pointers and streams of one runtime are "
            "invalid in the other; import torch (or this package) before loading libe2f.so by "
            "hand, in a fresh process.")


def _load():
    # torch first: its wheel ships its own HIP runtime (requested as
    # libamdhip64.so), while libe2f.so asks for libamdhip64.so.7.  Loading
    # torch first makes the library bind to that same runtime, so the streams
    # and device pointers torch hands over are valid in it.  Loaded the other
    # way round, the process would hold two HIP runtimes: refuse that.
    _check_one_runtime()
    import torch  # noqa: F401
    _check_one_runtime()
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python interatomic_potentials_amd/build.py` (no fallback exists)")
    so = ctypes.CDLL(LIB_PATH)
    _check_one_runtime()
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


lib = _load()


class E2FError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = f"{where}: {status_string(code)} ({code})"
        if code == STATUS_CODES["E2F_ERR_HIP"]:
            msg += f" [{lib.e2f_last_hip_error_name().decode()} = {lib.e2f_last_hip_error()}]"
        super().__init__(msg)
        self.code = code
        self.name = status_string(code)


def status_string(code: int) -> str:
    return lib.e2f_status_string(code).decode()


def path_count(lmax: int) -> int:
    return lib.e2f_path_count(lmax)


def _flags(validate: bool, targets_in_order: bool, msg_f32: bool = False,
           shared_rows: bool = False, matrix_tiles: bool = False) -> int:
    return ((VALIDATE_INDICES if validate else 0) | (TARGETS_IN_ORDER if targets_in_order else 0)
            | (MSG_F32 if msg_f32 else 0) | (SHARED_ROWS if shared_rows else 0)
            | (MATRIX_TILES if matrix_tiles else 0))


def _check(code: int, where: str) -> None:
    if code != 0:
        raise E2FError(code, where)


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"features must be float32 or bfloat16, got {t.dtype}")


def _dev(t, name: str, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t, name: str, shape) -> None:
    """Raise ValueError unless tensor t (if given) has exactly this shape.

    The C ABI receives bare pointers, so this is the one place where a buffer
    too small for the sizes passed alongside it can be caught.
    """
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _same_device(**tensors) -> None:
    devs = {n: t.device for n, t in tensors.items() if t is not None}
    if len(set(devs.values())) > 1:
        raise ValueError("tensors live on different devices: "
                         + ", ".join(f"{n} on {d}" for n, d in devs.items()))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _lmax_of(S: int) -> int:
    l = int(round(math.sqrt(S))) - 1
    if (l + 1) ** 2 != S:
        raise ValueError(f"component axis {S} is not a square (lmax+1)^2")
    return l


class _HostWeights:
    """Per-path weights as a host float32 array (kept alive for the call)."""

    def __init__(self, path_w):
        import numpy as np
        if path_w is None:
            self.arr = None
            return
        if hasattr(path_w, "detach"):
            path_w = path_w.detach().cpu().numpy()
        self.arr = np.ascontiguousarray(np.asarray(path_w, dtype=np.float32).reshape(-1))

    def data_ptr(self):
        return self.arr.ctypes.data


def _path_w(path_w, device=None):
    w = _HostWeights(path_w)
    return None if w.arr is None else w


# ------------------------------------------------------------ entry points
#
# Every entry point checks shapes first (ValueError), then that the tensors are
# contiguous GPU tensors of the right dtype on one device, and only then calls
# the library, so a mismatched buffer never reaches a kernel.

def _dims(h, name="h"):
    if h.dim() != 3:
        raise ValueError(f"{name} must be [N, S, C], got {list(h.shape)}")
    return tuple(h.shape)


def _nbr_dims(nbr_idx, nbr_mask, N):
    if nbr_idx.dim() != 2:
        raise ValueError(f"nbr_idx must be [N, K], got {list(nbr_idx.shape)}")
    K = nbr_idx.shape[1]
    _shape(nbr_idx, "nbr_idx", (N, K))
    _shape(nbr_mask, "nbr_mask", (N, K))
    return K


def eaas_couple(r, h, path_w=None, out=None):
    """h (x) R(r) through EAAS: r [n,3] fp32, h [n,S,C] fp32|bf16 -> [n,S,C]."""
    return _couple(lib.e2f_eaas_couple, "e2f_eaas_couple", r, h, path_w, out)


def dense_couple(r, h, path_w=None, out=None):
    """h (x) R(r) by the dense Clebsch-Gordan contraction (the baseline EAAS replaces)."""
    return _couple(lib.e2f_dense_couple, "e2f_dense_couple", r, h, path_w, out)


def _couple(fn, where, r, h, path_w, out):
    torch = _torch()
    n, S, C = _dims(h)
    lmax = _lmax_of(S)
    _shape(r, "r", (n, 3))
    _shape(out, "out", (n, S, C))
    _dev(r, "r", torch.float32)
    _dev(h, "h")
    if out is None:
        out = torch.empty_like(h)
    _dev(out, "out", h.dtype)
    _same_device(r=r, h=h, out=out)
    pw = _path_w(path_w, h.device)
    _check(fn(_stream(h), n, lmax, C, _dtype_code(h), _ptr(r), _ptr(h), _ptr(pw), _ptr(out)),
           where)
    return out


def attn_workspace_bytes(N: int, lmax: int, C: int, dtype: int = F32) -> int:
    return int(lib.e2f_attn_workspace_bytes(N, lmax, C, dtype))


def _new_workspace(N, lmax, C, dt, device):
    torch = _torch()
    nbytes = attn_workspace_bytes(N, lmax, C, dt)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _proj_shapes(proj, C, lmax):
    """Shape check of (w_q, w_k, w_v): [C, C], [C, C], [lmax + 1, C, C]."""
    if proj is None:
        return
    w_q, w_k, w_v = proj
    for t, name, shape in ((w_q, "w_q", (C, C)), (w_k, "w_k", (C, C)),
                           (w_v, "w_v", (lmax + 1, C, C))):
        _shape(t, name, shape)


def _proj_weights(proj, h, lmax):
    """(w_q, w_k, w_v) as device tensors of h's dtype: [C, C], [C, C], [lmax + 1, C, C]."""
    if proj is None:
        return None
    _proj_shapes(proj, h.shape[2], lmax)
    for t, name in zip(proj, ("w_q", "w_k", "w_v")):
        _dev(t, name, h.dtype)
        _same_device(h=h, **{name: t})
    return tuple(proj)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def attn_precouple(pos, h, ws=None, path_w=None, proj=None):
    """Step 1 into the workspace (allocated here if not given); returns it.

    ``proj`` = (w_q, w_k, w_v) adds the learned projections (q = h[l=0] w_q,
    k = h[l=0] w_k, v[l] = h[l] w_v[l] before the coupling) on the matrix cores.
    """
    torch = _torch()
    N, S, C = _dims(h)
    lmax = _lmax_of(S)
    _shape(pos, "pos", (N, 3))
    _proj_shapes(proj, C, lmax)
    _dev(pos, "pos", torch.float32)
    _dev(h, "h")
    dt = _dtype_code(h)
    if ws is None:
        ws = _new_workspace(N, lmax, C, dt, h.device)
    _dev(ws, "ws")
    _same_device(pos=pos, h=h, ws=ws)
    pw = _path_w(path_w, h.device)
    w = _proj_weights(proj, h, lmax)
    if w is None:
        _check(lib.e2f_attn_precouple(_stream(h), N, lmax, C, dt, _ptr(pos), _ptr(h), _ptr(pw),
                                      _ptr(ws), _nbytes(ws)),
               "e2f_attn_precouple")
    else:
        _check(lib.e2f_attn_precouple_proj(_stream(h), N, lmax, C, dt, _ptr(pos), _ptr(h),
                                           _ptr(w[0]), _ptr(w[1]), _ptr(w[2]), _ptr(pw), _ptr(ws),
                                           _nbytes(ws)),
               "e2f_attn_precouple_proj")
    return ws


def _results(out, msg, lse):
    extra = tuple(t for t in (msg, lse) if t is not None)
    return (out,) + extra if extra else out


def attn_aggregate(pos, nbr_idx, nbr_mask, ws, heads: int, lmax: int, C: int, dtype,
                   scale: Optional[float] = None, path_w=None, out=None,
                   return_msg: bool = False, validate: bool = False,
                   targets_in_order: bool = False, return_lse: bool = False,
                   env_cutoff: Optional[float] = None, msg_f32: bool = False,
                   shared_rows: bool = False, matrix_tiles: bool = False):
    """Steps 2-3 from a filled workspace; returns out, or (out[, m][, lse]) when asked.

    ``env_cutoff`` = r_env switches on the smooth distance envelope of the weights;
    ``msg_f32`` stores m in float32 whatever the storage type (what attn_backward takes).
    """
    torch = _torch()
    if nbr_idx.dim() != 2:
        raise ValueError(f"nbr_idx must be [N, K], got {list(nbr_idx.shape)}")
    N = nbr_idx.shape[0]
    K = _nbr_dims(nbr_idx, nbr_mask, N)
    S = (lmax + 1) ** 2
    _shape(pos, "pos", (N, 3))
    _shape(out, "out", (N, S, C))
    _dev(pos, "pos", torch.float32)
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    _dev(ws, "ws")
    if out is None:
        out = torch.empty((N, S, C), dtype=dtype, device=ws.device)
    _dev(out, "out", dtype)
    _same_device(pos=pos, nbr_idx=nbr_idx, nbr_mask=nbr_mask, ws=ws, out=out)
    msg = None
    if return_msg:
        msg = torch.empty_like(out, dtype=torch.float32 if msg_f32 else out.dtype)
    lse = torch.empty((N, heads), dtype=torch.float32, device=ws.device) if return_lse else None
    pw = _path_w(path_w, ws.device)
    _check(lib.e2f_attn_aggregate(_stream(ws), N, K, lmax, C, heads, _dtype_code(out), _ptr(pos),
                                  _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                  float(env_cutoff or 0.0), _ptr(pw),
                                  _ptr(ws), _nbytes(ws), _ptr(out), _ptr(msg),
                                  _ptr(lse),
                                  _flags(validate, targets_in_order, msg_f32, shared_rows,
                                         matrix_tiles)),
           "e2f_attn_aggregate")
    return _results(out, msg, lse)


def attn_forward(pos, h, nbr_idx, nbr_mask, heads: int, scale: Optional[float] = None,
                 path_w=None, ws=None, out=None, return_msg: bool = False,
                 validate: bool = False, targets_in_order: bool = False,
                 return_lse: bool = False, proj=None, env_cutoff: Optional[float] = None,
                 shared_rows: bool = False, matrix_tiles: bool = False):
    """Full path (steps 1-3): pos [N,3] fp32, h [N,S,C], nbr_idx [N,K] int32, nbr_mask [N,K] uint8.

    Returns out, or (out[, m][, lse]) when return_msg / return_lse ask for them.
    ``proj`` = (w_q, w_k, w_v) adds the learned projections (see attn_precouple);
    ``env_cutoff`` = r_env the smooth distance envelope of the weights;
    ``shared_rows`` runs the kernels in which several targets of a wave share rows at any N
    (E2F_SHARED_ROWS; by default above 4,096 atoms only); ``matrix_tiles`` the 16-target
    matrix-core aggregate at any N where it serves the layout (E2F_MATRIX_TILES).
    """
    torch = _torch()
    N, S, C = _dims(h)
    lmax = _lmax_of(S)
    K = _nbr_dims(nbr_idx, nbr_mask, N)
    _shape(pos, "pos", (N, 3))
    _shape(out, "out", (N, S, C))
    _proj_shapes(proj, C, lmax)
    _dev(pos, "pos", torch.float32)
    _dev(h, "h")
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    dt = _dtype_code(h)
    if ws is None:
        ws = _new_workspace(N, lmax, C, dt, h.device)
    _dev(ws, "ws")
    if out is None:
        out = torch.empty_like(h)
    _dev(out, "out", h.dtype)
    _same_device(pos=pos, h=h, nbr_idx=nbr_idx, nbr_mask=nbr_mask, ws=ws, out=out)
    msg = torch.empty_like(h) if return_msg else None
    lse = torch.empty((N, heads), dtype=torch.float32, device=h.device) if return_lse else None
    pw = _path_w(path_w, h.device)
    w = _proj_weights(proj, h, lmax)
    if w is None:
        _check(lib.e2f_attn_forward(_stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h),
                                    _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                    float(env_cutoff or 0.0), _ptr(pw),
                                    _ptr(ws), _nbytes(ws), _ptr(out), _ptr(msg),
                                    _ptr(lse),
                                    _flags(validate, targets_in_order, shared_rows=shared_rows,
                                           matrix_tiles=matrix_tiles)),
               "e2f_attn_forward")
    else:
        _check(lib.e2f_attn_forward_proj(_stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h),
                                         _ptr(w[0]), _ptr(w[1]), _ptr(w[2]), _ptr(nbr_idx),
                                         _ptr(nbr_mask), float(scale or 0.0),
                                         float(env_cutoff or 0.0), _ptr(pw), _ptr(ws),
                                         _nbytes(ws), _ptr(out), _ptr(msg),
                                         _ptr(lse),
                                         _flags(validate, targets_in_order,
                                                shared_rows=shared_rows,
                                                matrix_tiles=matrix_tiles)),
               "e2f_attn_forward_proj")
    return _results(out, msg, lse)


def attn_noalloc_max_bytes() -> int:
    """Size of the static per-GPU workspace of attn_forward_noalloc."""
    return int(lib.e2f_attn_noalloc_max_bytes())


def attn_forward_noalloc(pos, h, nbr_idx, nbr_mask, heads: int, scale: Optional[float] = None,
                         path_w=None, out=None, return_msg: bool = False,
                         validate: bool = False, targets_in_order: bool = False,
                         return_lse: bool = False, env_cutoff: Optional[float] = None,
                         shared_rows: bool = False, matrix_tiles: bool = False):
    """attn_forward with the library's static per-GPU workspace instead of a caller's one.

    The library call allocates nothing; pass ``out`` (and use no return_msg / return_lse)
    for a call in which torch allocates nothing either.  Calls overlapping on one GPU race.
    """
    torch = _torch()
    N, S, C = _dims(h)
    lmax = _lmax_of(S)
    K = _nbr_dims(nbr_idx, nbr_mask, N)
    _shape(pos, "pos", (N, 3))
    _shape(out, "out", (N, S, C))
    _dev(pos, "pos", torch.float32)
    _dev(h, "h")
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    dt = _dtype_code(h)
    if out is None:
        out = torch.empty_like(h)
    _dev(out, "out", h.dtype)
    _same_device(pos=pos, h=h, nbr_idx=nbr_idx, nbr_mask=nbr_mask, out=out)
    msg = torch.empty_like(h) if return_msg else None
    lse = torch.empty((N, heads), dtype=torch.float32, device=h.device) if return_lse else None
    pw = _path_w(path_w, h.device)
    _check(lib.e2f_attn_forward_noalloc(_stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h),
                                        _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                        float(env_cutoff or 0.0), _ptr(pw), _ptr(out), _ptr(msg),
                                        _ptr(lse),
                                        _flags(validate, targets_in_order,
                                               shared_rows=shared_rows,
                                               matrix_tiles=matrix_tiles)),
           "e2f_attn_forward_noalloc")
    return _results(out, msg, lse)


def attn_backward_workspace_bytes(N: int, K: int, lmax: int, C: int, H: int,
                                  dtype: int = F32) -> int:
    return int(lib.e2f_attn_backward_workspace_bytes(N, K, lmax, C, H, dtype))


def attn_backward_proj_workspace_bytes(N: int, K: int, lmax: int, C: int, H: int,
                                       dtype: int = F32) -> int:
    return int(lib.e2f_attn_backward_proj_workspace_bytes(N, K, lmax, C, H, dtype))


def attn_backward(pos, h, nbr_idx, nbr_mask, heads: int, ws, msg, lse, grad_out,
                  scale: Optional[float] = None, path_w=None, targets_in_order: bool = False,
                  bwd_ws=None, grad_h=None, grad_pos=None, env_cutoff: Optional[float] = None,
                  proj=None, shared_rows: bool = False, matrix_tiles: bool = False):
    """(dL/dh, dL/dpos) for L = <grad_out, out>; ws, msg, lse from the forward.

    With bf16 storage the library recomputes the message and the log-sum-exp in fp32, so
    msg and lse may be None (they are not read).  ``proj`` = (w_q, w_k, w_v), the weights
    the forward's workspace was built with: the gradients go through the projections, and
    (dL/dh, dL/dpos, dL/dW_Q, dL/dW_K, dL/dW_V) is returned, the weight gradients in fp32.
    """
    torch = _torch()
    N, S, C = _dims(h)
    lmax = _lmax_of(S)
    w = _proj_weights(proj, h, lmax)
    K = _nbr_dims(nbr_idx, nbr_mask, N)
    _shape(pos, "pos", (N, 3))
    for t, name in ((msg, "msg"), (grad_out, "grad_out"), (grad_h, "grad_h")):
        _shape(t, name, (N, S, C))
    _shape(lse, "lse", (N, heads))
    _shape(grad_pos, "grad_pos", (N, 3))
    _dev(pos, "pos", torch.float32)
    _dev(h, "h")
    dt = _dtype_code(h)
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    _dev(ws, "ws")
    if dt == F32 or msg is not None:
        _dev(msg, "msg", torch.float32)
    if dt == F32 or lse is not None:
        _dev(lse, "lse", torch.float32)
    _dev(grad_out, "grad_out", h.dtype)
    if bwd_ws is None:
        nbytes = (attn_backward_workspace_bytes if w is None
                  else attn_backward_proj_workspace_bytes)(N, K, lmax, C, heads, dt)
        bwd_ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=h.device)
    _dev(bwd_ws, "bwd_ws")
    grad_h = torch.empty_like(h) if grad_h is None else _dev(grad_h, "grad_h", h.dtype)
    grad_pos = (torch.empty_like(pos) if grad_pos is None
                else _dev(grad_pos, "grad_pos", torch.float32))
    _same_device(pos=pos, h=h, nbr_idx=nbr_idx, nbr_mask=nbr_mask, ws=ws, msg=msg, lse=lse,
                 grad_out=grad_out, bwd_ws=bwd_ws, grad_h=grad_h, grad_pos=grad_pos)
    pw = _path_w(path_w, h.device)
    flags = ((TARGETS_IN_ORDER if targets_in_order else 0)
             | (SHARED_ROWS if shared_rows else 0) | (MATRIX_TILES if matrix_tiles else 0))
    if w is not None:
        gw = (torch.empty((C, C), dtype=torch.float32, device=h.device),
              torch.empty((C, C), dtype=torch.float32, device=h.device),
              torch.empty((lmax + 1, C, C), dtype=torch.float32, device=h.device))
        _check(lib.e2f_attn_backward_proj(
            _stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h), _ptr(w[0]), _ptr(w[1]),
            _ptr(w[2]), _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
            float(env_cutoff or 0.0), _ptr(pw), _ptr(ws), _nbytes(ws), _ptr(msg), _ptr(lse),
            _ptr(grad_out), _ptr(grad_h), _ptr(grad_pos), _ptr(gw[0]), _ptr(gw[1]), _ptr(gw[2]),
            _ptr(bwd_ws), _nbytes(bwd_ws), flags), "e2f_attn_backward_proj")
        return (grad_h, grad_pos) + gw
    _check(lib.e2f_attn_backward(_stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h),
                                 _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                 float(env_cutoff or 0.0), _ptr(pw),
                                 _ptr(ws), _nbytes(ws), _ptr(msg), _ptr(lse),
                                 _ptr(grad_out), _ptr(grad_h), _ptr(grad_pos), _ptr(bwd_ws),
                                 _nbytes(bwd_ws), flags),
           "e2f_attn_backward")
    return grad_h, grad_pos


def neighbour_workspace_bytes(N: int) -> int:
    return int(lib.e2f_neighbour_workspace_bytes(N))


def neighbour_list(pos, cutoff: float, K: int, return_n_within: bool = False,
                   return_order: bool = False, ws=None):
    """Padded neighbour rows (nbr_idx [N,K] int32, nbr_mask [N,K] uint8) built on the GPU.

    Row i lists the atoms j != i closer than ``cutoff`` by increasing (distance, j),
    the first K of them; see e2f_neighbour_list in include/e2f.h.  Also returns
    n_within [N] int32 (the count before truncation) and/or order [N] int32 (atoms
    grouped by cell in Morton order) when asked.
    """
    torch = _torch()
    if pos.dim() != 2 or pos.shape[1] != 3:
        raise ValueError(f"pos must be [N, 3], got {list(pos.shape)}")
    _dev(pos, "pos", torch.float32)
    N = pos.shape[0]
    dev = pos.device
    idx = torch.empty((N, K), dtype=torch.int32, device=dev)
    mask = torch.empty((N, K), dtype=torch.uint8, device=dev)
    nw = torch.empty(N, dtype=torch.int32, device=dev) if return_n_within else None
    order = torch.empty(N, dtype=torch.int32, device=dev) if return_order else None
    if ws is None:
        ws = torch.empty(max(neighbour_workspace_bytes(N), 1), dtype=torch.uint8, device=dev)
    _dev(ws, "ws")
    _same_device(pos=pos, ws=ws)
    _check(lib.e2f_neighbour_list(_stream(pos), N, K, float(cutoff), _ptr(pos), _ptr(idx),
                                  _ptr(mask), _ptr(nw), _ptr(order), _ptr(ws),
                                  _nbytes(ws)), "e2f_neighbour_list")
    return (idx, mask) + tuple(t for t in (nw, order) if t is not None)


def frames(r, lmax: int = 2):
    """Alignment rotations Q [n,9] and Wigner-D blocks D [n,35] as the kernels build them."""
    torch = _torch()
    if r.dim() != 2 or r.shape[1] != 3:
        raise ValueError(f"r must be [n, 3], got {list(r.shape)}")
    _dev(r, "r", torch.float32)
    n = r.shape[0]
    Q = torch.zeros((n, 9), dtype=torch.float32, device=r.device)
    D = torch.zeros((n, 35), dtype=torch.float32, device=r.device)
    _check(lib.e2f_frames(_stream(r), n, lmax, _ptr(r), _ptr(Q), _ptr(D)), "e2f_frames")
    return Q, D
