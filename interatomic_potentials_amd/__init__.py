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
    "E2FError", "lib", "status_string", "path_count", "eaas_couple", "attn_workspace_bytes",
    "attn_precouple", "attn_aggregate", "attn_forward", "attn_backward",
    "attn_backward_workspace_bytes", "neighbour_workspace_bytes", "neighbour_list", "frames",
    "F32", "BF16",
    "VALIDATE_INDICES", "TARGETS_IN_ORDER",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libe2f.so")

F32 = 0
BF16 = 1
VALIDATE_INDICES = 1
TARGETS_IN_ORDER = 2

_STATUS = {
    0: "E2F_OK", -1: "E2F_ERR_NULL", -2: "E2F_ERR_SHAPE", -3: "E2F_ERR_DTYPE",
    -4: "E2F_ERR_ALIGN", -5: "E2F_ERR_WORKSPACE", -6: "E2F_ERR_ALIAS", -7: "E2F_ERR_HIP",
    -8: "E2F_ERR_INDEX", -9: "E2F_ERR_UNSUPPORTED",
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
    "e2f_attn_backward_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32]),
    "e2f_attn_backward": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _f32, _f32, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                 _u32]),
    "e2f_neighbour_workspace_bytes": (_sz, [_i64]),
    "e2f_neighbour_list": (_i32, [_vp, _i64, _i32, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _sz]),
    "e2f_frames": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
}


def _load():
    # torch first: its wheel ships its own HIP runtime (requested as
    # libamdhip64.so), while libe2f.so asks for libamdhip64.so.7.  Loading
    # torch first makes the library bind to that same runtime, so the streams
    # and device pointers torch hands over are valid in it.  Loaded the other
    # way round, the process would hold two HIP runtimes.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python interatomic_potentials_amd/build.py` (no fallback exists)")
    so = ctypes.CDLL(LIB_PATH)
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


def _flags(validate: bool, targets_in_order: bool) -> int:
    return (VALIDATE_INDICES if validate else 0) | (TARGETS_IN_ORDER if targets_in_order else 0)


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

def eaas_couple(r, h, path_w=None, out=None):
    """h (x) R(r) through EAAS: r [n,3] fp32, h [n,S,C] fp32|bf16 -> [n,S,C]."""
    torch = _torch()
    _dev(r, "r", torch.float32)
    _dev(h, "h")
    n, S, C = h.shape
    lmax = _lmax_of(S)
    if r.shape != (n, 3):
        raise ValueError("r must be [n, 3]")
    pw = _path_w(path_w, h.device)
    if out is None:
        out = torch.empty_like(h)
    _dev(out, "out", h.dtype)
    _check(lib.e2f_eaas_couple(_stream(h), n, lmax, C, _dtype_code(h), _ptr(r), _ptr(h), _ptr(pw),
                               _ptr(out)), "e2f_eaas_couple")
    return out


def attn_workspace_bytes(N: int, lmax: int, C: int, dtype: int = F32) -> int:
    return int(lib.e2f_attn_workspace_bytes(N, lmax, C, dtype))


def _new_workspace(N, lmax, C, dt, device):
    torch = _torch()
    nbytes = attn_workspace_bytes(N, lmax, C, dt)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _proj_weights(proj, h, lmax):
    """(w_q, w_k, w_v) as device tensors of h's dtype: [C, C], [C, C], [lmax + 1, C, C]."""
    if proj is None:
        return None
    w_q, w_k, w_v = proj
    C = h.shape[2]
    for t, name, shape in ((w_q, "w_q", (C, C)), (w_k, "w_k", (C, C)),
                           (w_v, "w_v", (lmax + 1, C, C))):
        _dev(t, name, h.dtype)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    return w_q, w_k, w_v


def attn_precouple(pos, h, ws=None, path_w=None, proj=None):
    """Step 1 into the workspace (allocated here if not given); returns it.

    ``proj`` = (w_q, w_k, w_v) adds the learned projections (q = h[l=0] w_q,
    k = h[l=0] w_k, v[l] = h[l] w_v[l] before the coupling) on the matrix cores.
    """
    torch = _torch()
    _dev(pos, "pos", torch.float32)
    _dev(h, "h")
    N, S, C = h.shape
    lmax = _lmax_of(S)
    dt = _dtype_code(h)
    if ws is None:
        ws = _new_workspace(N, lmax, C, dt, h.device)
    _dev(ws, "ws")
    pw = _path_w(path_w, h.device)
    w = _proj_weights(proj, h, lmax)
    if w is None:
        _check(lib.e2f_attn_precouple(_stream(h), N, lmax, C, dt, _ptr(pos), _ptr(h), _ptr(pw),
                                      _ptr(ws), ws.numel() * ws.element_size()),
               "e2f_attn_precouple")
    else:
        _check(lib.e2f_attn_precouple_proj(_stream(h), N, lmax, C, dt, _ptr(pos), _ptr(h),
                                           _ptr(w[0]), _ptr(w[1]), _ptr(w[2]), _ptr(pw), _ptr(ws),
                                           ws.numel() * ws.element_size()),
               "e2f_attn_precouple_proj")
    return ws


def _results(out, msg, lse):
    extra = tuple(t for t in (msg, lse) if t is not None)
    return (out,) + extra if extra else out


def attn_aggregate(pos, nbr_idx, nbr_mask, ws, heads: int, lmax: int, C: int, dtype,
                   scale: Optional[float] = None, path_w=None, out=None,
                   return_msg: bool = False, validate: bool = False,
                   targets_in_order: bool = False, return_lse: bool = False,
                   env_cutoff: Optional[float] = None):
    """Steps 2-3 from a filled workspace; returns out, or (out[, m][, lse]) when asked.

    ``env_cutoff`` = r_env switches on the smooth distance envelope of the weights.
    """
    torch = _torch()
    _dev(pos, "pos", torch.float32)
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    _dev(ws, "ws")
    N, K = nbr_idx.shape
    S = (lmax + 1) ** 2
    if out is None:
        out = torch.empty((N, S, C), dtype=dtype, device=ws.device)
    _dev(out, "out", dtype)
    msg = torch.empty_like(out) if return_msg else None
    lse = torch.empty((N, heads), dtype=torch.float32, device=ws.device) if return_lse else None
    pw = _path_w(path_w, ws.device)
    _check(lib.e2f_attn_aggregate(_stream(ws), N, K, lmax, C, heads, _dtype_code(out), _ptr(pos),
                                  _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                  float(env_cutoff or 0.0), _ptr(pw),
                                  _ptr(ws), ws.numel() * ws.element_size(), _ptr(out), _ptr(msg),
                                  _ptr(lse), _flags(validate, targets_in_order)),
           "e2f_attn_aggregate")
    return _results(out, msg, lse)


def attn_forward(pos, h, nbr_idx, nbr_mask, heads: int, scale: Optional[float] = None,
                 path_w=None, ws=None, out=None, return_msg: bool = False,
                 validate: bool = False, targets_in_order: bool = False,
                 return_lse: bool = False, proj=None, env_cutoff: Optional[float] = None):
    """Full path (steps 1-3): pos [N,3] fp32, h [N,S,C], nbr_idx [N,K] int32, nbr_mask [N,K] uint8.

    Returns out, or (out[, m][, lse]) when return_msg / return_lse ask for them.
    ``proj`` = (w_q, w_k, w_v) adds the learned projections (see attn_precouple);
    ``env_cutoff`` = r_env the smooth distance envelope of the weights.
    """
    torch = _torch()
    _dev(pos, "pos", torch.float32)
    _dev(h, "h")
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    N, S, C = h.shape
    K = nbr_idx.shape[1]
    lmax = _lmax_of(S)
    dt = _dtype_code(h)
    if ws is None:
        ws = _new_workspace(N, lmax, C, dt, h.device)
    _dev(ws, "ws")
    if out is None:
        out = torch.empty_like(h)
    _dev(out, "out", h.dtype)
    msg = torch.empty_like(h) if return_msg else None
    lse = torch.empty((N, heads), dtype=torch.float32, device=h.device) if return_lse else None
    pw = _path_w(path_w, h.device)
    w = _proj_weights(proj, h, lmax)
    if w is None:
        _check(lib.e2f_attn_forward(_stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h),
                                    _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                    float(env_cutoff or 0.0), _ptr(pw),
                                    _ptr(ws), ws.numel() * ws.element_size(), _ptr(out), _ptr(msg),
                                    _ptr(lse), _flags(validate, targets_in_order)),
               "e2f_attn_forward")
    else:
        _check(lib.e2f_attn_forward_proj(_stream(h), N, K, lmax, C, heads, dt, _ptr(pos), _ptr(h),
                                         _ptr(w[0]), _ptr(w[1]), _ptr(w[2]), _ptr(nbr_idx),
                                         _ptr(nbr_mask), float(scale or 0.0),
                                         float(env_cutoff or 0.0), _ptr(pw), _ptr(ws),
                                         ws.numel() * ws.element_size(), _ptr(out), _ptr(msg),
                                         _ptr(lse), _flags(validate, targets_in_order)),
               "e2f_attn_forward_proj")
    return _results(out, msg, lse)


def attn_backward_workspace_bytes(N: int, K: int, lmax: int, C: int, H: int,
                                  dtype: int = F32) -> int:
    return int(lib.e2f_attn_backward_workspace_bytes(N, K, lmax, C, H, dtype))


def attn_backward(pos, h, nbr_idx, nbr_mask, heads: int, ws, msg, lse, grad_out,
                  scale: Optional[float] = None, path_w=None, targets_in_order: bool = False,
                  bwd_ws=None, grad_h=None, grad_pos=None, env_cutoff: Optional[float] = None):
    """(dL/dh, dL/dpos) for L = <grad_out, out>; ws, msg, lse from the forward (fp32 only)."""
    torch = _torch()
    _dev(pos, "pos", torch.float32)
    _dev(h, "h", torch.float32)
    _dev(nbr_idx, "nbr_idx", torch.int32)
    _dev(nbr_mask, "nbr_mask", torch.uint8)
    _dev(ws, "ws")
    _dev(msg, "msg", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(grad_out, "grad_out", torch.float32)
    N, S, C = h.shape
    K = nbr_idx.shape[1]
    lmax = _lmax_of(S)
    if bwd_ws is None:
        nbytes = attn_backward_workspace_bytes(N, K, lmax, C, heads, F32)
        bwd_ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=h.device)
    _dev(bwd_ws, "bwd_ws")
    grad_h = torch.empty_like(h) if grad_h is None else _dev(grad_h, "grad_h", torch.float32)
    grad_pos = (torch.empty_like(pos) if grad_pos is None
                else _dev(grad_pos, "grad_pos", torch.float32))
    pw = _path_w(path_w, h.device)
    _check(lib.e2f_attn_backward(_stream(h), N, K, lmax, C, heads, F32, _ptr(pos), _ptr(h),
                                 _ptr(nbr_idx), _ptr(nbr_mask), float(scale or 0.0),
                                 float(env_cutoff or 0.0), _ptr(pw),
                                 _ptr(ws), ws.numel() * ws.element_size(), _ptr(msg), _ptr(lse),
                                 _ptr(grad_out), _ptr(grad_h), _ptr(grad_pos), _ptr(bwd_ws),
                                 bwd_ws.numel() * bwd_ws.element_size(),
                                 TARGETS_IN_ORDER if targets_in_order else 0),
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
    _dev(pos, "pos", torch.float32)
    N = pos.shape[0]
    if pos.shape != (N, 3):
        raise ValueError("pos must be [N, 3]")
    dev = pos.device
    idx = torch.empty((N, K), dtype=torch.int32, device=dev)
    mask = torch.empty((N, K), dtype=torch.uint8, device=dev)
    nw = torch.empty(N, dtype=torch.int32, device=dev) if return_n_within else None
    order = torch.empty(N, dtype=torch.int32, device=dev) if return_order else None
    if ws is None:
        ws = torch.empty(max(neighbour_workspace_bytes(N), 1), dtype=torch.uint8, device=dev)
    _dev(ws, "ws")
    _check(lib.e2f_neighbour_list(_stream(pos), N, K, float(cutoff), _ptr(pos), _ptr(idx),
                                  _ptr(mask), _ptr(nw), _ptr(order), _ptr(ws),
                                  ws.numel() * ws.element_size()), "e2f_neighbour_list")
    return (idx, mask) + tuple(t for t in (nw, order) if t is not None)


def frames(r, lmax: int = 2):
    """Alignment rotations Q [n,9] and Wigner-D blocks D [n,35] as the kernels build them."""
    torch = _torch()
    _dev(r, "r", torch.float32)
    n = r.shape[0]
    Q = torch.zeros((n, 9), dtype=torch.float32, device=r.device)
    D = torch.zeros((n, 35), dtype=torch.float32, device=r.device)
    _check(lib.e2f_frames(_stream(r), n, lmax, _ptr(r), _ptr(Q), _ptr(D)), "e2f_frames")
    return Q, D
