"""ctypes binding for liblizard_attn.so (see include/lizard_attn.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, their device pointers and the current HIP stream are passed to
the C ABI, and non-OK statuses become exceptions.  Every step of the attention
runs in the library's HIP kernels; there is no CPU path here.  torch provides
device memory (outputs, workspace) and streams.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

LIB_PATH = _build.LIB

LIZARD_OK = 0
_STATUS = {0: "LIZARD_OK", 1: "LIZARD_ERR_INVALID_ARG", 2: "LIZARD_ERR_UNSUPPORTED",
           3: "LIZARD_ERR_WORKSPACE", 4: "LIZARD_ERR_HIP"}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

EXPORTED = ("lizard_attn_fwd", "lizard_attn_fwd_workspace_bytes", "lizard_attn_fwd_hedgehog",
            "lizard_attn_fwd_ext", "lizard_attn_fwd_ext_workspace_bytes", "lizard_attn_decode",
            "lizard_attn_decode_hedgehog", "lizard_attn_decode_workspace_bytes",
            "lizard_status_string", "lizard_last_error", "lizard_version", "lizard_set_option",
            "lizard_get_option", "lizard_attn_decode_noalloc", "lizard_attn_bwd",
            "lizard_attn_bwd_hedgehog", "lizard_attn_bwd_workspace_bytes", "lizard_gla_fwd")

_lock = threading.Lock()
_lib = None


class LizardError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def _declare(lib):
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.lizard_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                    i32, i32, i32, i32, i32, i32, i32, f32, f32, i32, vp, sz, vp]
    lib.lizard_attn_fwd.restype = i32
    lib.lizard_attn_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.lizard_attn_fwd_workspace_bytes.restype = sz
    lib.lizard_attn_fwd_ext.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                        i32, i32, i32, i32, i32, i32, i32, f32, f32, i32,
                                        vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lizard_attn_fwd_ext.restype = i32
    lib.lizard_attn_fwd_ext_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.lizard_attn_fwd_ext_workspace_bytes.restype = sz
    lib.lizard_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                       i32, i32, i32, i32, i32, i32, f32, f32, i32, vp, sz, vp]
    lib.lizard_attn_decode.restype = i32
    lib.lizard_attn_fwd_hedgehog.argtypes = lib.lizard_attn_fwd.argtypes
    lib.lizard_attn_fwd_hedgehog.restype = i32
    lib.lizard_attn_decode_hedgehog.argtypes = lib.lizard_attn_decode.argtypes
    lib.lizard_attn_decode_hedgehog.restype = i32
    lib.lizard_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                               i32, i32, i32, i32, i32, i32, f32, f32, i32, vp]
    lib.lizard_attn_decode_noalloc.restype = i32
    lib.lizard_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    i32, i32, i32, i32, i32, i32, i32, f32, f32, i32, vp, sz, vp]
    lib.lizard_attn_bwd.restype = i32
    lib.lizard_attn_bwd_hedgehog.argtypes = lib.lizard_attn_bwd.argtypes
    lib.lizard_attn_bwd_hedgehog.restype = i32
    lib.lizard_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.lizard_attn_bwd_workspace_bytes.restype = sz
    lib.lizard_gla_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.lizard_gla_fwd.restype = i32
    lib.lizard_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.lizard_attn_decode_workspace_bytes.restype = sz
    lib.lizard_status_string.argtypes = [i32]
    lib.lizard_status_string.restype = ctypes.c_char_p
    lib.lizard_last_error.argtypes = []
    lib.lizard_last_error.restype = ctypes.c_char_p
    lib.lizard_version.argtypes = []
    lib.lizard_version.restype = ctypes.c_char_p
    lib.lizard_set_option.argtypes = [ctypes.c_char_p, i32]
    lib.lizard_set_option.restype = i32
    lib.lizard_get_option.argtypes = [ctypes.c_char_p]
    lib.lizard_get_option.restype = i32
    return lib


def load(path: str | None = None):
    """Load the HIP library (building it first only if no build exists)."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                _build.build()
            _lib = _declare(ctypes.CDLL(p))
    return _lib


def _check(status: int):
    if status != LIZARD_OK:
        lib = load()
        raise LizardError(status, lib.lizard_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def lizard_attn_fwd_workspace_bytes(B: int, Hq: int, Hkv: int, L: int, d: int, W: int,
                                    dtype: torch.dtype) -> int:
    return int(load().lizard_attn_fwd_workspace_bytes(B, Hq, Hkv, L, d, W, _DTYPES[dtype]))


def set_option(name: str, value: int) -> None:
    """Set a tuning / test option of the library (see lizard_set_option in the header)."""
    _check(load().lizard_set_option(name.encode(), int(value)))


def get_option(name: str) -> int:
    return int(load().lizard_get_option(name.encode()))


def _w_stride(w_q, w_k, d, Hq, Hkv, cols=None):
    cols = d if cols is None else cols
    if w_q.shape[-2:] != (d, cols) or w_k.shape[-2:] != (d, cols):
        raise ValueError(f"w_phi_q and w_phi_k must end in [{d},{cols}] for this feature map")
    if w_q.dim() == 2 and w_k.dim() == 2:
        return 0
    if w_q.dim() == 3 and w_k.dim() == 3:
        if w_q.shape[0] != Hq or w_k.shape[0] != Hkv:
            raise ValueError(f"per-head w_phi_q must be [{Hq},{d},{cols}] and w_phi_k [{Hkv},{d},{cols}]")
        return d * cols
    raise ValueError("w_phi_q and w_phi_k must both be shared or both per head")


def _out(out, like, name="out"):
    if out is None:
        return torch.empty_like(like)
    _dev(out, name, like.dtype)
    if out.shape != like.shape or out.device != like.device:
        raise ValueError(f"{name} must be {tuple(like.shape)} on {like.device}")
    return out


def _workspace(workspace, need, device):
    """The caller's workspace (a uint8 GPU tensor of at least `need` bytes on `device`), or a
    new one when None and `need` > 0."""
    if workspace is None:
        return None if need == 0 else torch.empty(need, dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", torch.uint8)
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}")
    if workspace.numel() < need:
        raise ValueError(f"workspace of {need} bytes needed, got {workspace.numel()}")
    return workspace


def _same_device(dev, *named):
    for t, n in named:
        if t is not None and t.device != dev:
            raise ValueError(f"{n} must be on {dev}")


def lizard_attn_fwd(q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, *, W: int, M: int,
                    mix: float = 0.5, scale: float | None = None, out=None, workspace=None,
                    stream=None):
    """Lizard attention forward on the GPU.  Shapes: q [B,Hq,L,d]; k, v, log_gamma
    [B,Hkv,L,d]; w_phi_q/w_phi_k [d,d] or [Hq|Hkv,d,d]; t_k, t_v [Hkv,M,d].
    Returns out [B,Hq,L,d] in the input dtype."""
    return _fwd(load().lizard_attn_fwd, q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, W=W, M=M,
                mix=mix, scale=scale, out=out, workspace=workspace, stream=stream, cols=q.shape[-1])


def lizard_attn_fwd_hedgehog(q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, *, W: int, M: int,
                             mix: float = 0.5, scale: float | None = None, out=None,
                             workspace=None, stream=None):
    """Forward with the Hedgehog map phi(x) = exp(xW) (+) exp(-xW): w_phi_q/w_phi_k [d, d/2] or
    per head [Hq|Hkv, d, d/2].  Otherwise as lizard_attn_fwd."""
    return _fwd(load().lizard_attn_fwd_hedgehog, q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v,
                W=W, M=M, mix=mix, scale=scale, out=out, workspace=workspace, stream=stream,
                cols=q.shape[-1] // 2)


def _fwd(fn, q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, *, W, M, mix, scale, out,
         workspace, stream, cols):
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"),
                 (w_phi_k, "w_phi_k")):
        _dev(t, n, dt)
    if M > 0:
        _dev(t_k, "t_k", dt)
        _dev(t_v, "t_v", dt)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or v.shape != k.shape or log_gamma.shape != k.shape:
        raise ValueError("k, v, log_gamma must be [B,Hkv,L,d] matching q")
    if M > 0 and (t_k.shape != (Hkv, M, d) or t_v.shape != (Hkv, M, d)):
        raise ValueError("t_k, t_v must be [Hkv,M,d]")
    _same_device(q.device, (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"),
                 (w_phi_k, "w_phi_k"), (t_k if M > 0 else None, "t_k"), (t_v if M > 0 else None, "t_v"))
    wstride = _w_stride(w_phi_q, w_phi_k, d, Hq, Hkv, cols)
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q)
    need = lizard_attn_fwd_workspace_bytes(B, Hq, Hkv, L, d, W, dt)
    workspace = _workspace(workspace, need, q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(w_phi_q), _ptr(w_phi_k),
        wstride, _ptr(t_k) if M > 0 else None, _ptr(t_v) if M > 0 else None,
        _ptr(out), B, Hq, Hkv, L, d, W, M, float(mix), float(scale), _DTYPES[dt],
        _ptr(workspace), wbytes, _stream(stream)))
    return out


def lizard_attn_fwd_ext_workspace_bytes(B: int, Hq: int, Hkv: int, L: int, d: int, W: int,
                                        dtype: torch.dtype) -> int:
    return int(load().lizard_attn_fwd_ext_workspace_bytes(B, Hq, Hkv, L, d, W, _DTYPES[dtype]))


def lizard_attn_fwd_ext(q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, *, W: int, M: int,
                        mix: float = 0.5, scale: float | None = None, state_in=None, win_k_in=None,
                        win_v_in=None, pos=None, state_out=None, win_k_out=None, win_v_out=None,
                        out=None, workspace=None, stream=None):
    """Forward over L new tokens that follow pos[b] earlier ones: state_in [B,Hkv,d,d] fp32,
    rings win_k_in/win_v_in [B,Hkv,W,d] (token t in slot t % W), pos [B] int32 (advanced by L);
    state_out, win_k_out/win_v_out receive the state and ring after the call.  Any of them may
    be None.  Shapes otherwise as lizard_attn_fwd.  Returns out."""
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"),
                 (w_phi_k, "w_phi_k")):
        _dev(t, n, dt)
    if M > 0:
        _dev(t_k, "t_k", dt)
        _dev(t_v, "t_v", dt)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or v.shape != k.shape or log_gamma.shape != k.shape:
        raise ValueError("k, v, log_gamma must be [B,Hkv,L,d] matching q")
    for t, n in ((state_in, "state_in"), (state_out, "state_out")):
        if t is not None:
            _dev(t, n, torch.float32)
            if t.shape != (B, Hkv, d, d):
                raise ValueError(f"{n} must be [B,Hkv,d,d]")
    for t, n in ((win_k_in, "win_k_in"), (win_v_in, "win_v_in"), (win_k_out, "win_k_out"),
                 (win_v_out, "win_v_out")):
        if t is not None:
            _dev(t, n, dt)
            if t.shape != (B, Hkv, W, d):
                raise ValueError(f"{n} must be [B,Hkv,W,d]")
    if pos is not None:
        _dev(pos, "pos", torch.int32)
        if pos.shape != (B,):
            raise ValueError("pos must be [B]")
    if M > 0 and (t_k.shape != (Hkv, M, d) or t_v.shape != (Hkv, M, d)):
        raise ValueError("t_k, t_v must be [Hkv,M,d]")
    _same_device(q.device, (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"),
                 (w_phi_k, "w_phi_k"), (t_k if M > 0 else None, "t_k"), (t_v if M > 0 else None, "t_v"),
                 (state_in, "state_in"), (state_out, "state_out"), (win_k_in, "win_k_in"),
                 (win_v_in, "win_v_in"), (win_k_out, "win_k_out"), (win_v_out, "win_v_out"), (pos, "pos"))
    wstride = _w_stride(w_phi_q, w_phi_k, d, Hq, Hkv)
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q)
    need = lizard_attn_fwd_ext_workspace_bytes(B, Hq, Hkv, L, d, W, dt)
    workspace = _workspace(workspace, need, q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().lizard_attn_fwd_ext(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(w_phi_q), _ptr(w_phi_k),
        wstride, _ptr(t_k) if M > 0 else None, _ptr(t_v) if M > 0 else None,
        _ptr(out), B, Hq, Hkv, L, d, W, M, float(mix), float(scale), _DTYPES[dt],
        _ptr(state_in), _ptr(win_k_in), _ptr(win_v_in), _ptr(pos), _ptr(state_out), _ptr(win_k_out),
        _ptr(win_v_out), _ptr(workspace), wbytes, _stream(stream)))
    return out


def lizard_attn_decode_workspace_bytes(N: int, Hq: int, Hkv: int, d: int, dtype: torch.dtype) -> int:
    return int(load().lizard_attn_decode_workspace_bytes(N, Hq, Hkv, d, _DTYPES[dtype]))


def lizard_attn_decode(state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v,
                       *, M: int, mix: float = 0.5, scale: float | None = None, out=None,
                       workspace=None, stream=None):
    """One decode step, in place on state [N,Hkv,d,d] fp32, win_k/win_v [N,Hkv,W,d],
    pos [N] int32.  q [N,Hq,d]; k, v, log_gamma [N,Hkv,d].  Returns out [N,Hq,d]."""
    return _decode(load().lizard_attn_decode, state, win_k, win_v, pos, q, k, v, log_gamma,
                   w_phi_q, w_phi_k, t_k, t_v, M=M, mix=mix, scale=scale, out=out,
                   workspace=workspace, stream=stream, cols=q.shape[-1])


def lizard_attn_decode_noalloc(state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v,
                               *, M: int, mix: float = 0.5, scale: float | None = None, out=None,
                               stream=None):
    """lizard_attn_decode without a workspace: the library's static per-GPU scratch serves the
    step (calls that overlap on one GPU race).  Arguments and results as lizard_attn_decode."""
    return _decode(load().lizard_attn_decode_noalloc, state, win_k, win_v, pos, q, k, v, log_gamma,
                   w_phi_q, w_phi_k, t_k, t_v, M=M, mix=mix, scale=scale, out=out, workspace=None,
                   stream=stream, cols=q.shape[-1], noalloc=True)


def lizard_attn_decode_hedgehog(state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k,
                                t_k, t_v, *, M: int, mix: float = 0.5, scale: float | None = None,
                                out=None, workspace=None, stream=None):
    """One decode step with the Hedgehog map: w_phi_q/w_phi_k [d, d/2] or [Hq|Hkv, d, d/2].
    Otherwise as lizard_attn_decode."""
    return _decode(load().lizard_attn_decode_hedgehog, state, win_k, win_v, pos, q, k, v,
                   log_gamma, w_phi_q, w_phi_k, t_k, t_v, M=M, mix=mix, scale=scale, out=out,
                   workspace=workspace, stream=stream, cols=q.shape[-1] // 2)


def _decode(fn, state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, *, M,
            mix, scale, out, workspace, stream, cols, noalloc=False):
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _dev(state, "state", torch.float32)
    _dev(pos, "pos", torch.int32)
    for t, n in ((win_k, "win_k"), (win_v, "win_v"), (q, "q"), (k, "k"), (v, "v"),
                 (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"), (w_phi_k, "w_phi_k")):
        _dev(t, n, dt)
    if M > 0:
        _dev(t_k, "t_k", dt)
        _dev(t_v, "t_v", dt)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    W = win_k.shape[2]
    if state.shape != (N, Hkv, d, d) or win_k.shape != (N, Hkv, W, d) or win_v.shape != win_k.shape:
        raise ValueError("state [N,Hkv,d,d] and win_k/win_v [N,Hkv,W,d] expected")
    if k.shape != (N, Hkv, d) or v.shape != k.shape or log_gamma.shape != k.shape or pos.shape != (N,):
        raise ValueError("k, v, log_gamma must be [N,Hkv,d] and pos [N]")
    if M > 0 and (t_k.shape != (Hkv, M, d) or t_v.shape != (Hkv, M, d)):
        raise ValueError("t_k, t_v must be [Hkv,M,d]")
    _same_device(q.device, (state, "state"), (win_k, "win_k"), (win_v, "win_v"), (pos, "pos"), (k, "k"),
                 (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"), (w_phi_k, "w_phi_k"),
                 (t_k if M > 0 else None, "t_k"), (t_v if M > 0 else None, "t_v"))
    wstride = _w_stride(w_phi_q, w_phi_k, d, Hq, Hkv, cols)
    if scale is None:
        scale = d ** -0.5
    out = _out(out, q)
    args = [_ptr(state), _ptr(win_k), _ptr(win_v), _ptr(pos), _ptr(q), _ptr(k), _ptr(v),
            _ptr(log_gamma), _ptr(w_phi_q), _ptr(w_phi_k), wstride,
            _ptr(t_k) if M > 0 else None, _ptr(t_v) if M > 0 else None, _ptr(out),
            N, Hq, Hkv, d, W, M, float(mix), float(scale), _DTYPES[dt]]
    if noalloc:
        _check(fn(*args, _stream(stream)))
        return out
    need = lizard_attn_decode_workspace_bytes(N, Hq, Hkv, d, dt)
    workspace = _workspace(workspace, max(need, 16), q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(fn(*args, _ptr(workspace), wbytes, _stream(stream)))
    return out


def lizard_attn_bwd_workspace_bytes(B: int, Hq: int, Hkv: int, L: int, d: int, M: int,
                                    dtype: torch.dtype) -> int:
    return int(load().lizard_attn_bwd_workspace_bytes(B, Hq, Hkv, L, d, M, _DTYPES[dtype]))


def lizard_attn_bwd(q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, dy, *, W: int, M: int,
                    mix: float = 0.5, scale: float | None = None, feature_map: str = "softmax",
                    workspace=None, stream=None):
    """Backward of lizard_attn_fwd (feature_map "softmax") or lizard_attn_fwd_hedgehog
    ("hedgehog"): gradients of a loss with dL/dy = dy [B,Hq,L,d].  Returns a dict: dq, dk, dv,
    dlg in the input dtype; dwq, dwk (shaped like w_phi_q / w_phi_k; kept apart even when one
    matrix serves both sides), dtk, dtv ([Hkv,M,d]) in fp32."""
    if feature_map not in ("softmax", "hedgehog"):
        raise ValueError(f"unknown feature map {feature_map!r}")
    hh = feature_map == "hedgehog"
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"),
                 (w_phi_k, "w_phi_k"), (dy, "dy")):
        _dev(t, n, dt)
    if M > 0:
        _dev(t_k, "t_k", dt)
        _dev(t_v, "t_v", dt)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or v.shape != k.shape or log_gamma.shape != k.shape:
        raise ValueError("k, v, log_gamma must be [B,Hkv,L,d] matching q")
    if dy.shape != q.shape:
        raise ValueError("dy must have the shape of q")
    if M > 0 and (t_k.shape != (Hkv, M, d) or t_v.shape != (Hkv, M, d)):
        raise ValueError("t_k, t_v must be [Hkv,M,d]")
    _same_device(q.device, (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi_q, "w_phi_q"),
                 (w_phi_k, "w_phi_k"), (dy, "dy"), (t_k if M > 0 else None, "t_k"),
                 (t_v if M > 0 else None, "t_v"))
    cols = d // 2 if hh else d
    wstride = _w_stride(w_phi_q, w_phi_k, d, Hq, Hkv, cols)
    if scale is None:
        scale = d ** -0.5
    dev = q.device
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dlg": torch.empty_like(log_gamma),
           "dwq": torch.empty(w_phi_q.shape, dtype=torch.float32, device=dev),
           "dwk": torch.empty(w_phi_k.shape, dtype=torch.float32, device=dev),
           "dtk": torch.empty((Hkv, M, d), dtype=torch.float32, device=dev),
           "dtv": torch.empty((Hkv, M, d), dtype=torch.float32, device=dev)}
    need = lizard_attn_bwd_workspace_bytes(B, Hq, Hkv, L, d, M, dt)
    workspace = _workspace(workspace, need, dev)
    wbytes = 0 if workspace is None else workspace.numel()
    fn = load().lizard_attn_bwd_hedgehog if hh else load().lizard_attn_bwd
    _check(fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(w_phi_q), _ptr(w_phi_k), wstride,
        _ptr(t_k) if M > 0 else None, _ptr(t_v) if M > 0 else None, _ptr(dy),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlg"]), _ptr(out["dwq"]),
        _ptr(out["dwk"]), _ptr(out["dtk"]) if M > 0 else None, _ptr(out["dtv"]) if M > 0 else None,
        B, Hq, Hkv, L, d, W, M, float(mix), float(scale), _DTYPES[dt], _ptr(workspace), wbytes,
        _stream(stream)))
    return out


GLA_MODES = {"standard": 0, "reparam": 1}


def lizard_gla_fwd(q, k, v, log_gamma, w_phi, *, mode: str = "standard", out=None, stream=None):
    """The gated-linear-attention branch alone (lizard_attn_fwd's output at mix = 1): q
    [B,Hq,L,d]; k, v, log_gamma [B,Hkv,L,d]; w_phi [d,d] shared by queries, keys and heads.
    mode "standard": secondary chunking with fp32 diagonal blocks; "reparam": the whole
    intra-chunk product on matrix cores.  bf16, d = 128."""
    if mode not in GLA_MODES:
        raise ValueError(f"mode must be one of {sorted(GLA_MODES)}")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi, "w_phi")):
        _dev(t, n, dt)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or v.shape != k.shape or log_gamma.shape != k.shape:
        raise ValueError("k, v, log_gamma must be [B,Hkv,L,d] matching q")
    if w_phi.shape != (d, d):
        raise ValueError(f"w_phi must be [{d},{d}]")
    _same_device(q.device, (k, "k"), (v, "v"), (log_gamma, "log_gamma"), (w_phi, "w_phi"))
    out = _out(out, q)
    _check(load().lizard_gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(w_phi), _ptr(out),
                                 B, Hq, Hkv, L, d, GLA_MODES[mode], _DTYPES[dt], _stream(stream)))
    return out


def version() -> str:
    return load().lizard_version().decode()
