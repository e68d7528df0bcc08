"""fp64 CPU oracle for Lizard attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it, and it shares no code with them.

The arithmetic lives in ``lizard_oracle.c`` (the literal recurrence and a
brute-force window softmax in double precision); this module only converts
arrays to float64, calls it through ctypes, and converts results back.

Pinned by ``tests/test_oracle_pins.py`` against closed forms, library routines
(torch's fp64 scaled-dot-product attention, cumulative sums) and brute force
on tiny inputs.  See the header of ``lizard_oracle.c`` for which passage of
the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lizard_oracle.c")
_SO = os.path.join(_HERE, "liblizard_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_SO)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int32)
            i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.oracle_lizard_fwd.argtypes = [dp, dp, dp, dp, dp, dp, i64, dp, dp,
                                              i32, i32, i32, i32, i32, i32, i32, i32,
                                              f64, f64, i32, dp, dp, dp, dp]
            lib.oracle_lizard_fwd.restype = i32
            lib.oracle_lizard_decode.argtypes = [dp, dp, dp, ip, dp, dp, dp, dp, dp, dp,
                                                 i64, dp, dp, i32, i32, i32, i32, i32,
                                                 i32, i32, f64, f64, i32, dp, dp, dp]
            lib.oracle_lizard_decode.restype = i32
            lib.oracle_lizard_bwd.argtypes = [dp, dp, dp, dp, dp, dp, i64, dp, dp, dp,
                                              i32, i32, i32, i32, i32, i32, i32, i32,
                                              f64, f64, i32, dp, dp, dp, dp, dp, dp, dp, dp]
            lib.oracle_lizard_bwd.restype = i32
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = i32
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """float64 C-contiguous copy; torch tensors (any dtype, any device) accepted.

    bf16 and fp32 values convert to float64 exactly."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


_FMAPS = {"softmax": 0, "hedgehog": 1}


def _fmap_code(feature_map: str) -> int:
    if feature_map not in _FMAPS:
        raise ValueError(f"unknown feature map {feature_map!r}")
    return _FMAPS[feature_map]


def lizard_fwd(q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, *, W: int, M: int,
               mix: float, scale: float, w_shared: bool | None = None,
               return_branches: bool = False, return_state: bool = False,
               feature_map: str = "softmax"):
    """Lizard attention forward in fp64.

    q [B,Hq,L,d]; k, v [B,Hkv,L,d]; log_gamma [B,Hkv,L,df];
    w_phi_q, w_phi_k: [d,c] shared by all heads, or [Hq,d,c] / [Hkv,d,c], with
    c = df for feature_map "softmax" and c = df/2 for "hedgehog"
    (phi(x) = exp(xW) concatenated with exp(-xW));
    t_k, t_v [Hkv,M,d].  Returns y [B,Hq,L,d] (float64), plus (y_gla, y_win)
    and/or the final state [B,Hkv,df,d] when asked.
    """
    fm = _fmap_code(feature_map)
    q, k, v, lg = _f64(q), _f64(k), _f64(v), _f64(log_gamma)
    wq, wk = _f64(w_phi_q), _f64(w_phi_k)
    tk, tv = _f64(t_k), _f64(t_v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    df = lg.shape[-1]
    cols = df // 2 if fm == 1 else df
    if wq.shape[-2:] != (d, cols) or wk.shape[-2:] != (d, cols):
        raise ValueError(f"W_phi must end in [{d},{cols}] for this feature map")
    if wq.ndim == 2:
        stride = 0
        if wk.ndim != 2:
            raise ValueError("w_phi_q and w_phi_k must both be shared or both per head")
    else:
        if wq.shape[0] != Hq or wk.shape[0] != Hkv:
            raise ValueError("per-head W_phi must be [Hq,d,c] and [Hkv,d,c]")
        stride = d * cols
    if M == 0:
        tk = np.zeros((Hkv, 1, d))
        tv = np.zeros((Hkv, 1, d))
    y = np.zeros((B, Hq, L, d))
    yg = np.zeros_like(y) if return_branches else None
    yw = np.zeros_like(y) if return_branches else None
    st = np.zeros((B, Hkv, df, d)) if return_state else None
    nul = ctypes.POINTER(ctypes.c_double)()
    rc = _load().oracle_lizard_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(lg), _ptr(wq), _ptr(wk), stride, _ptr(tk), _ptr(tv),
        B, Hq, Hkv, L, d, df, W, M, float(mix), float(scale), fm, _ptr(y),
        _ptr(yg) if yg is not None else nul, _ptr(yw) if yw is not None else nul,
        _ptr(st) if st is not None else nul)
    if rc != 0:
        raise ValueError("oracle_lizard_fwd rejected the shapes")
    out = [y]
    if return_branches:
        out += [yg, yw]
    if return_state:
        out.append(st)
    return out[0] if len(out) == 1 else tuple(out)


def lizard_decode(state, ring_k, ring_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k,
                  t_k, t_v, *, M: int, mix: float, scale: float,
                  return_branches: bool = False, feature_map: str = "softmax"):
    """One decode step in fp64.  Returns (out, state, ring_k, ring_v, pos) as new
    float64/int32 arrays (inputs are not modified), plus (y_gla, y_win) if asked.

    state [N,Hkv,df,d]; ring_k/ring_v [N,Hkv,W,d]; pos [N] (tokens seen so far);
    q [N,Hq,d]; k, v [N,Hkv,d]; log_gamma [N,Hkv,df]; W_phi and feature_map
    as in lizard_fwd."""
    fm = _fmap_code(feature_map)
    st, rk, rv = _f64(state).copy(), _f64(ring_k).copy(), _f64(ring_v).copy()
    try:
        import torch
        if isinstance(pos, torch.Tensor):
            pos = pos.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    ps = np.ascontiguousarray(np.asarray(pos, dtype=np.int32)).copy()
    q, k, v, lg = _f64(q), _f64(k), _f64(v), _f64(log_gamma)
    wq, wk, tk, tv = _f64(w_phi_q), _f64(w_phi_k), _f64(t_k), _f64(t_v)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    df = lg.shape[-1]
    W = rk.shape[2]
    cols = df // 2 if fm == 1 else df
    if wq.shape[-2:] != (d, cols) or wk.shape[-2:] != (d, cols):
        raise ValueError(f"W_phi must end in [{d},{cols}] for this feature map")
    stride = 0 if wq.ndim == 2 else d * cols
    if M == 0:
        tk = np.zeros((Hkv, 1, d))
        tv = np.zeros((Hkv, 1, d))
    out = np.zeros((N, Hq, d))
    yg = np.zeros_like(out) if return_branches else None
    yw = np.zeros_like(out) if return_branches else None
    nul = ctypes.POINTER(ctypes.c_double)()
    rc = _load().oracle_lizard_decode(
        _ptr(st), _ptr(rk), _ptr(rv), ps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        _ptr(q), _ptr(k), _ptr(v), _ptr(lg), _ptr(wq), _ptr(wk), stride, _ptr(tk), _ptr(tv),
        N, Hq, Hkv, d, df, W, M, float(mix), float(scale), fm, _ptr(out),
        _ptr(yg) if yg is not None else nul, _ptr(yw) if yw is not None else nul)
    if rc != 0:
        raise ValueError("oracle_lizard_decode rejected the shapes")
    res = (out, st, rk, rv, ps)
    if return_branches:
        res = res + (yg, yw)
    return res


def lizard_bwd(q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, dy, *, W: int, M: int,
               mix: float, scale: float, feature_map: str = "softmax"):
    """Gradients of sum(dy * y) through lizard_fwd, in fp64 (the chain rule through the
    literal recurrence and window softmax; see oracle_lizard_bwd in lizard_oracle.c).

    Same inputs as lizard_fwd plus dy [B,Hq,L,d].  Returns a dict of float64 arrays:
    dq, dk, dv, dlg (shapes of q, k, v, log_gamma), dwq, dwk (shapes of w_phi_q and
    w_phi_k; kept apart even when one matrix serves both sides: its gradient is then
    dwq + dwk), dtk, dtv (shapes of t_k, t_v; [Hkv,0,d] when M = 0).
    The forward states of one (batch, head) pair are all kept: L * df * d doubles per
    OpenMP thread."""
    fm = _fmap_code(feature_map)
    q, k, v, lg, dy = _f64(q), _f64(k), _f64(v), _f64(log_gamma), _f64(dy)
    wq, wk = _f64(w_phi_q), _f64(w_phi_k)
    tk, tv = _f64(t_k), _f64(t_v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    df = lg.shape[-1]
    cols = df // 2 if fm == 1 else df
    if wq.shape[-2:] != (d, cols) or wk.shape[-2:] != (d, cols):
        raise ValueError(f"W_phi must end in [{d},{cols}] for this feature map")
    if (wq.ndim == 2) != (wk.ndim == 2):
        raise ValueError("w_phi_q and w_phi_k must both be shared or both per head")
    if wq.ndim == 3 and (wq.shape[0] != Hq or wk.shape[0] != Hkv):
        raise ValueError("per-head W_phi must be [Hq,d,c] and [Hkv,d,c]")
    stride = 0 if wq.ndim == 2 else d * cols
    if dy.shape != q.shape:
        raise ValueError("dy must have the shape of q")
    Mc = max(M, 1)
    if M == 0:
        tk = np.zeros((Hkv, 1, d))
        tv = np.zeros((Hkv, 1, d))
    out = {"dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
           "dlg": np.zeros(lg.shape), "dwq": np.zeros(wq.shape), "dwk": np.zeros(wk.shape),
           "dtk": np.zeros((Hkv, Mc, d)), "dtv": np.zeros((Hkv, Mc, d))}
    rc = _load().oracle_lizard_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(lg), _ptr(wq), _ptr(wk), stride, _ptr(tk), _ptr(tv), _ptr(dy),
        B, Hq, Hkv, L, d, df, W, M, float(mix), float(scale), fm,
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlg"]), _ptr(out["dwq"]),
        _ptr(out["dwk"]), _ptr(out["dtk"]), _ptr(out["dtv"]))
    if rc != 0:
        raise ValueError("oracle_lizard_bwd rejected the shapes")
    out["dtk"] = out["dtk"][:, :M]
    out["dtv"] = out["dtv"][:, :M]
    return out
