"""Seeded synthetic inputs for Lizard attention.

This module is shared by the tests, the benchmark and the smoke check.  It
holds only input recipes -- random draws, the caller-side gate projection
that turns gate activations into log gamma, and rounding to the storage dtype
-- and none of the attention arithmetic itself.  Both the HIP path and the
fp64 oracle receive the very same arrays.

Recipe (all draws in float64 from ``numpy.random.Generator(PCG64(seed))``,
then rounded to nearest-even into the storage dtype):

* draw order: W_phi, W_gamma, x_gate, q, k, v, T_k, T_v (then state, ring for
  decode); the uniform-gate workload draws log gamma in place of W_gamma/x_gate;
* ``N(0, s)`` takes ``s`` as the variance: W_phi, W_gamma ~ N(0, 1/d),
  q, k, v, x_gate, T ~ N(0, 1), decode state ~ N(0, 0.1), ring ~ N(0, 1);
* log gamma = logsigmoid(x_gate @ W_gamma) / 16 per key dimension (the gate is
  computed by the caller, outside the attention op), or U[-5, -1e-4] i.i.d.
  for the long-context stress workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# The five workloads.  Index 0 is the small fp32 case, 1 the Llama-3-8B-shaped
# layer (the benchmark's forward workload), 2 the 32K stress, 3 decode, 4 GQA.
WORKLOADS = {
    0: dict(kind="fwd", dtype="f32", B=1, Hq=2, Hkv=2, L=256, d=64, W=64, M=4, gate="logsigmoid"),
    1: dict(kind="fwd", dtype="bf16", B=4, Hq=32, Hkv=32, L=4096, d=128, W=64, M=4, gate="logsigmoid"),
    2: dict(kind="fwd", dtype="bf16", B=1, Hq=32, Hkv=32, L=32768, d=128, W=128, M=8, gate="uniform"),
    3: dict(kind="decode", dtype="bf16", N=256, Hq=32, Hkv=32, d=128, W=64, M=4, steps=128, pos0=4096,
            gate="logsigmoid"),
    4: dict(kind="fwd", dtype="bf16", B=2, Hq=32, Hkv=8, L=8192, d=128, W=64, M=4, gate="logsigmoid"),
}

WORKLOAD_NAMES = {
    0: "tiny fp32 fwd B1 H2 L256 d64 W64 M4",
    1: "llama3-8b-layer fwd bf16 B4 H32 L4096 d128 W64 M4",
    2: "long-context stress fwd bf16 B1 H32 L32768 d128 W128 M8 uniform-gate",
    3: "decode bf16 N256 H32 d128 W64 M4 fp32-state 128 steps",
    4: "gqa fwd bf16 B2 Hq32 Hkv8 L8192 d128 W64 M4",
}

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp64 array -> CPU tensor in the storage dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPES[dtype])


def _normal(rng: np.random.Generator, shape, var: float = 1.0) -> np.ndarray:
    return rng.standard_normal(shape) * math.sqrt(var)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    # log(1 / (1 + e^-x)) = -softplus(-x), written stably
    return -(np.maximum(-x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def gate_from_activations(x_gate: np.ndarray, w_gamma: np.ndarray) -> np.ndarray:
    """Caller-side gate: log gamma = logsigmoid(x_gate @ W_gamma) / 16."""
    return _logsigmoid(x_gate @ w_gamma) / 16.0


@dataclass
class FwdInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    log_gamma: torch.Tensor
    w_phi_q: torch.Tensor
    w_phi_k: torch.Tensor
    t_k: torch.Tensor
    t_v: torch.Tensor
    W: int
    M: int
    mix: float
    scale: float
    extra: dict = field(default_factory=dict)

    def tensors(self):
        return (self.q, self.k, self.v, self.log_gamma, self.w_phi_q, self.w_phi_k,
                self.t_k, self.t_v)

    def to(self, device) -> "FwdInputs":
        """Copy to `device`; a W_phi shared by both sides stays one tensor."""
        moved = [t.to(device) for t in self.tensors()]
        if self.w_phi_k is self.w_phi_q:
            moved[5] = moved[4]
        return FwdInputs(*moved, W=self.W, M=self.M, mix=self.mix, scale=self.scale, extra=self.extra)


def make_fwd_inputs(*, B: int, Hq: int, Hkv: int, L: int, d: int, W: int, M: int,
                    dtype: str = "bf16", seed: int = 0, gate: str = "logsigmoid",
                    mix: float = 0.5, scale: float | None = None,
                    per_head_w: bool = False, separate_wk: bool = False,
                    q_var: float = 1.0, k_var: float = 1.0,
                    phi_cols: int | None = None) -> FwdInputs:
    """Draw one forward problem.

    gate: "logsigmoid" (config recipe), "uniform" (U[-5,-1e-4]), "one"
    (log gamma = 0), "zero" (log gamma = -1e4, i.e. gamma = 0 to fp precision),
    "const:<x>" (every entry equal to x), or "uniform:<lo>" (U[lo, -1e-4]).
    per_head_w: one W_phi per head ([Hq,d,d] / [Hkv,d,d]) instead of a shared one.
    separate_wk: draw an independent key-side W_phi (otherwise W_phi_k = W_phi_q).
    phi_cols: columns of W_phi (default d).  The Hedgehog map exp(xW) (+) exp(-xW)
    takes d // 2 columns, so that its feature dimension is d again.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cols = d if phi_cols is None else phi_cols
    wshape = (Hq, d, cols) if per_head_w else (d, cols)
    w_phi = _normal(rng, wshape, 1.0 / d)
    kshape = (B, Hkv, L, d)
    if gate == "logsigmoid":
        w_gamma = _normal(rng, (d, d), 1.0 / d)
        x_gate = _normal(rng, kshape)
        lg = gate_from_activations(x_gate, w_gamma)
    elif gate.startswith("uniform"):
        lo = float(gate.split(":")[1]) if ":" in gate else -5.0
        lg = rng.uniform(lo, -1e-4, size=kshape)
    elif gate == "one":
        lg = np.zeros(kshape)
    elif gate == "zero":
        lg = np.full(kshape, -1e4)
    elif gate.startswith("const:"):
        lg = np.full(kshape, float(gate.split(":")[1]))
    else:
        raise ValueError(f"unknown gate recipe {gate!r}")
    q = _normal(rng, (B, Hq, L, d), q_var)
    k = _normal(rng, kshape, k_var)
    v = _normal(rng, kshape)
    tk = _normal(rng, (Hkv, M, d))
    tv = _normal(rng, (Hkv, M, d))
    if separate_wk:
        wk = _normal(rng, (Hkv, d, cols) if per_head_w else (d, cols), 1.0 / d)
    elif per_head_w:
        G = Hq // Hkv
        wk = w_phi[::G].copy()
    else:
        wk = None
    wq_t = _round(w_phi, dtype)
    wk_t = wq_t if wk is None else _round(wk, dtype)
    return FwdInputs(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
                     log_gamma=_round(lg, dtype), w_phi_q=wq_t, w_phi_k=wk_t,
                     t_k=_round(tk, dtype), t_v=_round(tv, dtype), W=W, M=M, mix=mix,
                     scale=(1.0 / math.sqrt(d)) if scale is None else scale)


def workload_fwd_inputs(index: int) -> FwdInputs:
    """The seeded inputs of forward workload ``index`` (seed 1000 + index)."""
    c = WORKLOADS[index]
    if c["kind"] != "fwd":
        raise ValueError(f"workload {index} is not a forward workload")
    return make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"],
                           M=c["M"], dtype=c["dtype"], seed=1000 + index, gate=c["gate"])


@dataclass
class DecodeInputs:
    state: torch.Tensor        # [N,Hkv,d,d] fp32
    ring_k: torch.Tensor       # [N,Hkv,W,d]
    ring_v: torch.Tensor
    pos: torch.Tensor          # [N] int32
    w_phi_q: torch.Tensor
    w_phi_k: torch.Tensor
    t_k: torch.Tensor
    t_v: torch.Tensor
    steps: list                # per step: (q [N,Hq,d], k, v, log_gamma [N,Hkv,d])
    M: int
    mix: float
    scale: float


def make_decode_inputs(*, N: int, Hq: int, Hkv: int, d: int, W: int, M: int, steps: int,
                       pos0: int, dtype: str = "bf16", seed: int = 0,
                       state_var: float = 0.1, zero_state: bool = False,
                       mix: float = 0.5, gate: str = "logsigmoid",
                       phi_cols: int | None = None) -> DecodeInputs:
    """Draw one decode problem (phi_cols as in make_fwd_inputs)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w_phi = _normal(rng, (d, d if phi_cols is None else phi_cols), 1.0 / d)
    w_gamma = _normal(rng, (d, d), 1.0 / d)
    tk = _normal(rng, (Hkv, M, d))
    tv = _normal(rng, (Hkv, M, d))
    if zero_state:
        state = np.zeros((N, Hkv, d, d))
        ring_k = np.zeros((N, Hkv, W, d))
        ring_v = np.zeros((N, Hkv, W, d))
    else:
        state = _normal(rng, (N, Hkv, d, d), state_var)
        ring_k = _normal(rng, (N, Hkv, W, d))
        ring_v = _normal(rng, (N, Hkv, W, d))
    seq = []
    for _ in range(steps):
        if gate == "logsigmoid":
            x_gate = _normal(rng, (N, Hkv, d))
            lg = gate_from_activations(x_gate, w_gamma)
        elif gate.startswith("uniform"):
            lg = rng.uniform(-5.0, -1e-4, size=(N, Hkv, d))
        else:
            raise ValueError(gate)
        q = _normal(rng, (N, Hq, d))
        k = _normal(rng, (N, Hkv, d))
        v = _normal(rng, (N, Hkv, d))
        seq.append((_round(q, dtype), _round(k, dtype), _round(v, dtype), _round(lg, dtype)))
    w_t = _round(w_phi, dtype)
    return DecodeInputs(state=torch.from_numpy(state).to(torch.float32),
                        ring_k=_round(ring_k, dtype), ring_v=_round(ring_v, dtype),
                        pos=torch.full((N,), pos0, dtype=torch.int32), w_phi_q=w_t, w_phi_k=w_t,
                        t_k=_round(tk, dtype), t_v=_round(tv, dtype), steps=seq, M=M, mix=mix,
                        scale=1.0 / math.sqrt(d))


def workload_decode_inputs(index: int = 3, steps: int | None = None, N: int | None = None) -> DecodeInputs:
    c = WORKLOADS[index]
    return make_decode_inputs(N=c["N"] if N is None else N, Hq=c["Hq"], Hkv=c["Hkv"], d=c["d"],
                              W=c["W"], M=c["M"], steps=c["steps"] if steps is None else steps,
                              pos0=c["pos0"], dtype=c["dtype"], seed=1000 + index)
