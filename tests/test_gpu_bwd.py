"""Parity of the HIP backward pass (lizard_attn_bwd / lizard_attn_bwd_hedgehog) with the fp64
oracle's backward (oracle.lizard_bwd, itself pinned by finite differences and autograd).

Relative L2 of every gradient: dq per (batch, query head), dk / dv / dlog_gamma per (batch,
key/value head) over L x d, dW_phi over the whole matrix, dT per key/value head; <= 2e-2 for bf16
inputs and <= 1e-4 for fp32 (the benchmark spec's tolerances of the forward)."""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd import api
from linearized_attention_amd.synthetic import WORKLOADS, make_fwd_inputs

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(got, want, axes, floor=1e-300):
    num = np.sqrt(((got - want) ** 2).sum(axis=axes))
    den = np.sqrt((want ** 2).sum(axis=axes))
    return num / np.maximum(den, floor)


def dlg_floor(want):
    """Denominator floor for the log-gate gradient: 1e-3 of the RMS of the key-side gradient.
    With gamma = 0 the exact log-gate gradient is 0 (the gate multiplies every term) and only
    an absolute bound is meaningful; elsewhere the floor is far below the gradient's size."""
    return 1e-3 * np.sqrt((want["dk"] ** 2).mean()) * np.sqrt(want["dlg"][0, 0].size)


def check_bwd(label, inp, dtype, mix=0.5, fmap="softmax", heads=None):
    """heads: None (compare everything) or a list of (b, hq) pairs for sampled comparison."""
    _say(f"[bwd] {label}: q{tuple(inp.q.shape)} k{tuple(inp.k.shape)} W={inp.W} M={inp.M} {fmap}")
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    dy = torch.tensor(rng.standard_normal(inp.q.shape)).to(DT[dtype])
    dev = inp.to("cuda")
    g = api.lizard_attn_bwd(dev.q, dev.k, dev.v, dev.log_gamma, dev.w_phi_q, dev.w_phi_k, dev.t_k, dev.t_v,
                            dy.cuda(), W=inp.W, M=inp.M, mix=mix, scale=inp.scale, feature_map=fmap)
    torch.cuda.synchronize()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    for k, v in got.items():
        assert np.isfinite(v).all(), f"{label}: non-finite {k}"
    errs = {}
    if heads is None:
        want = oracle.lizard_bwd(*inp.tensors(), dy, W=inp.W, M=inp.M, mix=mix, scale=inp.scale, feature_map=fmap)
        for k in ("dq", "dk", "dv"):
            errs[k] = float(rel(got[k], want[k], (-2, -1)).max())
        errs["dlg"] = float(rel(got["dlg"], want["dlg"], (-2, -1), dlg_floor(want)).max())
        for k in ("dwq", "dwk"):
            errs[k] = float(rel(got[k].reshape(1, -1), want[k].reshape(1, -1), (-1,)).max())
        if inp.M > 0:
            for k in ("dtk", "dtv"):
                errs[k] = float(rel(got[k], want[k], (-2, -1)).max())
    else:
        G = inp.q.shape[1] // inp.k.shape[1]
        for (b, hq) in heads:
            hk = hq // G
            sl = lambda t, h: t[b:b + 1, h:h + 1]
            wq = inp.w_phi_q if inp.w_phi_q.dim() == 2 else inp.w_phi_q[hq:hq + 1]
            wk = inp.w_phi_k if inp.w_phi_k.dim() == 2 else inp.w_phi_k[hk:hk + 1]
            want = oracle.lizard_bwd(sl(inp.q, hq), sl(inp.k, hk), sl(inp.v, hk), sl(inp.log_gamma, hk), wq, wk,
                                     inp.t_k[hk:hk + 1], inp.t_v[hk:hk + 1], sl(dy, hq), W=inp.W, M=inp.M,
                                     mix=mix, scale=inp.scale, feature_map=fmap)
            errs[f"dq[{b},{hq}]"] = float(rel(got["dq"][b, hq], want["dq"][0, 0], (-2, -1)))
            if G == 1:
                for k in ("dk", "dv"):
                    errs[f"{k}[{b},{hk}]"] = float(rel(got[k][b, hk], want[k][0, 0], (-2, -1)))
                errs[f"dlg[{b},{hk}]"] = float(rel(got["dlg"][b, hk], want["dlg"][0, 0], (-2, -1),
                                                   dlg_floor(want)))
    _say(f"      rel-L2: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL[dtype], f"{label}: {k} rel L2 {e:.3e} > {TOL[dtype]}"


CASES = [
    ("fp32 d64 L256 W64 M4 (tiny workload)", dict(B=1, Hq=2, Hkv=2, L=256, d=64, W=64, M=4), "f32", "softmax", 0.5),
    ("fp32 d64 gqa 4:2 ragged L77 W20 M3 per-head W", dict(B=2, Hq=4, Hkv=2, L=77, d=64, W=20, M=3, per_head_w=True),
     "f32", "softmax", 0.3),
    ("bf16 d128 ragged L200 W64 M4", dict(B=2, Hq=2, Hkv=2, L=200, d=128, W=64, M=4), "bf16", "softmax", 0.5),
    ("bf16 d128 gqa 4:2 L300 separate W_k", dict(B=1, Hq=4, Hkv=2, L=300, d=128, W=64, M=4, separate_wk=True),
     "bf16", "softmax", 0.5),
    ("bf16 d128 per-head W L150", dict(B=1, Hq=2, Hkv=2, L=150, d=128, W=40, M=2, per_head_w=True), "bf16",
     "softmax", 0.7),
    ("bf16 d128 uniform gate U[-5,0) W128 M8", dict(B=1, Hq=2, Hkv=2, L=260, d=128, W=128, M=8, gate="uniform"),
     "bf16", "softmax", 0.5),
    ("bf16 d128 gamma=0 (exact steps)", dict(B=1, Hq=2, Hkv=1, L=100, d=128, W=64, M=4, gate="zero"), "bf16",
     "softmax", 0.5),
    ("bf16 d128 gamma=1", dict(B=1, Hq=2, Hkv=2, L=150, d=128, W=64, M=4, gate="one"), "bf16", "softmax", 0.5),
    ("bf16 d128 mixed steps uniform:-1.6", dict(B=1, Hq=2, Hkv=2, L=180, d=128, W=65, M=16, gate="uniform:-1.6"),
     "bf16", "softmax", 0.5),
    ("bf16 d64 W1 M0", dict(B=1, Hq=2, Hkv=2, L=70, d=64, W=1, M=0), "bf16", "softmax", 0.5),
    ("bf16 d128 W>=L M0 mix1", dict(B=1, Hq=2, Hkv=2, L=120, d=128, W=200, M=0), "bf16", "softmax", 1.0),
    ("bf16 d128 mix0 (window only)", dict(B=1, Hq=2, Hkv=2, L=90, d=128, W=30, M=4), "bf16", "softmax", 0.0),
    ("hedgehog bf16 d128 gqa 2:1 L200", dict(B=1, Hq=2, Hkv=1, L=200, d=128, W=64, M=4, phi_cols=64), "bf16",
     "hedgehog", 0.5),
    ("hedgehog fp32 d64 per-head L90", dict(B=1, Hq=2, Hkv=2, L=90, d=64, W=20, M=2, phi_cols=32, per_head_w=True),
     "f32", "hedgehog", 0.6),
]


@pytest.mark.parametrize("label,kw,dtype,fmap,mix", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(gpu_lib, label, kw, dtype, fmap, mix):
    inp = make_fwd_inputs(dtype=dtype, seed=zlib.crc32(label.encode()) % 10000, **kw)
    check_bwd(label, inp, dtype, mix=mix, fmap=fmap)


def test_bwd_full_size_sampled_heads(gpu_lib):
    """The 4 x 32 x 4096 layer shape (bf16, d = 128, W = 64, M = 4): every head's gradients on the
    GPU, the oracle on sampled (batch, head) pairs (dq, dk, dv, dlog_gamma of those heads)."""
    c = WORKLOADS[1]
    inp = make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"], M=c["M"],
                          dtype="bf16", seed=3001)
    check_bwd("full size 4x32x4096", inp, "bf16", heads=[(0, 0), (3, 31)])


def test_bwd_is_deterministic(gpu_lib):
    inp = make_fwd_inputs(B=1, Hq=4, Hkv=2, L=260, d=128, W=64, M=4, dtype="bf16", seed=44)
    dev = inp.to("cuda")
    dy = torch.randn(inp.q.shape, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).cuda()
    a = api.lizard_attn_bwd(dev.q, dev.k, dev.v, dev.log_gamma, dev.w_phi_q, dev.w_phi_k, dev.t_k, dev.t_v, dy,
                            W=inp.W, M=inp.M, scale=inp.scale)
    b = api.lizard_attn_bwd(dev.q, dev.k, dev.v, dev.log_gamma, dev.w_phi_q, dev.w_phi_k, dev.t_k, dev.t_v, dy,
                            W=inp.W, M=inp.M, scale=inp.scale)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), f"{k} differs between two identical calls"
