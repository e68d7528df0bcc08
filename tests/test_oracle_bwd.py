"""Pins of the oracle's backward pass (oracle.lizard_bwd), on the CPU.

The backward oracle is the chain rule taken by hand through the literal
recurrence and window softmax.  It is pinned to things other than itself:

* central finite differences of the forward oracle, element by element, for every
  input (queries, keys, values, log gates, both feature-map matrices, meta keys and
  values), on tiny shapes: softmax and Hedgehog maps, grouped heads, per-head and
  shared W_phi, several gates, windows shorter and longer than the sequence,
  no meta tokens;
* torch autograd (fp64) of an independent formulation of the forward: the global
  branch as explicit decayed products over all (t, s) pairs from cumulative sums of
  the log gate (not the recurrence), the window as one masked softmax over
  [T_k ; K].
"""
import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd.synthetic import make_fwd_inputs

NAMES = ("dq", "dk", "dv", "dlg", "dwq", "dwk", "dtk", "dtv")


def _inputs(seed, B=1, Hq=2, Hkv=1, L=9, d=4, W=3, M=2, gate="logsigmoid", per_head=False,
            hedgehog=False):
    inp = make_fwd_inputs(B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, W=W, M=M, dtype="f32", seed=seed, gate=gate,
                          per_head_w=per_head, phi_cols=d // 2 if hedgehog else None)
    base = [oracle._f64(x).copy() for x in inp.tensors()]
    if not per_head:
        base[5] = base[5] + 0.1 * np.random.default_rng(seed).standard_normal(base[5].shape)  # separate W_phi_k
    return inp, base


def _loss(base, dy, W, M, mix, scale, fmap):
    y = oracle.lizard_fwd(*base, W=W, M=M, mix=mix, scale=scale, feature_map=fmap)
    return float((y * dy).sum())


FD_CASES = [
    ("softmax gqa 2:1 W3 M2 mix0.3", dict(Hq=2, Hkv=1, W=3, M=2), 0.3, "softmax"),
    ("softmax per-head W, W>=L, M0, mix0.7", dict(Hq=2, Hkv=2, W=20, M=0, per_head=True), 0.7, "softmax"),
    ("softmax uniform gate -2, W1, M1", dict(Hq=1, Hkv=1, W=1, M=1, gate="uniform:-2"), 0.5, "softmax"),
    ("softmax gamma=1, B2", dict(B=2, Hq=1, Hkv=1, W=4, M=2, gate="one"), 0.5, "softmax"),
    ("hedgehog gqa 2:1", dict(Hq=2, Hkv=1, W=3, M=2, hedgehog=True), 0.4, "hedgehog"),
    ("hedgehog per-head, W>=L", dict(Hq=2, Hkv=2, W=12, M=1, per_head=True, hedgehog=True), 1.0, "hedgehog"),
]


def check_fd(label, kw, mix, fmap, seed=5):
    inp, base = _inputs(seed, **kw)
    scale = 0.6
    dy = np.random.default_rng(seed + 1).standard_normal(base[0].shape)
    g = oracle.lizard_bwd(*base, dy, W=inp.W, M=inp.M, mix=mix, scale=scale, feature_map=fmap)
    h = 1e-6
    for ti, name in enumerate(NAMES):
        x = base[ti]
        got = g[name]
        if name in ("dtk", "dtv") and inp.M == 0:
            continue
        want = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(base, dy, inp.W, inp.M, mix, scale, fmap)
            x[idx] = old - h
            lm = _loss(base, dy, inp.W, inp.M, mix, scale, fmap)
            x[idx] = old
            want[idx] = (lp - lm) / (2 * h)
        err = np.abs(got - want).max()
        assert err <= 1e-6 * (1.0 + np.abs(want).max()), f"{label}: {name} off by {err:.3e} from finite differences"


@pytest.mark.parametrize("label,kw,mix,fmap", FD_CASES, ids=[c[0] for c in FD_CASES])
def test_bwd_matches_central_differences(label, kw, mix, fmap):
    check_fd(label, kw, mix, fmap)


def _torch_forward(t, W, M, mix, scale, fmap, G):
    """Independent fp64 formulation: explicit decayed products from cumulative log gates."""
    q, k, v, lg, wq, wk, tk, tv = t
    B, Hq, L, d = q.shape
    hk = torch.arange(Hq) // G
    kq, vq, lgq = k[:, hk], v[:, hk], lg[:, hk]
    wq_h = wq if wq.dim() == 3 else wq.expand(Hq, *wq.shape)
    wk_h = (wk if wk.dim() == 3 else wk.expand(k.shape[1], *wk.shape))[hk]

    def phi(x, w):
        z = torch.einsum("bhtd,hdc->bhtc", x, w)
        if fmap == "hedgehog":
            return torch.cat([torch.exp(z), torch.exp(-z)], dim=-1)
        return torch.softmax(z, dim=-1)

    pq, pk = phi(q, wq_h), phi(kq, wk_h)
    b = torch.cumsum(lgq, dim=2)                                  # [B,Hq,L,df]
    diff = b[:, :, :, None, :] - b[:, :, None, :, :]              # b_t - b_s
    causal = torch.tril(torch.ones(L, L, dtype=torch.bool))
    dec = torch.where(causal[None, None, :, :, None], torch.exp(torch.where(causal[None, None, :, :, None], diff, 0.0)), 0.0)
    a = torch.einsum("bhtf,bhsf,bhtsf->bhts", pq, pk, dec)
    y_gla = a @ vq
    keys = torch.cat([tk[hk][None].expand(B, -1, -1, -1), kq], dim=2)
    vals = torch.cat([tv[hk][None].expand(B, -1, -1, -1), vq], dim=2)
    logits = scale * q @ keys.transpose(-1, -2)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    band = (j <= i) & (j > i - W)
    mask = torch.cat([torch.ones(L, M, dtype=torch.bool), band], dim=1)
    p = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1)
    y_win = p @ vals
    return mix * y_gla + (1 - mix) * y_win


AG_CASES = [
    ("softmax gqa 4:2 W5 M3", dict(B=2, Hq=4, Hkv=2, L=40, d=8, W=5, M=3), 0.5, "softmax"),
    ("softmax per-head, uniform gate -1, W>=L", dict(B=1, Hq=2, Hkv=2, L=30, d=8, W=40, M=2, per_head=True,
                                                   gate="uniform:-1"), 0.3, "softmax"),
    ("hedgehog gqa 2:1 W7 M0", dict(B=1, Hq=2, Hkv=1, L=36, d=8, W=7, M=0, hedgehog=True), 0.8, "hedgehog"),
]


@pytest.mark.parametrize("label,kw,mix,fmap", AG_CASES, ids=[c[0] for c in AG_CASES])
def test_bwd_matches_autograd_of_explicit_products(label, kw, mix, fmap):
    inp, base = _inputs(11, **kw)
    scale = 0.4
    dy = np.random.default_rng(12).standard_normal(base[0].shape)
    g = oracle.lizard_bwd(*base, dy, W=inp.W, M=inp.M, mix=mix, scale=scale, feature_map=fmap)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in base]
    G = base[0].shape[1] // base[1].shape[1]
    y = _torch_forward(t, inp.W, inp.M, mix, scale, fmap, G)
    assert np.abs(y.detach().numpy() - oracle.lizard_fwd(*base, W=inp.W, M=inp.M, mix=mix, scale=scale,
                                                         feature_map=fmap)).max() < 1e-10
    (y * torch.tensor(dy)).sum().backward()
    for ti, name in enumerate(NAMES):
        if name in ("dtk", "dtv") and inp.M == 0:
            continue
        want = t[ti].grad.numpy()
        err = np.abs(g[name] - want).max()
        assert err <= 1e-9 * (1.0 + np.abs(want).max()), f"{label}: {name} off by {err:.3e} from autograd"
