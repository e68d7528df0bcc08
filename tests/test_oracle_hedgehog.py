"""Pins for the oracle's Hedgehog feature map, phi(x) = exp(xW) (+) exp(-xW).

The map is the Lizard paper's own (arXiv page, Method section, the hardware-efficient
reparameterization paragraph): the two halves are concatenated, the first holds exp(xW),
and there is no normalisation.  The recurrence around it is the one pinned in
test_oracle_pins.py.  None of these re-types the oracle's loop:

* the feature products are cosh sums: phi(q).phi(k) = sum_j 2 cosh((qW_q)_j + (kW_k)_j),
  so with gamma = 1 the global branch is a causal kernel sum with that kernel;
* W = 0 gives phi = 1 in every feature, and a constant scalar gate a geometric closed form;
* flipping the signs of q and k swaps the two halves, so permuting the gate's halves
  with them leaves the whole output unchanged;
* a gate of one on the first half and zero on the second separates the halves, which
  fixes their order against the gate's feature dimensions;
* the decode step from an empty state reproduces the forward.
"""
import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd.synthetic import make_decode_inputs, make_fwd_inputs

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _draw(seed, B=1, Hq=2, Hkv=2, L=13, d=6, cols=5, M=2, per_head=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    wq = rng.standard_normal((Hq, d, cols) if per_head else (d, cols)) / np.sqrt(d)
    wk = rng.standard_normal((Hkv, d, cols) if per_head else (d, cols)) / np.sqrt(d)
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    tk = rng.standard_normal((Hkv, M, d))
    tv = rng.standard_normal((Hkv, M, d))
    return q, k, v, wq, wk, tk, tv


def _run(q, k, v, lg, wq, wk, tk, tv, W=4, M=2, mix=0.5, scale=0.4, **kw):
    return oracle.lizard_fwd(q, k, v, lg, wq, wk, tk, tv, W=W, M=M, mix=mix, scale=scale,
                             return_branches=True, feature_map="hedgehog", **kw)


@pytest.mark.parametrize("per_head", [False, True])
def test_gamma_one_is_a_causal_cosh_kernel_sum(per_head):
    """gamma = 1: y_i = sum_{s<=i} [sum_j 2 cosh(a_ij + b_sj)] v_s, a = q W_q, b = k W_k."""
    B, Hq, Hkv, L, d, cols = 2, 4, 2, 11, 6, 5
    q, k, v, wq, wk, tk, tv = _draw(3, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, cols=cols, per_head=per_head)
    lg = np.zeros((B, Hkv, L, 2 * cols))
    _, yg, _ = _run(q, k, v, lg, wq, wk, tk, tv)
    G = Hq // Hkv
    want = np.zeros((B, Hq, L, d))
    for h in range(Hq):
        hk = h // G
        a = q[:, h] @ (wq[h] if per_head else wq)            # [B, L, cols]
        b = k[:, hk] @ (wk[hk] if per_head else wk)
        kern = 2.0 * np.cosh(a[:, :, None, :] + b[:, None, :, :]).sum(-1)  # [B, i, s]
        kern = np.tril(kern)
        want[:, h] = kern @ v[:, hk]
    np.testing.assert_allclose(yg, want, rtol=1e-12, atol=1e-12)


def test_zero_weights_give_unit_features_and_a_geometric_gate():
    """W = 0: phi = 1 in all df features; gamma_i = lam in every dimension gives
    y_i = df sum_{s<=i} lam^(i-s) v_s."""
    B, H, L, d, cols = 1, 2, 17, 6, 4
    q, k, v, _, _, tk, tv = _draw(5, B=B, Hq=H, Hkv=H, L=L, d=d, cols=cols)
    w0 = np.zeros((d, cols))
    lam_log = -0.25
    lg = np.full((B, H, L, 2 * cols), lam_log)
    _, yg, _ = _run(q, k, v, lg, w0, w0, tk, tv)
    i = np.arange(L)[:, None]
    s = np.arange(L)[None, :]
    decay = np.where(s <= i, np.exp(lam_log) ** np.maximum(i - s, 0), 0.0)
    want = 2 * cols * (decay @ v)
    np.testing.assert_allclose(yg, want, rtol=1e-12, atol=1e-12)


def test_sign_flip_swaps_the_halves():
    """phi(-x) is phi(x) with its halves swapped; with the gate's halves swapped too the
    whole output (both branches: the window sees (-q).(-k) = q.k) is unchanged."""
    B, H, L, d, cols = 2, 2, 19, 6, 5
    q, k, v, wq, wk, tk, tv = _draw(9, B=B, Hq=H, Hkv=H, L=L, d=d, cols=cols)
    rng = np.random.Generator(np.random.PCG64(10))
    lg = rng.uniform(-1.5, -1e-3, size=(B, H, L, 2 * cols))
    swap = np.concatenate([np.arange(cols, 2 * cols), np.arange(cols)])
    y0, yg0, yw0 = _run(q, k, v, lg, wq, wk, tk, tv)
    y1, yg1, yw1 = _run(-q, -k, v, lg[..., swap], wq, wk, -tk, tv)
    np.testing.assert_allclose(yg1, yg0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(yw1, yw0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12)


def test_gate_halves_fix_the_order_of_the_halves():
    """gamma = 1 on features 0..c-1 and 0 on c..2c-1: the first half (exp(+xW)) sums over
    all earlier tokens, the second (exp(-xW)) keeps only the current one:
    y_i = sum_{s<=i} sum_j e^{a_ij + b_sj} v_s + sum_j e^{-a_ij - b_ij} v_i."""
    B, H, L, d, cols = 1, 2, 15, 6, 5
    q, k, v, wq, wk, tk, tv = _draw(13, B=B, Hq=H, Hkv=H, L=L, d=d, cols=cols)
    lg = np.concatenate([np.zeros((B, H, L, cols)), np.full((B, H, L, cols), -1e4)], axis=-1)
    _, yg, _ = _run(q, k, v, lg, wq, wk, tk, tv)
    a = q @ wq
    b = k @ wk
    plus = np.tril(np.exp(a[:, :, :, None, :] + b[:, :, None, :, :]).sum(-1))   # [B,H,i,s]
    minus = np.exp(-a - b).sum(-1, keepdims=True)                               # [B,H,i,1]
    want = plus @ v + minus * v
    np.testing.assert_allclose(yg, want, rtol=1e-12, atol=1e-12)


def test_window_branch_does_not_depend_on_the_feature_map():
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=30, d=8, W=5, M=3, dtype="f32", seed=4, phi_cols=4)
    args = dict(W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale, return_branches=True)
    _, _, yw_h = oracle.lizard_fwd(*inp.tensors(), feature_map="hedgehog", **args)
    w_full = torch.zeros(8, 8, dtype=inp.w_phi_q.dtype)
    _, _, yw_s = oracle.lizard_fwd(inp.q, inp.k, inp.v, inp.log_gamma, w_full, w_full, inp.t_k,
                                   inp.t_v, feature_map="softmax", **args)
    np.testing.assert_array_equal(yw_h, yw_s)


def test_rejects_mismatched_weight_shapes():
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=8, d=8, W=4, M=1, dtype="f32", seed=1)
    with pytest.raises(ValueError):  # [d, d] weights would give 2d features, log gamma has d
        oracle.lizard_fwd(*inp.tensors(), W=4, M=1, mix=0.5, scale=0.3, feature_map="hedgehog")


def test_decode_from_empty_equals_forward():
    L, d, W, M = 21, 8, 5, 2
    dec = make_decode_inputs(N=3, Hq=4, Hkv=2, d=d, W=W, M=M, steps=L, pos0=0, dtype="f32",
                             seed=12, zero_state=True, gate="uniform", phi_cols=d // 2)
    st, rk, rv, pos = dec.state, dec.ring_k, dec.ring_v, dec.pos
    outs = []
    for (q, k, v, lg) in dec.steps:
        out, st, rk, rv, pos = oracle.lizard_decode(st, rk, rv, pos, q, k, v, lg, dec.w_phi_q,
                                                    dec.w_phi_k, dec.t_k, dec.t_v, M=M,
                                                    mix=dec.mix, scale=dec.scale,
                                                    feature_map="hedgehog")
        outs.append(out)
    ydec = np.stack(outs, axis=2)
    stack = lambda i: torch.stack([s[i] for s in dec.steps], dim=2)
    yf, sf = oracle.lizard_fwd(stack(0), stack(1), stack(2), stack(3), dec.w_phi_q, dec.w_phi_k,
                               dec.t_k, dec.t_v, W=W, M=M, mix=dec.mix, scale=dec.scale,
                               return_state=True, feature_map="hedgehog")
    np.testing.assert_allclose(ydec, yf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, sf, rtol=1e-12, atol=1e-12)
