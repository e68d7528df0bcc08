"""Pins for the fp64 oracle: closed forms, library routines, brute force.

None of these re-types the oracle's loop.  Each one states what the pages'
definitions fix in a different form, chosen so that a plausible mistake in the
oracle -- a dropped term, a gate applied after instead of before the update,
a gate on the wrong state dimension, an off-by-one window, a transposed
operand, the wrong softmax scale -- fails at least one of them.

Definitions (Lizard: An Efficient Linearization Framework for LLMs; the
papernotes.org summary, "key designs"): h_i = gamma_i (.) h_{i-1} + phi(k_i) v_i^T,
y_i = phi(q_i)^T h_i; local branch = softmax over [q_i.T_k ; q_i.k_{i-W+1..i}]
applied to [T_v ; v]; "overall framework": weighted merge of the two branches.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from linearized_attention_amd.synthetic import make_fwd_inputs, make_decode_inputs

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _np(t):
    return t.detach().to(torch.float64).numpy()


def _phi(x, w):
    """Feature map through torch's own softmax (a library routine)."""
    x = torch.as_tensor(np.asarray(x), dtype=torch.float64)
    w = torch.as_tensor(np.asarray(w), dtype=torch.float64)
    return torch.softmax(x @ w, dim=-1).numpy()


def _run(inp, return_state=False):
    return oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                             return_branches=True, return_state=return_state)


def _small(gate="logsigmoid", **kw):
    args = dict(B=2, Hq=2, Hkv=2, L=40, d=8, W=5, M=3, dtype="f32", seed=7, gate=gate)
    args.update(kw)
    return make_fwd_inputs(**args)


# --------------------------------------------------------------------------
# A worked example derived by hand from the definitions (d = 2).
# W_phi = [[ln 3, 0], [0, 0]] makes phi take the values (3/4,1/4), (1/2,1/2),
# (1/4,3/4) for x = (1,0), (0,1), (-1,0).
#   k = (1,0),(0,1),(-1,0)  -> phi_k = (3/4,1/4),(1/2,1/2),(1/4,3/4)
#   q = (0,1),(1,0),(-1,0)  -> phi_q = (1/2,1/2),(3/4,1/4),(1/4,3/4)
#   v = (1,0),(0,2),(1,1);  gamma_1 = (1/2,1/4), gamma_2 = (1,1/2)
#   h_0 = [[3/4,0],[1/4,0]]
#   h_1 = diag(1/2,1/4) h_0 + (1/2,1/2)(0,2) = [[3/8,1],[1/16,1]]
#   h_2 = diag(1,1/2) h_1 + (1/4,3/4)(1,1)   = [[5/8,5/4],[25/32,5/4]]
#   y_gla = (1/2,0), (19/64,1), (95/128,5/4)
# Window, M = 1, T_k = (0,0), T_v = (2,0), W = 2, scale 1:
#   i=0: logits (0 meta, 0) -> ((2,0)+(1,0))/2 = (3/2,0)
#   i=1: logits (0, 1, 0) over (T, k0, k1) -> ((2,0)+e(1,0)+(0,2))/(2+e) = (1, 2/(2+e))
#   i=2: logits (0, 0, 1) over (T, k1, k2) -> ((2,0)+(0,2)+e(1,1))/(2+e) = (1, 1)
# --------------------------------------------------------------------------
def test_hand_worked_example():
    ln3 = math.log(3.0)
    wphi = np.array([[ln3, 0.0], [0.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]])
    q = np.array([[0.0, 1.0], [1.0, 0.0], [-1.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 2.0], [1.0, 1.0]])
    lg = np.log(np.array([[0.5, 0.25], [0.5, 0.25], [1.0, 0.5]]))
    tk = np.array([[[0.0, 0.0]]])
    tv = np.array([[[2.0, 0.0]]])
    y, yg, yw = oracle.lizard_fwd(q[None, None], k[None, None], v[None, None], lg[None, None],
                                  wphi, wphi, tk, tv, W=2, M=1, mix=0.5, scale=1.0,
                                  return_branches=True)
    e = math.e
    want_g = np.array([[0.5, 0.0], [19 / 64, 1.0], [95 / 128, 1.25]])
    want_w = np.array([[1.5, 0.0], [1.0, 2 / (2 + e)], [1.0, 1.0]])
    np.testing.assert_allclose(yg[0, 0], want_g, rtol=0, atol=1e-14)
    np.testing.assert_allclose(yw[0, 0], want_w, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[0, 0], 0.5 * (want_g + want_w), rtol=0, atol=1e-14)


# ------------------------------ global branch ------------------------------
def test_gamma_one_is_causal_linear_attention():
    """gamma = 1: y_i = phi(q_i)^T sum_{s<=i} phi(k_s) v_s^T (torch cumsum)."""
    inp = _small(gate="one")
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))
    outer = torch.einsum("bhlf,bhle->bhlfe", torch.from_numpy(phk), torch.from_numpy(_np(inp.v)))
    S = torch.cumsum(outer, dim=2).numpy()
    want = np.einsum("bhlf,bhlfe->bhle", phq, S)
    np.testing.assert_allclose(yg, want, rtol=1e-12, atol=1e-13)


def test_gamma_zero_keeps_only_current_token():
    """gamma = 0: y_i = (phi(q_i) . phi(k_i)) v_i."""
    inp = _small(gate="zero")
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))
    want = (phq * phk).sum(-1, keepdims=True) * _np(inp.v)
    np.testing.assert_allclose(yg, want, rtol=1e-12, atol=1e-14)


def test_constant_scalar_gate_geometric_closed_form():
    """gamma_i = lam for every dim: y = ((phi_q phi_k^T) * lam^(i-s) * [s<=i]) v."""
    lam_log = -0.3
    inp = _small(gate=f"const:{lam_log}", L=33)
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))
    lam = float(np.exp(np.float64(torch.tensor(lam_log, dtype=torch.float32).item())))
    L = inp.q.shape[2]
    i = np.arange(L)[:, None]
    s = np.arange(L)[None, :]
    decay = np.where(s <= i, lam ** np.maximum(i - s, 0), 0.0)
    A = np.einsum("bhif,bhsf->bhis", phq, phk) * decay
    want = A @ _np(inp.v)
    np.testing.assert_allclose(yg, want, rtol=1e-11, atol=1e-13)


def test_per_dim_gate_brute_force_products():
    """y_i = sum_{s<=i} sum_f phq_if phk_sf (prod_{j=s+1..i} gamma_jf) v_s, with
    the gate products multiplied out directly (no logs, no recurrence)."""
    inp = _small(L=9, d=4, B=1, Hq=1, Hkv=1, gate="uniform:-2")
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))[0, 0]
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))[0, 0]
    gam = np.exp(_np(inp.log_gamma)[0, 0])
    v = _np(inp.v)[0, 0]
    L = v.shape[0]
    want = np.zeros_like(v)
    for i in range(L):
        for s in range(i + 1):
            prod = np.ones(gam.shape[1])
            for j in range(s + 1, i + 1):
                prod = prod * gam[j]
            want[i] += (phq[i] * phk[s] * prod).sum() * v[s]
    np.testing.assert_allclose(yg[0, 0], want, rtol=1e-12, atol=1e-14)


def test_gate_acts_on_key_dimension_not_value_dimension():
    """Decaying the value dimension instead would match the per-dim brute force
    only if the gate were constant across dims; here it is not."""
    inp = _small(L=6, d=4, B=1, Hq=1, Hkv=1, gate="uniform:-3")
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))[0, 0]
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))[0, 0]
    gam = np.exp(_np(inp.log_gamma)[0, 0])
    v = _np(inp.v)[0, 0]
    S_wrong = np.zeros((4, 4))
    wrong = np.zeros_like(v)
    for i in range(v.shape[0]):
        S_wrong = S_wrong * gam[i][None, :] + np.outer(phk[i], v[i])
        wrong[i] = phq[i] @ S_wrong
    assert np.abs(yg[0, 0] - wrong).max() > 1e-3


def _chunked_gla(phq, phk, lg, v, C):
    """Chunkwise fp64 GLA: per chunk, local inclusive cumsum b of log gamma;
    intra = sum_{s<=t} sum_f phq_t phk_s exp(b_t - b_s) v_s; inter =
    (phq_t * exp(b_t)) S; S <- exp(b_last) S + sum_s (phk_s * exp(b_last - b_s)) v_s^T."""
    L, df = phk.shape
    dv = v.shape[1]
    S = np.zeros((df, dv))
    y = np.zeros((L, dv))
    for c0 in range(0, L, C):
        c1 = min(L, c0 + C)
        b = np.cumsum(lg[c0:c1], axis=0)
        qq, kk, vv = phq[c0:c1], phk[c0:c1], v[c0:c1]
        n = c1 - c0
        diff = b[:, None, :] - b[None, :, :]
        mask = np.tril(np.ones((n, n), dtype=bool))
        A = np.where(mask, np.einsum("tf,sf,tsf->ts", qq, kk, np.exp(np.where(mask[..., None], diff, 0.0))), 0.0)
        y[c0:c1] = A @ vv + (qq * np.exp(b)) @ S
        S = np.exp(b[-1])[:, None] * S + (kk * np.exp(b[-1][None, :] - b)).T @ vv
    return y


@pytest.mark.parametrize("C", [1, 7, 16, 64, 1000])
def test_chunked_form_equals_recurrence(C):
    inp = _small(L=150, d=8, gate="uniform:-5", B=1, Hq=2, Hkv=2)
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))
    lg, v = _np(inp.log_gamma), _np(inp.v)
    for h in range(2):
        want = _chunked_gla(phq[0, h], phk[0, h], lg[0, h], v[0, h], C)
        np.testing.assert_allclose(yg[0, h], want, rtol=1e-10, atol=1e-13)


def test_first_token_any_gate():
    inp = _small(gate="uniform")
    _, yg, _ = _run(inp)
    phq = _phi(_np(inp.q), _np(inp.w_phi_q))[:, :, 0]
    phk = _phi(_np(inp.k), _np(inp.w_phi_k))[:, :, 0]
    want = (phq * phk).sum(-1, keepdims=True) * _np(inp.v)[:, :, 0]
    np.testing.assert_allclose(yg[:, :, 0], want, rtol=1e-12, atol=1e-14)


def test_linear_in_v_and_feature_permutation_invariant():
    inp = _small()
    _, yg, _ = _run(inp)
    # linearity in v (the local branch is linear in v too)
    v2 = make_fwd_inputs(B=2, Hq=2, Hkv=2, L=40, d=8, W=5, M=3, dtype="f32", seed=99).v
    a, b = 0.75, -1.5
    comb = torch.from_numpy(a * _np(inp.v) + b * _np(v2))
    y1 = oracle.lizard_fwd(inp.q, inp.k, inp.v, inp.log_gamma, inp.w_phi_q, inp.w_phi_k,
                           inp.t_k, inp.t_v, W=inp.W, M=inp.M, mix=1.0, scale=inp.scale)
    y2 = oracle.lizard_fwd(inp.q, inp.k, v2, inp.log_gamma, inp.w_phi_q, inp.w_phi_k,
                           inp.t_k, inp.t_v, W=inp.W, M=inp.M, mix=1.0, scale=inp.scale)
    y3 = oracle.lizard_fwd(inp.q, inp.k, comb, inp.log_gamma, inp.w_phi_q, inp.w_phi_k,
                           inp.t_k, inp.t_v, W=inp.W, M=inp.M, mix=1.0, scale=inp.scale)
    np.testing.assert_allclose(y3, a * y1 + b * y2, rtol=1e-11, atol=1e-12)
    # a joint permutation of feature dims (W_phi columns with log gamma dims)
    perm = np.random.default_rng(3).permutation(8)
    wq = _np(inp.w_phi_q)[:, perm]
    lgp = _np(inp.log_gamma)[..., perm]
    _, ygp, _ = oracle.lizard_fwd(inp.q, inp.k, inp.v, lgp, wq, wq, inp.t_k, inp.t_v,
                                  W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                  return_branches=True)
    np.testing.assert_allclose(ygp, yg, rtol=1e-11, atol=1e-13)
    # permuting only W_phi (gate left in place) must change the answer
    _, ygx, _ = oracle.lizard_fwd(inp.q, inp.k, inp.v, inp.log_gamma, wq, wq, inp.t_k, inp.t_v,
                                  W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                  return_branches=True)
    assert np.abs(ygx - yg).max() > 1e-4


def test_state_out_matches_last_readout():
    inp = _small(gate="uniform")
    _, yg, _, st = _run(inp, return_state=True)
    phq_last = _phi(_np(inp.q)[:, :, -1], _np(inp.w_phi_q))
    want = np.einsum("bhf,bhfe->bhe", phq_last, st)
    np.testing.assert_allclose(yg[:, :, -1], want, rtol=1e-12, atol=1e-14)


# ------------------------------ local branch ------------------------------
def _sdpa(q, keys, vals, mask, scale):
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(keys),
                                          torch.from_numpy(vals), attn_mask=torch.from_numpy(mask),
                                          scale=scale).numpy()


def test_window_covering_sequence_is_causal_softmax_attention():
    inp = _small(W=40, M=0, L=40)
    _, _, yw = _run(inp)
    want = F.scaled_dot_product_attention(torch.from_numpy(_np(inp.q)), torch.from_numpy(_np(inp.k)),
                                          torch.from_numpy(_np(inp.v)), is_causal=True,
                                          scale=inp.scale).numpy()
    np.testing.assert_allclose(yw, want, rtol=1e-11, atol=1e-13)
    inp2 = _small(W=1000, M=0, L=40)
    _, _, yw2 = _run(inp2)
    np.testing.assert_allclose(yw2, want, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("W,M", [(1, 2), (3, 4), (5, 1), (17, 3), (64, 8)])
def test_window_with_meta_tokens_matches_masked_sdpa(W, M):
    """softmax over [T_k ; K] with the mask  meta: always;  key j: i-W < j <= i."""
    inp = _small(W=W, M=M, L=40, d=16)
    _, _, yw = _run(inp)
    q, k, v = _np(inp.q), _np(inp.k), _np(inp.v)
    B, H, L, d = q.shape
    tk = np.broadcast_to(_np(inp.t_k)[None], (B, H, M, d))
    tv = np.broadcast_to(_np(inp.t_v)[None], (B, H, M, d))
    keys = np.concatenate([tk, k], axis=2)
    vals = np.concatenate([tv, v], axis=2)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    band = (j <= i) & (j > i - W)
    mask = np.concatenate([np.ones((L, M), dtype=bool), band], axis=1)
    want = _sdpa(q, np.ascontiguousarray(keys), np.ascontiguousarray(vals), mask, inp.scale)
    np.testing.assert_allclose(yw, want, rtol=1e-11, atol=1e-13)


def test_window_one_no_meta_returns_v():
    inp = _small(W=1, M=0)
    _, _, yw = _run(inp)
    np.testing.assert_array_equal(yw, _np(inp.v))


def test_mix_isolates_branches():
    inp = _small()
    y, yg, yw = _run(inp)
    np.testing.assert_allclose(y, 0.5 * yg + 0.5 * yw, rtol=1e-14, atol=1e-15)
    args = (inp.q, inp.k, inp.v, inp.log_gamma, inp.w_phi_q, inp.w_phi_k, inp.t_k, inp.t_v)
    y1 = oracle.lizard_fwd(*args, W=inp.W, M=inp.M, mix=1.0, scale=inp.scale)
    y0 = oracle.lizard_fwd(*args, W=inp.W, M=inp.M, mix=0.0, scale=inp.scale)
    np.testing.assert_array_equal(y1, yg)
    np.testing.assert_array_equal(y0, yw)


# ------------------------------ GQA, decode ------------------------------
def test_gqa_equals_repeated_heads():
    inp = _small(Hq=6, Hkv=2, L=30, d=8, gate="uniform", per_head_w=True, separate_wk=True)
    y = oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale)
    G = 3
    rep = lambda t: torch.repeat_interleave(t, G, dim=1)
    rep0 = lambda t: torch.repeat_interleave(t, G, dim=0)
    y_mha = oracle.lizard_fwd(inp.q, rep(inp.k), rep(inp.v), rep(inp.log_gamma), inp.w_phi_q,
                              rep0(inp.w_phi_k), rep0(inp.t_k), rep0(inp.t_v), W=inp.W, M=inp.M,
                              mix=inp.mix, scale=inp.scale)
    np.testing.assert_allclose(y, y_mha, rtol=1e-13, atol=1e-14)


def test_decode_from_empty_equals_forward():
    L, d, W, M = 23, 8, 5, 2
    dec = make_decode_inputs(N=3, Hq=4, Hkv=2, d=d, W=W, M=M, steps=L, pos0=0, dtype="f32",
                             seed=11, zero_state=True, gate="uniform")
    st, rk, rv, pos = dec.state, dec.ring_k, dec.ring_v, dec.pos
    outs = []
    for (q, k, v, lg) in dec.steps:
        out, st, rk, rv, pos = oracle.lizard_decode(st, rk, rv, pos, q, k, v, lg, dec.w_phi_q,
                                                    dec.w_phi_k, dec.t_k, dec.t_v, M=M,
                                                    mix=dec.mix, scale=dec.scale)
        outs.append(out)
    assert (pos == L).all()
    ydec = np.stack(outs, axis=2)                       # [N,Hq,L,d]
    stack = lambda i: torch.stack([s[i] for s in dec.steps], dim=2)
    yf, sf = oracle.lizard_fwd(stack(0), stack(1), stack(2), stack(3), dec.w_phi_q, dec.w_phi_k,
                               dec.t_k, dec.t_v, W=W, M=M, mix=dec.mix, scale=dec.scale,
                               return_state=True)
    np.testing.assert_allclose(ydec, yf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, sf, rtol=1e-12, atol=1e-13)


def test_decode_window_reads_ring_by_position():
    """Ring holds tokens pos-W..pos-1 in slots t % W; after the step the window
    is meta + tokens pos-W+1..pos (torch sdpa over keys rebuilt by position)."""
    N, H, d, W, M, pos0 = 2, 2, 8, 6, 3, 37
    dec = make_decode_inputs(N=N, Hq=H, Hkv=H, d=d, W=W, M=M, steps=1, pos0=pos0, dtype="f32",
                             seed=5)
    q, k, v, lg = dec.steps[0]
    _, _, _, _, _, yg, yw = oracle.lizard_decode(dec.state, dec.ring_k, dec.ring_v, dec.pos, q, k, v,
                                                 lg, dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v,
                                                 M=M, mix=0.5, scale=dec.scale, return_branches=True)
    rk, rv = _np(dec.ring_k), _np(dec.ring_v)
    toks = list(range(pos0 - W + 1, pos0 + 1))
    keys = np.stack([k.double().numpy() if t == pos0 else rk[:, :, t % W] for t in toks], axis=2)
    vals = np.stack([v.double().numpy() if t == pos0 else rv[:, :, t % W] for t in toks], axis=2)
    tk = np.broadcast_to(_np(dec.t_k)[None], (N, H, M, d))
    tv = np.broadcast_to(_np(dec.t_v)[None], (N, H, M, d))
    K = np.ascontiguousarray(np.concatenate([tk, keys], axis=2))
    V = np.ascontiguousarray(np.concatenate([tv, vals], axis=2))
    want = _sdpa(_np(q)[:, :, None], K, V, np.ones((1, M + W), dtype=bool), dec.scale)[:, :, 0]
    np.testing.assert_allclose(yw, want, rtol=1e-11, atol=1e-13)
    # global branch: h' = gamma h + phi(k) v^T, read out with phi(q)
    S = _np(dec.state)
    phk = _phi(_np(k), _np(dec.w_phi_k))
    phq = _phi(_np(q), _np(dec.w_phi_q))
    S2 = np.exp(_np(lg))[..., None] * S + phk[..., None] * _np(v)[..., None, :]
    np.testing.assert_allclose(yg, np.einsum("nhf,nhfe->nhe", phq, S2), rtol=1e-12, atol=1e-13)
