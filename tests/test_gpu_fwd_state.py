"""Forward as a continuation (state and ring in/out) against the fp64 oracle.

* Chunked prefill: two calls over a split sequence, the second continuing from
  the first one's state and ring, give the outputs, final state and ring of
  one oracle forward over the whole sequence.
* Continuation from an arbitrary state and full ring: the same as the oracle's
  decode steps over those tokens (decode == recurrence is pinned separately).
* Prefill then decode: the GPU decode step continues a GPU prefill exactly as
  the oracle forward over prefill + decode tokens.
Relative L2 per (batch, head): <= 1e-4 for fp32 inputs, <= 2e-2 for bf16; rings
and pos exactly.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd import api
from linearized_attention_amd.synthetic import make_decode_inputs, make_fwd_inputs
from tests.conftest import SHIFT_AUTO

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, want, axes):
    num = np.sqrt(((got - want) ** 2).sum(axis=axes))
    den = np.sqrt((want ** 2).sum(axis=axes))
    return num / np.maximum(den, 1e-300)


def _part(t, a, b):
    return t[:, :, a:b].contiguous()


CASES = [
    # label, shapes, split point, dtype
    ("fp32 d64 W64 split 130", dict(B=2, Hq=2, Hkv=2, L=300, d=64, W=64, M=4), 130, "f32"),
    ("bf16 d128 W64 split 64", dict(B=2, Hq=2, Hkv=2, L=256, d=128, W=64, M=4), 64, "bf16"),
    ("bf16 d128 W64 split 10 (short history)", dict(B=1, Hq=2, Hkv=2, L=200, d=128, W=64, M=4), 10, "bf16"),
    ("fp32 d64 W100 split 150 (two-chunk history, general window)",
     dict(B=1, Hq=2, Hkv=2, L=330, d=64, W=100, M=2), 150, "f32"),
    ("fp32 d64 W200 split 190 (history past the rings)", dict(B=1, Hq=1, Hkv=1, L=400, d=64, W=200, M=3),
     190, "f32"),
    ("bf16 gqa 4:2 split 100", dict(B=1, Hq=4, Hkv=2, L=260, d=128, W=64, M=4), 100, "bf16"),
    ("bf16 d128 W128 split 150 (window two chunks back)", dict(B=1, Hq=2, Hkv=2, L=330, d=128, W=128, M=8),
     150, "bf16"),
    ("bf16 d128 W100 split 40 (history shorter than the window)",
     dict(B=1, Hq=2, Hkv=2, L=230, d=128, W=100, M=4, gate="uniform:-1"), 40, "bf16"),
    ("fp32 d64 uniform gate split 70", dict(B=1, Hq=2, Hkv=2, L=250, d=64, W=64, M=4, gate="uniform"), 70, "f32"),
    # separate query-side W_phi: its fragment-ordered copy sits in the workspace before the history rows
    ("bf16 d128 separate W split 100", dict(B=2, Hq=2, Hkv=2, L=260, d=128, W=64, M=4, separate_wk=True),
     100, "bf16"),
    ("bf16 gqa 4:2 per-head W W100 split 150", dict(B=1, Hq=4, Hkv=2, L=300, d=128, W=100, M=4,
                                                   per_head_w=True, separate_wk=True), 150, "bf16"),
]


@pytest.mark.parametrize("label,kw,split,dtype", CASES, ids=[c[0] for c in CASES])
def test_chunked_prefill_matches_one_forward(gpu_lib, label, kw, split, dtype):
    _say(f"[fwd-ext] {label}")
    inp = make_fwd_inputs(dtype=dtype, seed=41 + split, **kw)
    B, Hq, L, d = inp.q.shape
    Hkv, W = inp.k.shape[1], inp.W
    g = inp.to("cuda")
    parts = [(0, split), (split, L)]
    for mix in (inp.mix, 1.0, 0.0):
        y, st = oracle.lizard_fwd(*inp.tensors(), W=W, M=inp.M, mix=mix, scale=inp.scale, return_state=True)
        pos = torch.zeros(B, dtype=torch.int32, device="cuda")
        rk = torch.zeros(B, Hkv, W, d, dtype=g.q.dtype, device="cuda")
        rv = torch.zeros_like(rk)
        s_prev = None
        outs = []
        for (a, b) in parts:
            s_next = torch.empty(B, Hkv, d, d, dtype=torch.float32, device="cuda")
            o = api.lizard_attn_fwd_ext(_part(g.q, a, b), _part(g.k, a, b), _part(g.v, a, b),
                                        _part(g.log_gamma, a, b), g.w_phi_q, g.w_phi_k, g.t_k, g.t_v, W=W,
                                        M=inp.M, mix=mix, scale=inp.scale, state_in=s_prev,
                                        win_k_in=rk if a > 0 else None, win_v_in=rv if a > 0 else None,
                                        pos=pos, state_out=s_next, win_k_out=rk, win_v_out=rv)
            outs.append(o.double().cpu().numpy())
            s_prev = s_next
        torch.cuda.synchronize()
        got = np.concatenate(outs, axis=2)
        err = rel_l2(got, y, axes=(2, 3)).max()
        serr = rel_l2(s_prev.double().cpu().numpy(), st, axes=(2, 3)).max()
        _say(f"      mix={mix}: out rel-L2 {err:.3e}  state rel-L2 {serr:.3e}")
        assert err <= TOL[dtype], f"mix={mix}: {err}"
        assert serr <= TOL[dtype], f"mix={mix}: state {serr}"
        assert pos.cpu().tolist() == [L] * B
        # the ring holds the last W tokens, token t in slot t % W
        k_np, v_np = inp.k.double().numpy(), inp.v.double().numpy()
        want_k = np.zeros((B, Hkv, W, d))
        want_v = np.zeros((B, Hkv, W, d))
        for t in range(max(0, L - W), L):
            want_k[:, :, t % W] = k_np[:, :, t]
            want_v[:, :, t % W] = v_np[:, :, t]
        assert np.array_equal(rk.double().cpu().numpy(), want_k)
        assert np.array_equal(rv.double().cpu().numpy(), want_v)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_continuation_from_state_and_full_ring(gpu_lib, dtype, d):
    """An arbitrary start state and a full ring at pos = 4096: the forward over L tokens
    equals L oracle decode steps from the same state and ring."""
    L, W = 80, 64
    dec = make_decode_inputs(N=2, Hq=2, Hkv=2, d=d, W=W, M=4, steps=L, pos0=4096, dtype=dtype, seed=59)
    _say(f"[fwd-ext] {dtype} d{d}: continuation from a random state, L={L}")
    q = torch.stack([s[0] for s in dec.steps], dim=2)    # [N, H, L, d]
    k = torch.stack([s[1] for s in dec.steps], dim=2)
    v = torch.stack([s[2] for s in dec.steps], dim=2)
    lg = torch.stack([s[3] for s in dec.steps], dim=2)
    st, rk_o, rv_o, ps = dec.state, dec.ring_k, dec.ring_v, dec.pos
    ys = []
    for (qs, ks, vs, ls) in dec.steps:
        o, st, rk_o, rv_o, ps = oracle.lizard_decode(st, rk_o, rv_o, ps, qs, ks, vs, ls, dec.w_phi_q, dec.w_phi_k,
                                                      dec.t_k, dec.t_v, M=dec.M, mix=dec.mix, scale=dec.scale)
        ys.append(o)
    want = np.stack(ys, axis=2)
    dev = lambda t: t.contiguous().cuda()
    s_out = torch.empty(2, 2, d, d, dtype=torch.float32, device="cuda")
    rk, rv, pos = dev(dec.ring_k), dev(dec.ring_v), dev(dec.pos)
    out = api.lizard_attn_fwd_ext(dev(q), dev(k), dev(v), dev(lg), dev(dec.w_phi_q), dev(dec.w_phi_k),
                                  dev(dec.t_k), dev(dec.t_v), W=W, M=dec.M, mix=dec.mix, scale=dec.scale,
                                  state_in=dev(dec.state), win_k_in=rk, win_v_in=rv, pos=pos, state_out=s_out,
                                  win_k_out=rk, win_v_out=rv)
    torch.cuda.synchronize()
    err = rel_l2(out.double().cpu().numpy(), want, axes=(2, 3)).max()
    serr = rel_l2(s_out.double().cpu().numpy(), st, axes=(2, 3)).max()
    _say(f"      out rel-L2 {err:.3e}  state rel-L2 {serr:.3e}")
    assert err <= TOL[dtype] and serr <= TOL[dtype]
    assert np.array_equal(pos.cpu().numpy(), ps)
    assert np.array_equal(rk.double().cpu().numpy(), rk_o)
    assert np.array_equal(rv.double().cpu().numpy(), rv_o)


def test_prefill_then_decode(gpu_lib):
    """A GPU prefill's state and ring feed GPU decode steps: outputs equal the oracle forward
    over the whole prefill + decode sequence."""
    Lp, n, W, d = 190, 6, 64, 128
    inp = make_fwd_inputs(B=2, Hq=2, Hkv=2, L=Lp + n, d=d, W=W, M=4, dtype="bf16", seed=83)
    _say(f"[fwd-ext] prefill {Lp} then {n} decode steps")
    y = oracle.lizard_fwd(*inp.tensors(), W=W, M=inp.M, mix=inp.mix, scale=inp.scale)
    g = inp.to("cuda")
    B, Hkv = 2, 2
    st = torch.empty(B, Hkv, d, d, dtype=torch.float32, device="cuda")
    rk = torch.zeros(B, Hkv, W, d, dtype=torch.bfloat16, device="cuda")
    rv = torch.zeros_like(rk)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    o = api.lizard_attn_fwd_ext(_part(g.q, 0, Lp), _part(g.k, 0, Lp), _part(g.v, 0, Lp),
                                _part(g.log_gamma, 0, Lp), g.w_phi_q, g.w_phi_k, g.t_k, g.t_v, W=W, M=inp.M,
                                mix=inp.mix, scale=inp.scale, pos=pos, state_out=st, win_k_out=rk, win_v_out=rv)
    outs = [o.double().cpu().numpy()]
    for t in range(Lp, Lp + n):
        sl = lambda x: x[:, :, t].contiguous()
        od = api.lizard_attn_decode(st, rk, rv, pos, sl(g.q), sl(g.k), sl(g.v), sl(g.log_gamma), g.w_phi_q,
                                    g.w_phi_k, g.t_k, g.t_v, M=inp.M, mix=inp.mix, scale=inp.scale)
        outs.append(od.double().cpu().numpy()[:, :, None])
    torch.cuda.synchronize()
    got = np.concatenate(outs, axis=2)
    err = rel_l2(got, y, axes=(2, 3)).max()
    _say(f"      rel-L2 {err:.3e}")
    assert err <= TOL["bf16"]
    assert pos.cpu().tolist() == [Lp + n] * B


def test_ext_with_segments(gpu_lib, lz_opts):
    """Sequence segments of the continuation call combine with the imported state."""
    lz_opts("fwd_segments", 3)
    test_chunked_prefill_matches_one_forward(gpu_lib, "fp32 3 segments", dict(B=1, Hq=2, Hkv=2, L=400, d=64,
                                                                                W=64, M=4), 100, "f32")


@pytest.mark.parametrize("nseg", [2, 3])
def test_ext_whole_head_with_segments(gpu_lib, lz_opts, nseg):
    """The whole-head path in a continuation: the first call (no state in, no history: with two
    segments its second one starts itself) exports state and ring, the second imports them
    (the state pass then, since the walk starts from zero)."""
    lz_opts("fwd_segments", nseg)
    lz_opts("fwd_split_shift", SHIFT_AUTO)
    test_chunked_prefill_matches_one_forward(gpu_lib, f"bf16 whole-head {nseg} segments",
                                             dict(B=2, Hq=2, Hkv=1, L=900, d=128, W=64, M=4), 600, "bf16")
