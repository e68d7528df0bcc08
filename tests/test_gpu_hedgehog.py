"""Parity of the Hedgehog-map entry points with the fp64 oracle.

phi(x) = exp(xW) (+) exp(-xW) with W_phi [d, d/2] (the Lizard paper's own feature map:
arXiv page, Method section, hardware-efficient reparameterization paragraph).  Relative
L2 per (batch, head) over L x d, for the merged output and each branch (mix = 1: the gated
linear attention branch, mix = 0: the window): <= 2e-2 for bf16.  Decode: the same per head
over all (sequence, step) outputs, plus the fp32 state; L steps from an empty state equal
the forward.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd import api
from linearized_attention_amd.synthetic import WORKLOADS, make_decode_inputs, make_fwd_inputs

pytestmark = pytest.mark.gpu
TOL = 2e-2  # bf16


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, want, axes):
    num = np.sqrt(((got - want) ** 2).sum(axis=axes))
    den = np.sqrt((want ** 2).sum(axis=axes))
    return num / np.maximum(den, 1e-300)


def hh_inputs(label, **kw):
    kw.setdefault("dtype", "bf16")
    return make_fwd_inputs(seed=zlib.crc32(label.encode()) % 10000, phi_cols=kw["d"] // 2, **kw)


def gpu_fwd_hh(dev, inp, mix):
    out = api.lizard_attn_fwd_hedgehog(dev.q, dev.k, dev.v, dev.log_gamma, dev.w_phi_q, dev.w_phi_k,
                                       dev.t_k, dev.t_v, W=inp.W, M=inp.M, mix=mix, scale=inp.scale)
    torch.cuda.synchronize()
    return out


def check_case(label, inp):
    _say(f"[hedgehog fwd] {label}: q{tuple(inp.q.shape)} k{tuple(inp.k.shape)} W={inp.W} M={inp.M}")
    y, yg, yw = oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                  return_branches=True, feature_map="hedgehog")
    dev = inp.to("cuda")
    worst = {}
    for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
        got = gpu_fwd_hh(dev, inp, mix).double().cpu().numpy()
        assert np.isfinite(got).all(), f"{label}/{name}: non-finite output"
        worst[name] = float(rel_l2(got, want, axes=(-2, -1)).max())
    _say(f"      rel-L2 max per head: {worst}")
    for name, e in worst.items():
        assert e <= TOL, f"{label}/{name}: rel L2 {e:.3e} > {TOL}"


CASES = [
    ("ragged L200", dict(B=2, Hq=2, Hkv=2, L=200, d=128, W=64, M=4), 1),
    ("gqa 4:2 L300", dict(B=1, Hq=4, Hkv=2, L=300, d=128, W=64, M=4), 1),
    ("uniform gate W128 M8", dict(B=1, Hq=2, Hkv=2, L=256, d=128, W=128, M=8, gate="uniform"), 1),
    ("gamma=0 (exact diag)", dict(B=1, Hq=2, Hkv=2, L=130, d=128, W=64, M=4, gate="zero"), 1),
    ("gamma=1", dict(B=1, Hq=2, Hkv=2, L=256, d=128, W=64, M=4, gate="one"), 1),
    ("W>=L M0", dict(B=1, Hq=2, Hkv=2, L=120, d=128, W=128, M=0), 1),
    ("L1", dict(B=2, Hq=2, Hkv=2, L=1, d=128, W=64, M=4), 1),
    ("3 segments, mixed references", dict(B=1, Hq=2, Hkv=2, L=650, d=128, W=65, M=16, gate="uniform:-1.6"), 3),
    ("2 segments, logsigmoid, decayed chunks dropped", dict(B=2, Hq=2, Hkv=2, L=1600, d=128, W=64, M=4), 2),
    ("2 segments, gamma=1", dict(B=1, Hq=2, Hkv=2, L=1000, d=128, W=64, M=4, gate="one"), 2),
    ("W129 ragged, 2 segments", dict(B=2, Hq=1, Hkv=1, L=201, d=128, W=129, M=16), 2),
]


@pytest.mark.parametrize("label,kw,nseg", CASES, ids=[c[0] for c in CASES])
def test_fwd_hedgehog_matches_oracle(gpu_lib, lz_opts, label, kw, nseg):
    lz_opts("fwd_segments", nseg)
    check_case(label, hh_inputs(label, **kw))


@pytest.mark.parametrize("nseg,big_chunk,last", [(2, 7, 640), (3, 9, 768)])
def test_fwd_hedgehog_large_features_beyond_the_decay_cutoff(gpu_lib, lz_opts, nseg, big_chunk, last):
    """The unnormalised Hedgehog features can reach e^60 (logits up to the documented bound of
    about 80).  A chunk whose keys carry such features and that reaches the next segment decayed
    by about e^-45 still dominates its outputs (e^15 against O(e^3) terms), so the segment walks
    must not drop it at the softmax map's cutoff of e^-24.  Gate -0.35 per token (22.4 per chunk),
    16 chunks; the last four keys of chunk `big_chunk` point along one column of W_phi so that
    one logit is 60.  With two segments the second starts at chunk 10 (split shift 2) and walks
    back; with three the state pass walks the middle block.  The global branch (mix = 1) of the
    last segment's rows is compared with the oracle: without those chunks it would be off by
    about 100% (checked on the CPU with the oracle when the case was written)."""
    lz_opts("fwd_segments", nseg)
    inp = make_fwd_inputs(B=1, Hq=1, Hkv=1, L=1024, d=128, W=64, M=4, dtype="bf16", seed=77 + nseg,
                          gate="const:-0.35", phi_cols=64)
    w = inp.w_phi_k.double().numpy()
    col = w[:, int(np.argmax((w ** 2).sum(0)))]
    k = inp.k.double().numpy().copy()
    t1 = (big_chunk + 1) * 64
    k[0, 0, t1 - 4:t1] = col * (60.0 / (col @ col))
    inp.k = torch.tensor(k).to(torch.bfloat16)
    _say(f"[hedgehog fwd] large features beyond the cutoff, {nseg} segments, chunk {big_chunk}")
    _, yg, _ = oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=1.0, scale=inp.scale,
                                 return_branches=True, feature_map="hedgehog")
    got = gpu_fwd_hh(inp.to("cuda"), inp, 1.0).double().cpu().numpy()
    assert np.isfinite(got).all()
    e = float(rel_l2(got[:, :, last:], yg[:, :, last:], axes=(-2, -1)).max())
    e_all = float(rel_l2(got, yg, axes=(-2, -1)).max())
    _say(f"      rel-L2 of the last segment's rows {e:.3e}, all rows {e_all:.3e}")
    assert e <= TOL and e_all <= TOL


def test_fwd_hedgehog_full_size_sampled_heads(gpu_lib):
    """The 4 x 32 x 4096 layer shape with the Hedgehog map (two segments per head, so the
    state pass runs), oracle on sampled heads."""
    c = WORKLOADS[1]
    inp = make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"], M=c["M"],
                          dtype="bf16", seed=2001, phi_cols=c["d"] // 2)
    _say(f"[hedgehog fwd] full size q{tuple(inp.q.shape)}")
    dev = inp.to("cuda")
    outs = {mix: gpu_fwd_hh(dev, inp, mix).cpu() for mix in (inp.mix, 1.0, 0.0)}
    for (b, h) in [(0, 0), (3, 31), (1, 20)]:
        sl = lambda t: t[b:b + 1, h:h + 1]
        y, yg, yw = oracle.lizard_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.log_gamma), inp.w_phi_q,
                                      inp.w_phi_k, inp.t_k[h:h + 1], inp.t_v[h:h + 1], W=inp.W, M=inp.M,
                                      mix=inp.mix, scale=inp.scale, return_branches=True,
                                      feature_map="hedgehog")
        for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
            e = float(rel_l2(outs[mix][b:b + 1, h:h + 1].double().numpy(), want, axes=(-2, -1)).max())
            _say(f"      (b={b}, h={h}) {name}: rel-L2 {e:.3e}")
            assert e <= TOL, f"(b={b},h={h}) {name}: {e:.3e}"


def test_fwd_hedgehog_rejects_unsupported_shapes(gpu_lib):
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=64, d=64, W=64, M=4, dtype="bf16", seed=1, phi_cols=32)
    g = inp.to("cuda")
    with pytest.raises(api.LizardError):  # d = 64 is not built for the Hedgehog forward
        api.lizard_attn_fwd_hedgehog(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, g.w_phi_k, g.t_k, g.t_v,
                                     W=64, M=4)


def _decode_steps(dec, hedgehog=True):
    st = dec.state.clone().cuda()
    rk, rv, pos = dec.ring_k.clone().cuda(), dec.ring_v.clone().cuda(), dec.pos.clone().cuda()
    args = [t.cuda() for t in (dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v)]
    fn = api.lizard_attn_decode_hedgehog if hedgehog else api.lizard_attn_decode
    outs = []
    for (q, k, v, lg) in dec.steps:
        o = fn(st, rk, rv, pos, q.cuda(), k.cuda(), v.cuda(), lg.cuda(), *args, M=dec.M, mix=dec.mix,
               scale=dec.scale)
        outs.append(o.double().cpu().numpy())
    torch.cuda.synchronize()
    return np.stack(outs, axis=2), st.double().cpu().numpy(), pos.cpu().numpy()


DEC_CASES = [
    ("bf16 d128 pos0=100", dict(N=6, Hq=3, Hkv=3, d=128, W=64, M=4, steps=3, pos0=100, dtype="bf16")),
    ("bf16 d64 gqa 8:2 W100", dict(N=9, Hq=8, Hkv=2, d=64, W=100, M=16, steps=4, pos0=250, dtype="bf16")),
    ("fp32 d64 gqa from empty", dict(N=5, Hq=4, Hkv=2, d=64, W=16, M=2, steps=30, pos0=0, dtype="f32",
                                     zero_state=True)),
]


@pytest.mark.parametrize("label,kw", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_hedgehog_matches_oracle(gpu_lib, label, kw):
    _say(f"[hedgehog decode] {label}")
    dec = make_decode_inputs(seed=zlib.crc32(label.encode()) % 10000, phi_cols=kw["d"] // 2, **kw)
    yg, sg, pg = _decode_steps(dec)
    st, rk, rv, pos = dec.state, dec.ring_k, dec.ring_v, dec.pos
    outs = []
    for (q, k, v, lg) in dec.steps:
        out, st, rk, rv, pos = oracle.lizard_decode(st, rk, rv, pos, q, k, v, lg, dec.w_phi_q, dec.w_phi_k,
                                                    dec.t_k, dec.t_v, M=dec.M, mix=dec.mix, scale=dec.scale,
                                                    feature_map="hedgehog")
        outs.append(out)
    yo = np.stack(outs, axis=2)
    tol = 1e-4 if kw["dtype"] == "f32" else TOL
    err = rel_l2(yg, yo, axes=(0, 2, 3)).max()
    serr = rel_l2(sg, st, axes=(0, 2, 3)).max()
    _say(f"      out rel-L2 {err:.3e}   state rel-L2 {serr:.3e}")
    assert err <= tol and serr <= tol
    assert np.array_equal(pg, pos)


def test_decode_hedgehog_from_empty_equals_gpu_forward(gpu_lib):
    L, H, W, M, d = 70, 2, 64, 4, 128
    _say(f"[hedgehog decode] decode==forward L={L}")
    dec = make_decode_inputs(N=2, Hq=H, Hkv=H, d=d, W=W, M=M, steps=L, pos0=0, dtype="bf16", seed=29,
                             zero_state=True, phi_cols=d // 2)
    yd, sd, _ = _decode_steps(dec)
    stack = lambda i: torch.stack([s[i] for s in dec.steps], dim=2).contiguous()
    q, k, v, lg = (stack(i).cuda() for i in range(4))
    w = dec.w_phi_q.cuda()  # one W_phi for both sides (the decode inputs share it)
    assert dec.w_phi_k is dec.w_phi_q
    yf = api.lizard_attn_fwd_hedgehog(q, k, v, lg, w, w, dec.t_k.cuda(), dec.t_v.cuda(), W=W, M=M,
                                      mix=dec.mix, scale=dec.scale)
    yf = yf.double().cpu().numpy()
    yo, so = oracle.lizard_fwd(stack(0), stack(1), stack(2), stack(3), dec.w_phi_q, dec.w_phi_k, dec.t_k,
                               dec.t_v, W=W, M=M, mix=dec.mix, scale=dec.scale, return_state=True,
                               feature_map="hedgehog")
    e_df = rel_l2(yd, yf, axes=(2, 3)).max()
    e_do = rel_l2(yd, yo, axes=(2, 3)).max()
    e_fo = rel_l2(yf, yo, axes=(2, 3)).max()
    e_s = rel_l2(sd, so, axes=(2, 3)).max()
    _say(f"      decode~fwd {e_df:.3e}  decode~oracle {e_do:.3e}  fwd~oracle {e_fo:.3e}  state {e_s:.3e}")
    for e in (e_df, e_do, e_fo, e_s):
        assert e <= TOL
