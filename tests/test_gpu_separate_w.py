"""Separate and per-head W_phi on the whole-head forward path, for both feature maps.

The pages train the query and key feature maps separately (arXiv page, Experiments: the first
stage trains phi_q and phi_k); the Hedgehog map is the paper's own (arXiv page, Method).  When the
query side's matrix differs from the key side's, the query waves read their W_phi^T operands
from a fragment-ordered copy in global memory (windows above 65 keys: the query feature maps
come from a pass of their own), and the main kernel keeps the key side's W_phi^T in LDS.
Parity with the fp64 oracle per (batch, head): relative L2 <= 2e-2 (bf16) for the merged output and each branch; and bitwise equality with
the shared-matrix call when the separate matrices hold equal values.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd import api
from linearized_attention_amd.synthetic import WORKLOADS, make_fwd_inputs

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAPS = ("softmax", "hedgehog")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, want):
    num = np.sqrt(((got - want) ** 2).sum(axis=(-2, -1)))
    den = np.sqrt((want ** 2).sum(axis=(-2, -1)))
    return num / np.maximum(den, 1e-300)


def gpu_fwd(dev, inp, mix, fmap):
    fn = api.lizard_attn_fwd_hedgehog if fmap == "hedgehog" else api.lizard_attn_fwd
    out = fn(dev.q, dev.k, dev.v, dev.log_gamma, dev.w_phi_q, dev.w_phi_k, dev.t_k, dev.t_v, W=inp.W, M=inp.M,
             mix=mix, scale=inp.scale)
    torch.cuda.synchronize()
    return out


def inputs(label, fmap, **kw):
    d = kw["d"]
    return make_fwd_inputs(dtype="bf16", seed=zlib.crc32(label.encode()) % 10000,
                           phi_cols=d // 2 if fmap == "hedgehog" else None, **kw)


def check(label, inp, fmap):
    _say(f"[separate W, {fmap}] {label}: q{tuple(inp.q.shape)} k{tuple(inp.k.shape)} "
         f"w_q{tuple(inp.w_phi_q.shape)} w_k{tuple(inp.w_phi_k.shape)} W={inp.W}")
    y, yg, yw = oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                  return_branches=True, feature_map=fmap)
    dev = inp.to("cuda")
    for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
        got = gpu_fwd(dev, inp, mix, fmap).double().cpu().numpy()
        assert np.isfinite(got).all(), f"{label}/{name}: non-finite output"
        e = float(rel_l2(got, want).max())
        _say(f"      {name}: rel-L2 max per head {e:.3e}")
        assert e <= TOL, f"{label}/{name}: {e:.3e} > {TOL}"


CASES = [
    ("separate, ragged L200", dict(B=2, Hq=2, Hkv=2, L=200, d=128, W=64, M=4, separate_wk=True), 1),
    ("per-head G1", dict(B=1, Hq=3, Hkv=3, L=150, d=128, W=64, M=4, per_head_w=True), 1),
    ("per-head gqa 4:2", dict(B=1, Hq=4, Hkv=2, L=190, d=128, W=64, M=4, per_head_w=True, separate_wk=True), 1),
    ("separate, gamma=0 (exact diagonal)", dict(B=1, Hq=2, Hkv=2, L=130, d=128, W=64, M=4, gate="zero",
                                                separate_wk=True), 1),
    ("separate, W100 M8 (window two chunks back)", dict(B=1, Hq=2, Hkv=2, L=300, d=128, W=100, M=8,
                                                        separate_wk=True), 1),
    ("per-head, 3 segments (state pass)", dict(B=1, Hq=2, Hkv=2, L=650, d=128, W=65, M=16, gate="uniform:-1.6",
                                               per_head_w=True, separate_wk=True), 3),
    ("separate, 2 segments (self-started)", dict(B=2, Hq=2, Hkv=2, L=700, d=128, W=64, M=4, separate_wk=True), 2),
    ("L1", dict(B=2, Hq=2, Hkv=2, L=1, d=128, W=64, M=4, separate_wk=True), 1),
]


@pytest.mark.parametrize("fmap", MAPS)
@pytest.mark.parametrize("label,kw,nseg", CASES, ids=[c[0] for c in CASES])
def test_separate_w_matches_oracle(gpu_lib, lz_opts, fmap, label, kw, nseg):
    lz_opts("fwd_segments", nseg)
    check(label, inputs(label, fmap, **kw), fmap)


@pytest.mark.parametrize("fmap", MAPS)
@pytest.mark.parametrize("nseg", [1, 2, 3])
@pytest.mark.parametrize("W", [64, 100])
def test_separate_matrices_with_equal_values_match_the_shared_call(gpu_lib, lz_opts, fmap, nseg, W):
    """w_phi_k a copy of w_phi_q (another allocation, the same values), and per-head matrices that
    are all the same: the query logits take the same operand values in the same order (from the
    fragment-ordered copy, or with W = 100 from the feature-map pass), with the same map and
    rounding as with the shared matrix, so every output bit matches the shared call."""
    lz_opts("fwd_segments", nseg)
    inp = inputs(f"equal {fmap} {nseg}", fmap, B=1, Hq=4, Hkv=2, L=600, d=128, W=W, M=4,
                 gate="uniform:-1.6")
    dev = inp.to("cuda")
    shared = gpu_fwd(dev, inp, inp.mix, fmap).cpu()
    fn = api.lizard_attn_fwd_hedgehog if fmap == "hedgehog" else api.lizard_attn_fwd
    wk = dev.w_phi_q.clone()
    sep = fn(dev.q, dev.k, dev.v, dev.log_gamma, dev.w_phi_q, wk, dev.t_k, dev.t_v, W=inp.W, M=inp.M,
             mix=inp.mix, scale=inp.scale).cpu()
    wq_h = dev.w_phi_q.unsqueeze(0).repeat(4, 1, 1).contiguous()
    wk_h = dev.w_phi_q.unsqueeze(0).repeat(2, 1, 1).contiguous()
    per = fn(dev.q, dev.k, dev.v, dev.log_gamma, wq_h, wk_h, dev.t_k, dev.t_v, W=inp.W, M=inp.M,
             mix=inp.mix, scale=inp.scale).cpu()
    torch.cuda.synchronize()
    assert torch.equal(sep, shared), "separate equal matrices differ from the shared call"
    assert torch.equal(per, shared), "equal per-head matrices differ from the shared call"


@pytest.mark.parametrize("fmap", MAPS)
def test_separate_per_head_w_full_size_sampled_heads(gpu_lib, fmap):
    """The 4 x 32 x 4096 layer with a W_phi per query head and per key/value head (separate for
    the two sides), oracle on sampled heads."""
    c = WORKLOADS[1]
    inp = make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"], M=c["M"],
                          dtype="bf16", seed=3001, per_head_w=True, separate_wk=True,
                          phi_cols=c["d"] // 2 if fmap == "hedgehog" else None)
    _say(f"[separate W, {fmap}] full size q{tuple(inp.q.shape)} w_q{tuple(inp.w_phi_q.shape)}")
    dev = inp.to("cuda")
    outs = {mix: gpu_fwd(dev, inp, mix, fmap).cpu() for mix in (inp.mix, 1.0, 0.0)}
    for (b, h) in [(0, 0), (3, 31), (2, 14)]:
        sl = lambda t: t[b:b + 1, h:h + 1]
        y, yg, yw = oracle.lizard_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.log_gamma),
                                      inp.w_phi_q[h:h + 1], inp.w_phi_k[h:h + 1], inp.t_k[h:h + 1],
                                      inp.t_v[h:h + 1], W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                      return_branches=True, feature_map=fmap)
        for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
            e = float(rel_l2(outs[mix][b:b + 1, h:h + 1].double().numpy(), want).max())
            _say(f"      (b={b}, h={h}) {name}: rel-L2 {e:.3e}")
            assert e <= TOL, f"(b={b},h={h}) {name}: {e:.3e}"


@pytest.mark.parametrize("idx,fmap,heads", [
    (4, "softmax", [(0, 0), (1, 13), (1, 31)]),
    (4, "hedgehog", [(1, 7)]),
    (2, "softmax", [(0, 5)]),
    (2, "hedgehog", [(0, 17)]),
], ids=["gqa-softmax", "gqa-hedgehog", "32k-softmax", "32k-hedgehog"])
def test_separate_per_head_w_gqa_and_long_context_sampled_heads(gpu_lib, idx, fmap, heads):
    """The grouped-query layer (32 query heads on 8 key/value heads, one W_phi copy per query head)
    and the 32K uniform-gate stress (windows of 128 keys: the feature-map pass) with a W_phi per
    query head and per key/value head, oracle on sampled heads."""
    c = WORKLOADS[idx]
    G = c["Hq"] // c["Hkv"]
    inp = make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"], M=c["M"],
                          dtype="bf16", seed=3100 + idx, gate=c["gate"], per_head_w=True, separate_wk=True,
                          phi_cols=c["d"] // 2 if fmap == "hedgehog" else None)
    _say(f"[separate W, {fmap}] workload {idx} q{tuple(inp.q.shape)} k{tuple(inp.k.shape)} "
         f"w_q{tuple(inp.w_phi_q.shape)} w_k{tuple(inp.w_phi_k.shape)}")
    dev = inp.to("cuda")
    outs = {mix: gpu_fwd(dev, inp, mix, fmap).cpu() for mix in (inp.mix, 1.0, 0.0)}
    del dev
    for (b, h) in heads:
        hk = h // G
        qs = lambda t: t[b:b + 1, h:h + 1]
        ks = lambda t: t[b:b + 1, hk:hk + 1]
        y, yg, yw = oracle.lizard_fwd(qs(inp.q), ks(inp.k), ks(inp.v), ks(inp.log_gamma),
                                      inp.w_phi_q[h:h + 1], inp.w_phi_k[hk:hk + 1], inp.t_k[hk:hk + 1],
                                      inp.t_v[hk:hk + 1], W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                      return_branches=True, feature_map=fmap)
        for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
            e = float(rel_l2(outs[mix][b:b + 1, h:h + 1].double().numpy(), want).max())
            _say(f"      (b={b}, h={h}, kv head {hk}) {name}: rel-L2 {e:.3e}")
            assert e <= TOL, f"(b={b},h={h}) {name}: {e:.3e}"
