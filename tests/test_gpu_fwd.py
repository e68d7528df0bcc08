"""Parity of the HIP forward kernel with the fp64 oracle.

Relative L2 error per (batch, head) over L x d, for the merged output and for
each branch on its own (mix = 1 isolates the gated-linear-attention branch,
mix = 0 the window branch): <= 1e-4 for fp32 inputs, <= 2e-2 for bf16.
"""
import dataclasses
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd import api
from linearized_attention_amd.synthetic import make_fwd_inputs, workload_fwd_inputs
from tests.conftest import SHIFT_AUTO

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_l2_per_head(got, want):
    num = np.sqrt(((got - want) ** 2).sum(axis=(-2, -1)))
    den = np.sqrt((want ** 2).sum(axis=(-2, -1)))
    return num / np.maximum(den, 1e-300)


def gpu_fwd(inp, mix, dev=None):
    g = dev if dev is not None else inp.to("cuda")
    out = api.lizard_attn_fwd(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, g.w_phi_k, g.t_k, g.t_v,
                              W=inp.W, M=inp.M, mix=mix, scale=inp.scale)
    torch.cuda.synchronize()
    return out


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_case(label, inp, dtype):
    _say(f"[fwd] {label}: B={inp.q.shape[0]} Hq={inp.q.shape[1]} Hkv={inp.k.shape[1]} "
         f"L={inp.q.shape[2]} d={inp.q.shape[3]} W={inp.W} M={inp.M} {dtype}")
    y, yg, yw = oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale,
                                  return_branches=True)
    dev = inp.to("cuda")
    worst = {}
    for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
        got = gpu_fwd(inp, mix, dev).double().cpu().numpy()
        assert np.isfinite(got).all(), f"{label}/{name}: non-finite output"
        err = rel_l2_per_head(got, want)
        worst[name] = float(err.max())
    _say(f"      rel-L2 max per head: {worst}")
    for name, e in worst.items():
        assert e <= TOL[dtype], f"{label}/{name}: rel L2 {e:.3e} > {TOL[dtype]}"
    return worst


SMALL = [
    ("workload0 fp32 d64 L256", None, "f32"),
    ("bf16 d128 ragged L200", dict(B=2, Hq=2, Hkv=2, L=200, d=128, W=64, M=4), "bf16"),
    ("bf16 d64 L130", dict(B=1, Hq=3, Hkv=3, L=130, d=64, W=64, M=4), "bf16"),
    ("fp32 d64 ragged L150 W20 M3", dict(B=2, Hq=1, Hkv=1, L=150, d=64, W=20, M=3), "f32"),
    ("bf16 uniform gate W128 M8", dict(B=1, Hq=2, Hkv=2, L=256, d=128, W=128, M=8, gate="uniform"), "bf16"),
    ("fp32 uniform gate -8 (mixed safe/exact diag)", dict(B=1, Hq=2, Hkv=2, L=192, d=64, W=64, M=4,
                                                          gate="uniform:-8"), "f32"),
    ("bf16 gamma=0 (exact diag)", dict(B=1, Hq=2, Hkv=2, L=130, d=128, W=64, M=4, gate="zero"), "bf16"),
    ("fp32 gamma=0 (exact diag)", dict(B=1, Hq=2, Hkv=2, L=100, d=64, W=64, M=4, gate="zero"), "f32"),
    ("bf16 gamma=1", dict(B=1, Hq=2, Hkv=2, L=256, d=128, W=64, M=4, gate="one"), "bf16"),
    ("fp32 gamma=1", dict(B=1, Hq=1, Hkv=1, L=256, d=64, W=64, M=4, gate="one"), "f32"),
    ("bf16 W>=L M0 (full causal softmax)", dict(B=1, Hq=2, Hkv=2, L=300, d=128, W=300, M=0), "bf16"),
    ("fp32 W>=L M0", dict(B=1, Hq=1, Hkv=1, L=257, d=64, W=1000, M=0), "f32"),
    ("fp32 W1 M0", dict(B=1, Hq=2, Hkv=2, L=70, d=64, W=1, M=0), "f32"),
    ("fp32 W65 M16", dict(B=1, Hq=1, Hkv=1, L=200, d=64, W=65, M=16), "f32"),
    ("fp32 W66 (3-chunk ring)", dict(B=1, Hq=1, Hkv=1, L=200, d=64, W=66, M=1), "f32"),
    ("fp32 L1", dict(B=2, Hq=2, Hkv=2, L=1, d=64, W=64, M=4), "f32"),
    ("fp32 L17", dict(B=1, Hq=2, Hkv=2, L=17, d=64, W=8, M=2), "f32"),
    ("fp32 L64", dict(B=1, Hq=2, Hkv=2, L=64, d=64, W=64, M=4), "f32"),
    ("fp32 L65", dict(B=1, Hq=2, Hkv=2, L=65, d=64, W=64, M=4), "f32"),
    ("bf16 gqa 4:2 shared W", dict(B=2, Hq=4, Hkv=2, L=150, d=128, W=64, M=4), "bf16"),
    ("fp32 gqa 6:2 per-head W", dict(B=1, Hq=6, Hkv=2, L=140, d=64, W=32, M=4, per_head_w=True,
                                     separate_wk=True), "f32"),
    ("bf16 separate W, W128 (value/key tiles past the LDS rings)", dict(B=1, Hq=2, Hkv=2, L=300, d=128,
                                                                      W=128, M=8, gate="uniform",
                                                                      separate_wk=True), "bf16"),
    ("bf16 per-head W G1", dict(B=1, Hq=2, Hkv=2, L=100, d=128, W=64, M=4, per_head_w=True,
                                separate_wk=True), "bf16"),
]


@pytest.mark.parametrize("label,kw,dtype", SMALL, ids=[s[0] for s in SMALL])
def test_fwd_matches_oracle(gpu_lib, label, kw, dtype):
    if kw is None:
        inp = workload_fwd_inputs(0)
    else:
        inp = make_fwd_inputs(dtype=dtype, seed=zlib.crc32(label.encode()) % 10000, **kw)
    check_case(label, inp, dtype)


@pytest.mark.parametrize("W", [64, 100])
@pytest.mark.parametrize("pattern", ["all fast", "half slow"])
def test_fwd_decayed_out_products(gpu_lib, W, pattern):
    """log gamma = -2 per token (32 per 16-token sub-chunk, sub-chunk references): the query waves
    leave out the products with key sub-chunks two or more back and the inter-chunk product, which
    have decayed below e^-16 in every feature.  With half the features at -0.01 per token instead,
    nothing may be left out (the slow features keep every product): a wrong cutoff, taken over
    the fast features only, would lose half of the global branch.  Both against the oracle per
    branch, for the narrow and the wide-window variant."""
    label = f"decayed-out {pattern} W{W}"
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=320, d=128, W=W, M=4, dtype="bf16",
                          seed=zlib.crc32(label.encode()) % 10000)
    lg = torch.full_like(inp.log_gamma, -2.0)
    if pattern == "half slow":
        lg[..., 64:] = -0.01
    check_case(label, dataclasses.replace(inp, log_gamma=lg), "bf16")


def _chunk_kinds(log_gamma, chunk=64, fast_span=60.0):
    """How many 64-token chunks have |sum log gamma| <= fast_span for every feature
    (the kernel refers their decays to the chunk start) and how many do not."""
    lg = log_gamma.double().numpy()
    L = lg.shape[2]
    mild = general = 0
    for c0 in range(0, L, chunk):
        tot = lg[:, :, c0:c0 + chunk, :].sum(axis=2)  # [B, H, d]
        m = (-tot).max(axis=-1)
        mild += int((m <= fast_span).sum())
        general += int((m > fast_span).sum())
    return mild, general


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_fwd_mixed_chunk_references(gpu_lib, dtype, d):
    """A gate whose chunk totals straddle the chunk-start reference bound, so one launch
    takes both the chunk-start and the sub-chunk decay references."""
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=640, d=d, W=64, M=4, dtype=dtype, seed=77,
                          gate="uniform:-1.6")
    mild, general = _chunk_kinds(inp.log_gamma)
    _say(f"      chunks: {mild} mild, {general} general")
    assert mild > 0 and general > 0
    check_case(f"{dtype} d{d} mixed chunk references", inp, dtype)


@pytest.mark.parametrize("label", ["bf16 d128 ragged L200", "bf16 gqa 4:2 shared W", "fp32 uniform gate -8 (mixed safe/exact diag)",
                                   "fp32 W66 (3-chunk ring)"])
def test_fwd_four_wave_kernel(gpu_lib, lz_opts, label):
    """The 4-wave kernel (used for grouped heads and the segment state pass) on single-head
    cases as well."""
    lz_opts("fwd_kernel", 2)
    kw, dtype = {s[0]: (s[1], s[2]) for s in SMALL}[label]
    inp = make_fwd_inputs(dtype=dtype, seed=zlib.crc32(label.encode()) % 10000, **kw)
    check_case(label + " [4-wave]", inp, dtype)


@pytest.mark.parametrize("nseg", [2, 3, 5])
def test_fwd_sequence_segments(gpu_lib, lz_opts, nseg):
    """Segments joined through the workspace states give the same answer."""
    lz_opts("fwd_segments", nseg)
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=330, d=64, W=70, M=4, dtype="f32", seed=31,
                          gate="uniform:-1")
    check_case(f"fp32 {nseg} segments", inp, "f32")
    inp = make_fwd_inputs(B=1, Hq=4, Hkv=2, L=300, d=128, W=64, M=4, dtype="bf16", seed=32)
    check_case(f"bf16 gqa {nseg} segments", inp, "bf16")


@pytest.mark.parametrize("nseg", [1, 2, 3, 5])
def test_fwd_whole_head_segments(gpu_lib, lz_opts, nseg):
    """The whole-head kernel (bf16, d = 128, one W_phi for queries and keys) over
    sequence segments joined through its state pass: a gate that mixes both decay
    references with a ragged tail, and gamma = 0 (exact diagonal blocks from the fixup
    kernel) across segment boundaries."""
    lz_opts("fwd_segments", nseg)
    inp = make_fwd_inputs(B=1, Hq=2, Hkv=2, L=650, d=128, W=65, M=16, dtype="bf16", seed=90 + nseg,
                          gate="uniform:-1.6")
    check_case(f"bf16 whole-head {nseg} segments, mixed references", inp, "bf16")
    inp = make_fwd_inputs(B=2, Hq=1, Hkv=1, L=300, d=128, W=64, M=4, dtype="bf16", seed=95 + nseg, gate="zero")
    check_case(f"bf16 whole-head {nseg} segments, gamma=0", inp, "bf16")


WIDE = [
    ("W66 M1 ragged, mixed references", dict(B=1, Hq=2, Hkv=2, L=300, d=128, W=66, M=1, gate="uniform:-1.6"), 1),
    ("W100 M8 gqa 4:2", dict(B=2, Hq=4, Hkv=2, L=400, d=128, W=100, M=8), 1),
    ("W128 M8 uniform gate, 3 segments", dict(B=1, Hq=2, Hkv=2, L=650, d=128, W=128, M=8, gate="uniform"), 3),
    ("W129 M16 ragged, 2 segments", dict(B=2, Hq=1, Hkv=1, L=201, d=128, W=129, M=16), 2),
    ("W128 M0 L100 (full causal softmax)", dict(B=1, Hq=2, Hkv=2, L=100, d=128, W=128, M=0), 1),
    ("W128 gamma=0 (exact diag)", dict(B=1, Hq=2, Hkv=2, L=260, d=128, W=128, M=4, gate="zero"), 2),
]


@pytest.mark.parametrize("label,kw,nseg", WIDE, ids=[c[0] for c in WIDE])
def test_fwd_whole_head_wide_window(gpu_lib, lz_opts, label, kw, nseg):
    """The whole-head kernel with windows of 66..129 keys: the window reaches into the chunk
    two back (computed one chunk early and carried), with segments and grouped heads."""
    lz_opts("fwd_segments", nseg)
    inp = make_fwd_inputs(dtype="bf16", seed=zlib.crc32(label.encode()) % 10000, **kw)
    check_case(f"bf16 whole-head {label}", inp, "bf16")


@pytest.mark.parametrize("gate", ["one", "const:-0.1", "const:-0.5", "logsigmoid"])
def test_fwd_whole_head_state_pass_drops_decayed_chunks(gpu_lib, lz_opts, gate):
    """The state pass leaves out the chunks of a segment that reach its end decayed below
    e^-24 in every feature (with -0.1 per token: all but the last 4 of 13 chunks; -0.5: all but
    the last one), and splits the rest over its pieces; gamma = 1 keeps everything."""
    lz_opts("fwd_segments", 2)
    lz_opts("fwd_split_shift", -1)  # the state pass, not the self-started split
    inp = make_fwd_inputs(B=2, Hq=2, Hkv=2, L=1600, d=128, W=64, M=4, dtype="bf16",
                          seed=zlib.crc32(gate.encode()) % 10000, gate=gate)
    check_case(f"bf16 whole-head 2 segments, gate {gate}", inp, "bf16")


@pytest.mark.parametrize("shift", [None, "-1", "0", "2", "100"])
def test_fwd_whole_head_two_segment_split(gpu_lib, lz_opts, shift):
    """Two segments on the whole-head path: the second one's workgroups walk the chunks before
    its start themselves (no state pass), and the first takes `shift` chunks beyond the even
    split (None: estimated from the gates in the kernel; 100 is capped at a quarter segment;
    -1: the state pass instead).  Gates with long, short and no decay, a ragged tail, GQA."""
    lz_opts("fwd_segments", 2)
    if shift is None:
        lz_opts("fwd_split_shift", SHIFT_AUTO)
    else:
        lz_opts("fwd_split_shift", int(shift))
    for gate, kw in (("logsigmoid", dict(B=1, Hq=4, Hkv=2, L=1650)), ("uniform:-1.6", dict(B=2, Hq=1, Hkv=1, L=900)),
                     ("one", dict(B=1, Hq=2, Hkv=2, L=1000))):
        inp = make_fwd_inputs(d=128, W=64, M=4, dtype="bf16", seed=zlib.crc32(f"{gate}{shift}".encode()) % 10000,
                              gate=gate, **kw)
        check_case(f"bf16 whole-head 2 segments, shift {shift}, gate {gate}", inp, "bf16")


@pytest.mark.parametrize("L", [65, 100, 129, 190])
def test_fwd_whole_head_two_segment_split_short(gpu_lib, lz_opts, L):
    """Two self-started segments on 2-3 chunks: a one-chunk walk, a ragged last chunk, a last
    segment of one token (L = 129), and no room for a shift."""
    lz_opts("fwd_segments", 2)
    lz_opts("fwd_split_shift", SHIFT_AUTO)
    for gate in ("logsigmoid", "one"):
        inp = make_fwd_inputs(B=2, Hq=2, Hkv=1, L=L, d=128, W=64, M=4, dtype="bf16", seed=L, gate=gate)
        check_case(f"bf16 whole-head 2 segments, L={L}, gate {gate}", inp, "bf16")


@pytest.mark.parametrize("label", ["bf16 d128 ragged L200", "bf16 gamma=0 (exact diag)", "bf16 gamma=1"])
def test_fwd_value_block_kernel(gpu_lib, lz_opts, label):
    """The value-block (role-split) kernel on cases the whole-head kernel would otherwise take
    (it still serves separate or per-head W_phi and grouped heads)."""
    lz_opts("fwd_kernel", 1)
    kw, dtype = {s[0]: (s[1], s[2]) for s in SMALL}[label]
    inp = make_fwd_inputs(dtype=dtype, seed=zlib.crc32(label.encode()) % 10000, **kw)
    check_case(label + " [value blocks]", inp, dtype)


def _sampled_check(index, heads, label):
    inp = workload_fwd_inputs(index)
    dtype = "bf16"
    _say(f"[fwd] {label}: full size, shapes q{tuple(inp.q.shape)} k{tuple(inp.k.shape)}")
    dev = inp.to("cuda")
    outs = {}
    for mix in (inp.mix, 1.0, 0.0):
        outs[mix] = gpu_fwd(inp, mix, dev).cpu()
    G = inp.q.shape[1] // inp.k.shape[1]
    for (b, h) in heads:
        hk = h // G
        sl = lambda t, hh: t[b:b + 1, hh:hh + 1]
        y, yg, yw = oracle.lizard_fwd(sl(inp.q, h), sl(inp.k, hk), sl(inp.v, hk), sl(inp.log_gamma, hk),
                                      inp.w_phi_q, inp.w_phi_k, inp.t_k[hk:hk + 1], inp.t_v[hk:hk + 1],
                                      W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale, return_branches=True)
        for mix, want, name in ((inp.mix, y, "merged"), (1.0, yg, "gla"), (0.0, yw, "window")):
            got = outs[mix][b:b + 1, h:h + 1].double().numpy()
            e = float(rel_l2_per_head(got, want).max())
            _say(f"      (b={b}, h={h}) {name}: rel-L2 {e:.3e}")
            assert e <= TOL[dtype], f"{label} (b={b},h={h}) {name}: {e:.3e}"
    return outs


def test_fwd_workload1_full_size_sampled_heads(gpu_lib):
    outs = _sampled_check(1, [(0, 0), (3, 31), (2, 17)], "llama3-8b layer")
    # run-to-run determinism at full size (no atomics in the forward)
    inp = workload_fwd_inputs(1)
    again = gpu_fwd(inp, inp.mix).cpu()
    assert torch.equal(again, outs[inp.mix]), "forward is not bitwise reproducible"


def test_fwd_workload2_full_size_sampled_heads(gpu_lib):
    _sampled_check(2, [(0, 5), (0, 30)], "32K stress")


def test_fwd_workload4_full_size_sampled_heads(gpu_lib):
    _sampled_check(4, [(0, 0), (1, 13), (1, 31)], "gqa 32/8")
