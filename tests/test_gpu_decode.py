"""Parity of the HIP decode step with the fp64 oracle, and decode-vs-forward
equivalence.  Relative L2 per head over all (sequence, step, d) outputs:
<= 1e-4 for fp32 inputs, <= 2e-2 for bf16; the fp32 state is compared too."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linearized_attention_amd import api
from linearized_attention_amd.synthetic import make_decode_inputs, make_fwd_inputs, workload_decode_inputs

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, want, axes):
    num = np.sqrt(((got - want) ** 2).sum(axis=axes))
    den = np.sqrt((want ** 2).sum(axis=axes))
    return num / np.maximum(den, 1e-300)


def run_gpu_steps(dec, nsteps=None, shared_workspace=False):
    ws = None
    if shared_workspace:
        N, Hq, d = dec.steps[0][0].shape
        nb = api.lizard_attn_decode_workspace_bytes(N, Hq, dec.steps[0][1].shape[1], d, dec.steps[0][0].dtype)
        ws = torch.full((nb,), 255, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    st = dec.state.clone().cuda()
    rk, rv, pos = dec.ring_k.clone().cuda(), dec.ring_v.clone().cuda(), dec.pos.clone().cuda()
    args = [t.cuda() for t in (dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v)]
    outs = []
    for (q, k, v, lg) in dec.steps[:nsteps]:
        o = api.lizard_attn_decode(st, rk, rv, pos, q.cuda(), k.cuda(), v.cuda(), lg.cuda(), *args,
                                   M=dec.M, mix=dec.mix, scale=dec.scale, workspace=ws)
        outs.append(o.double().cpu().numpy())
    torch.cuda.synchronize()
    return np.stack(outs, axis=2), st.double().cpu().numpy(), rk.cpu(), rv.cpu(), pos.cpu()


def run_oracle_steps(dec, nsteps=None, seqs=None):
    sel = (lambda t: t) if seqs is None else (lambda t: t[seqs])
    st, rk, rv, pos = sel(dec.state), sel(dec.ring_k), sel(dec.ring_v), sel(dec.pos)
    outs = []
    for (q, k, v, lg) in dec.steps[:nsteps]:
        out, st, rk, rv, pos = oracle.lizard_decode(st, rk, rv, pos, sel(q), sel(k), sel(v), sel(lg),
                                                    dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v, M=dec.M,
                                                    mix=dec.mix, scale=dec.scale)
        outs.append(out)
    return np.stack(outs, axis=2), st, rk, rv, pos


CASES = [
    ("bf16 d128 pos0=100", dict(N=6, Hq=3, Hkv=3, d=128, W=64, M=4, steps=3, pos0=100, dtype="bf16"), "bf16"),
    ("fp32 d64 gqa from empty", dict(N=5, Hq=4, Hkv=2, d=64, W=16, M=2, steps=40, pos0=0, dtype="f32",
                                     zero_state=True), "f32"),
    ("fp32 d64 pos0=3 W7 M0", dict(N=3, Hq=2, Hkv=2, d=64, W=7, M=0, steps=9, pos0=3, dtype="f32"), "f32"),
    ("bf16 d64 gqa 8:2 W100", dict(N=9, Hq=8, Hkv=2, d=64, W=100, M=16, steps=4, pos0=250, dtype="bf16"), "bf16"),
    ("bf16 d128 gqa 6:1 (three head passes)", dict(N=4, Hq=6, Hkv=1, d=128, W=64, M=4, steps=3, pos0=64,
                                                    dtype="bf16"), "bf16"),
    ("bf16 d128 gqa 3:1 (a partial head pass)", dict(N=5, Hq=3, Hkv=1, d=128, W=64, M=4, steps=3, pos0=20,
                                                     dtype="bf16"), "bf16"),
    ("bf16 d128 W256 M16 (four logits passes)", dict(N=3, Hq=2, Hkv=2, d=128, W=256, M=16, steps=3, pos0=300,
                                                      dtype="bf16"), "bf16"),
]


@pytest.mark.parametrize("label,kw,dtype", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(gpu_lib, label, kw, dtype):
    _say(f"[decode] {label}")
    dec = make_decode_inputs(seed=17, **kw)
    yg, sg, rkg, rvg, pg = run_gpu_steps(dec)
    yo, so, rko, rvo, po = run_oracle_steps(dec)
    err = rel_l2(yg, yo, axes=(0, 2, 3)).max()
    serr = rel_l2(sg, so, axes=(0, 2, 3)).max()
    _say(f"      out rel-L2 {err:.3e}   state rel-L2 {serr:.3e}")
    assert err <= TOL[dtype]
    assert serr <= TOL[dtype]
    assert np.array_equal(pg.numpy(), po)
    # the rings hold exactly the input keys/values (bit-exact copies)
    assert np.array_equal(rkg.double().numpy(), rko)
    assert np.array_equal(rvg.double().numpy(), rvo)


def test_decode_shared_workspace_is_deterministic(gpu_lib):
    """One workspace reused (with stale contents) across steps gives the same
    bits as a fresh workspace per call."""
    _say("[decode] shared workspace vs per-call workspace")
    dec = make_decode_inputs(seed=5, N=7, Hq=8, Hkv=2, d=128, W=64, M=4, steps=4, pos0=30, dtype="bf16")
    a = run_gpu_steps(dec)
    b = run_gpu_steps(dec, shared_workspace=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_from_empty_equals_gpu_forward(gpu_lib, dtype, d):
    """L decode steps from S = 0, pos = 0 reproduce the forward on the same tokens."""
    L, H, W, M = 70, 2, 64, 4
    _say(f"[decode] decode==forward {dtype} d={d} L={L}")
    dec = make_decode_inputs(N=2, Hq=H, Hkv=H, d=d, W=W, M=M, steps=L, pos0=0, dtype=dtype, seed=23,
                             zero_state=True)
    yd, sd, _, _, _ = run_gpu_steps(dec)
    stack = lambda i: torch.stack([s[i] for s in dec.steps], dim=2).contiguous()
    q, k, v, lg = (stack(i).cuda() for i in range(4))
    yf = api.lizard_attn_fwd(q, k, v, lg, dec.w_phi_q.cuda(), dec.w_phi_k.cuda(), dec.t_k.cuda(),
                             dec.t_v.cuda(), W=W, M=M, mix=dec.mix, scale=dec.scale)
    yf = yf.double().cpu().numpy()
    yo, so = oracle.lizard_fwd(stack(0), stack(1), stack(2), stack(3), dec.w_phi_q, dec.w_phi_k, dec.t_k,
                               dec.t_v, W=W, M=M, mix=dec.mix, scale=dec.scale, return_state=True)
    e_df = rel_l2(yd, yf, axes=(2, 3)).max()
    e_do = rel_l2(yd, yo, axes=(2, 3)).max()
    e_fo = rel_l2(yf, yo, axes=(2, 3)).max()
    e_s = rel_l2(sd, so, axes=(2, 3)).max()
    _say(f"      decode~fwd {e_df:.3e}  decode~oracle {e_do:.3e}  fwd~oracle {e_fo:.3e}  state {e_s:.3e}")
    for e in (e_df, e_do, e_fo, e_s):
        assert e <= TOL[dtype]


def test_decode_workload3_full_size_sampled(gpu_lib):
    """N=256, H=32, d=128: two steps on the GPU; eight sequences checked in fp64."""
    _say("[decode] workload 3 full size, 2 steps")
    dec = workload_decode_inputs(3, steps=2)
    yg, sg, _, _, pg = run_gpu_steps(dec)
    seqs = np.array([0, 1, 77, 128, 200, 254, 255, 31])
    yo, so, _, _, po = run_oracle_steps(dec, seqs=torch.from_numpy(seqs))
    err = rel_l2(yg[seqs], yo, axes=(0, 2, 3)).max()
    serr = rel_l2(sg[seqs], so, axes=(0, 2, 3)).max()
    _say(f"      out rel-L2 {err:.3e}  state rel-L2 {serr:.3e}")
    assert err <= TOL["bf16"] and serr <= TOL["bf16"]
    assert (pg.numpy() == 4098).all()


def test_decode_workload3_128_steps_sampled(gpu_lib):
    """The benchmark's decode run: N=256 sequences, H=32, d=128, 128 consecutive steps on the
    GPU from the seeded start (pos 4096); six sequences followed through all 128 steps in fp64,
    every step's output and the final state compared."""
    _say("[decode] workload 3 full size, 128 consecutive steps")
    dec = workload_decode_inputs(3, steps=128)
    yg, sg, rkg, _, pg = run_gpu_steps(dec)
    seqs = np.array([0, 5, 99, 160, 223, 255])
    yo, so, rko, _, po = run_oracle_steps(dec, seqs=torch.from_numpy(seqs))
    err = rel_l2(yg[seqs], yo, axes=(0, 2, 3)).max()
    serr = rel_l2(sg[seqs], so, axes=(0, 2, 3)).max()
    _say(f"      out rel-L2 (per head, all 128 steps) {err:.3e}  final state rel-L2 {serr:.3e}")
    assert err <= TOL["bf16"] and serr <= TOL["bf16"]
    assert (pg.numpy() == 4096 + 128).all()
    assert torch.equal(rkg[torch.from_numpy(seqs)], torch.from_numpy(np.asarray(rko)).to(rkg.dtype))


@pytest.mark.parametrize("fmap", ["softmax", "hedgehog"])
def test_decode_steps_captured_in_a_graph_match_eager(gpu_lib, fmap):
    """Consecutive decode steps captured once in a HIP graph (as a serving loop would run them)
    and replayed three times, the buffers restored by eager copies between replays: every replay
    gives the eager steps' outputs, state, ring and positions bit for bit."""
    hh = fmap == "hedgehog"
    dec = make_decode_inputs(N=8, Hq=4, Hkv=2, d=128, W=64, M=4, steps=6, pos0=60, dtype="bf16", seed=23,
                             phi_cols=64 if hh else None)
    fn = api.lizard_attn_decode_hedgehog if hh else api.lizard_attn_decode
    w = [t.cuda() for t in (dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v)]
    xs = [tuple(t.cuda() for t in s) for s in dec.steps]
    init = [t.clone().cuda() for t in (dec.state, dec.ring_k, dec.ring_v, dec.pos)]
    N, Hq, d = xs[0][0].shape
    nb = api.lizard_attn_decode_workspace_bytes(N, Hq, xs[0][1].shape[1], d, xs[0][0].dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    bufs = [t.clone() for t in init]
    outs = [torch.empty_like(x[0]) for x in xs]

    def steps():
        for (q, k, v, lg), o in zip(xs, outs):
            fn(*bufs, q, k, v, lg, *w, M=dec.M, mix=dec.mix, scale=dec.scale, out=o, workspace=ws)

    steps()  # eager
    torch.cuda.synchronize()
    want = [t.clone() for t in outs + bufs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    for rep in range(3):
        for b, i in zip(bufs, init):
            b.copy_(i)
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs + bufs
        for name, g, e in zip([f"out{s}" for s in range(len(outs))] + ["state", "ring_k", "ring_v", "pos"], got, want):
            assert torch.equal(g, e), f"replay {rep}: {name} differs from the eager steps"
    _say(f"[decode graph, {fmap}] {len(xs)} steps captured, 3 replays equal to eager")
