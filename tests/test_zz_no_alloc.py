"""lizard_attn_decode_noalloc (the decode step with the library's static per-GPU scratch instead
of a caller workspace) against lizard_attn_decode on the same inputs: two calls in a row, the
second with fewer sequences, so the second call runs on scratch the first one left behind.  Both
entry points run the same kernels, so outputs, states, rings and positions must agree exactly
(well inside the 2e-2 relative L2 allowed for bf16)."""
import sys

import numpy as np
import pytest
import torch

from linearized_attention_amd import api
from linearized_attention_amd.synthetic import make_decode_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(dec, fn, **kw):
    st = dec.state.clone().cuda()
    rk, rv, pos = dec.ring_k.clone().cuda(), dec.ring_v.clone().cuda(), dec.pos.clone().cuda()
    w = [t.cuda() for t in (dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v)]
    outs = []
    for (q, k, v, lg) in dec.steps:
        outs.append(fn(st, rk, rv, pos, q.cuda(), k.cuda(), v.cuda(), lg.cuda(), *w, M=dec.M, mix=dec.mix,
                       scale=dec.scale, **kw).cpu())
    torch.cuda.synchronize()
    return torch.stack(outs), st.cpu(), rk.cpu(), rv.cpu(), pos.cpu()


def test_decode_noalloc_matches_decode_on_two_calls(gpu_lib):
    for i, (N, Hq, Hkv) in enumerate(((48, 8, 4), (20, 4, 4))):
        dec = make_decode_inputs(N=N, Hq=Hq, Hkv=Hkv, d=128, W=64, M=4, steps=2, pos0=90 + i, dtype="bf16",
                                 seed=700 + i)
        _say(f"[decode noalloc] call {i + 1}: N={N} Hq={Hq} Hkv={Hkv} d=128 W=64 M=4, 2 steps")
        want = _run(dec, api.lizard_attn_decode)
        got = _run(dec, api.lizard_attn_decode_noalloc)
        for name, a, b in zip(("out", "state", "ring_k", "ring_v", "pos"), got, want):
            assert torch.equal(a, b), f"call {i + 1}: {name} differs from lizard_attn_decode"
        o, r = got[0].double().numpy(), want[0].double().numpy()
        rel = np.sqrt(((o - r) ** 2).sum() / (r ** 2).sum())
        assert rel <= 2e-2
        _say(f"      equal to lizard_attn_decode (outputs, state, rings, pos)")


def test_decode_noalloc_rejects_shapes_beyond_its_scratch(gpu_lib):
    """N * Hkv * (1 + G) * d floats plus N counters must fit the 32 MiB scratch; a larger step is
    refused before anything is launched, and the state is left untouched."""
    dec = make_decode_inputs(N=2, Hq=2, Hkv=2, d=128, W=64, M=4, steps=1, pos0=5, dtype="bf16", seed=9)
    st = dec.state.clone().cuda()
    before = st.clone()
    # 4100 sequences x 8 heads x 2 x 128 floats = 8.4e6 > 32 MiB / 4
    N = 4100
    big = [torch.zeros(N, 8, 128, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    state = torch.zeros(N, 8, 128, 128, dtype=torch.float32, device="cuda")
    ring = torch.zeros(N, 8, 64, 128, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(N, dtype=torch.int32, device="cuda")
    w = [t.cuda() for t in (dec.w_phi_q, dec.w_phi_k)]
    tk = torch.zeros(8, 4, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.LizardError) as ei:
        api.lizard_attn_decode_noalloc(state, ring, ring.clone(), pos, *big, *w, tk, tk.clone(), M=4)
    assert ei.value.status == 2 and "static" in ei.value.detail
    torch.cuda.synchronize()
    assert int(pos.abs().sum()) == 0 and torch.equal(st, before)
