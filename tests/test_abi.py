"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and host-side validation returns the documented status codes
without launching anything."""
import ctypes
import os
import re

import pytest

from linearized_attention_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lizard_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lizard_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in api.EXPORTED:
        assert n in names
    assert set(names) == set(api.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(api.LIB_PATH) if os.path.exists(api.LIB_PATH) else api.load()
    for n in _declared():
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings_and_version():
    lib = api.load()
    for code in range(5):
        assert lib.lizard_status_string(code)
    assert b"gfx950" in lib.lizard_version()


def _fwd(lib, fn="lizard_attn_fwd", **kw):
    a = dict(q=16, k=16, v=16, lg=16, wq=16, wk=16, stride=0, tk=16, tv=16, out=16, B=1, Hq=2, Hkv=2,
             L=64, d=128, W=64, M=4, mix=0.5, scale=0.1, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, fn)(P(a["q"]), P(a["k"]), P(a["v"]), P(a["lg"]), P(a["wq"]), P(a["wk"]),
                               a["stride"], P(a["tk"]), P(a["tv"]), P(a["out"]), a["B"], a["Hq"],
                               a["Hkv"], a["L"], a["d"], a["W"], a["M"], a["mix"], a["scale"],
                               a["dtype"], P(a["ws"]), a["wsb"], P(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(Hq=3, Hkv=2), 1), (dict(Hkv=0), 1),
    (dict(W=0), 1), (dict(M=-1), 1), (dict(L=-5), 1), (dict(dtype=7), 1),
    (dict(q=24), 1),                       # misaligned
    (dict(stride=-1), 1), (dict(stride=100), 1), (dict(stride=128 * 128 + 4), 1),  # misaligned matrices
    (dict(d=96), 2), (dict(d=128, dtype=0), 2), (dict(M=17), 2),
    (dict(tk=None), 1),
    (dict(mix=-0.25), 1), (dict(mix=float("nan")), 1), (dict(mix=float("inf")), 1),
    (dict(scale=float("nan")), 1), (dict(mix=-0.25, B=0), 1),   # checked before the empty case
])
def test_fwd_validation_codes(kw, code):
    lib = api.load()
    assert _fwd(lib, **kw) == code
    assert lib.lizard_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(Hq=3, Hkv=2), 1), (dict(stride=100), 1),
    (dict(stride=128 * 64 - 1), 1),                          # overlaps matrices of d x d/2 elements
    (dict(stride=128 * 64 + 4), 1),                          # matrices off 16-byte alignment
    (dict(d=64), 2), (dict(d=64, dtype=0), 2),            # only bf16, d = 128
    (dict(W=130), 2),                                       # windows of at most 129 keys
])
def test_fwd_hedgehog_validation_codes(kw, code):
    lib = api.load()
    assert _fwd(lib, fn="lizard_attn_fwd_hedgehog", **kw) == code
    assert lib.lizard_last_error()


def test_fwd_hedgehog_empty_problem_is_ok():
    lib = api.load()
    assert _fwd(lib, fn="lizard_attn_fwd_hedgehog", B=0) == 0


def test_fwd_empty_problem_is_ok_without_launch():
    lib = api.load()
    assert _fwd(lib, B=0) == 0
    assert _fwd(lib, L=0) == 0
    assert _fwd(lib, B=0, q=None, k=None) == 0


def test_fwd_workspace_required_when_segmented():
    lib = api.load()
    need = lib.lizard_attn_fwd_workspace_bytes(1, 32, 32, 32768, 128, 128, 1)
    assert need > 0
    assert _fwd(lib, B=1, Hq=32, Hkv=32, L=32768, ws=None) == 3
    # the size covers a separate query-side W_phi (its fragment-ordered copy): one byte less fails
    assert _fwd(lib, B=1, Hq=32, Hkv=32, L=32768, wk=32, ws=4096, wsb=need - 1) == 3
    # one chunk: nothing to split; only the query-side W_phi copy (d x d bf16 per query head),
    # which a shared W_phi does not use
    assert lib.lizard_attn_fwd_workspace_bytes(1, 2, 2, 64, 128, 64, 1) == 2 * 128 * 128 * 2
    assert _fwd(lib, L=64, wk=32, ws=None) == 3
    assert _fwd(lib, L=64, wk=32, ws=4096, wsb=2 * 128 * 128 * 2 - 1) == 3


def test_workspace_bytes_matches_plan_formula():
    lib = api.load()
    B, Hkv, L, d = 1, 32, 32768, 128
    got = lib.lizard_attn_fwd_workspace_bytes(B, Hkv, Hkv, L, d, 128, 1)
    # value-block plan: B*Hkv*ndvb = 64 groups -> 4 segments of 128 chunks, end states per
    # 64-column block
    nseg = 4
    split = B * Hkv * 2 * (nseg - 1) * d * 64 * 4 + B * Hkv * (nseg - 1) * d * 4
    # whole-head plan (bf16, d = 128, W <= 129): B*Hq = 32 blocks -> 8 segments of 64 chunks;
    # the state pass in max(1, 256 // (32 * 7)) = 1 piece per segment, full d x d states
    nseg, sss = 8, 1
    pieces = B * Hkv * (nseg - 1) * sss
    full = pieces * d * d * 4 + -(-pieces * d * 4 // 256) * 256
    # then one fragment-ordered W_phi_q^T copy (d x d bf16) per query head, 256-byte aligned
    full = -(-full // 256) * 256 + Hkv * d * d * 2
    assert got == max(split, full)


def test_whole_head_segments_cover_at_most_1024_chunks():
    """The whole-head kernel keeps one LDS flag bit per chunk of its segment (1024 at most): a
    sequence of 2048 chunks over 256 (batch, head) pairs, which would otherwise run as one
    segment, is split in two and needs the state-pass workspace; 1024 chunks need none (beyond
    the query-side W_phi copies that every whole-head call's size covers)."""
    lib = api.load()
    wq_copies = 32 * 128 * 128 * 2  # one W_phi_q^T copy per query head (separate W_phi only)
    assert lib.lizard_attn_fwd_workspace_bytes(8, 32, 32, 1024 * 64, 128, 64, 1) == wq_copies
    need = lib.lizard_attn_fwd_workspace_bytes(8, 32, 32, 2048 * 64, 128, 64, 1)
    pieces = 8 * 32 * 1 * 1  # B*Hkv*(nseg - 1)*sss with nseg = 2, sss = 256 // 256
    assert need == pieces * 128 * 128 * 4 + pieces * 128 * 4 + wq_copies


def _dec(lib, fn="lizard_attn_decode", **kw):
    a = dict(state=16, wk=16, wv=16, pos=16, q=16, k=16, v=16, lg=16, wq=16, wkm=16, stride=0, tk=16,
             tv=16, out=16, N=4, Hq=2, Hkv=2, d=128, W=64, M=4, mix=0.5, scale=0.1, dtype=1, ws=16,
             wsb=1 << 30, stream=None)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, fn)(P(a["state"]), P(a["wk"]), P(a["wv"]), P(a["pos"]), P(a["q"]),
                                  P(a["k"]), P(a["v"]), P(a["lg"]), P(a["wq"]), P(a["wkm"]),
                                  a["stride"], P(a["tk"]), P(a["tv"]), P(a["out"]), a["N"], a["Hq"],
                                  a["Hkv"], a["d"], a["W"], a["M"], a["mix"], a["scale"], a["dtype"],
                                  P(a["ws"]), a["wsb"], P(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), 1), (dict(pos=None), 1), (dict(Hq=3), 1), (dict(W=0), 1), (dict(N=-1), 1),
    (dict(d=32), 2), (dict(W=257), 2), (dict(M=20), 2), (dict(q=8), 1), (dict(pos=18), 1),
    (dict(ws=None), 3), (dict(wsb=100), 3), (dict(ws=24), 1),
    (dict(mix=-1.0), 1), (dict(mix=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(stride=128 * 128 + 2), 1),                        # matrices off 16-byte alignment
])
def test_decode_validation_codes(kw, code):
    lib = api.load()
    assert _dec(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), 1), (dict(d=32), 2), (dict(W=257), 2), (dict(ws=None), 3),
    (dict(stride=128 * 64 - 1), 1),                         # W_phi [d, d/2]: d*d/2 elements apart
])
def test_decode_hedgehog_validation_codes(kw, code):
    assert _dec(api.load(), fn="lizard_attn_decode_hedgehog", **kw) == code


def test_decode_empty_is_ok():
    assert _dec(api.load(), N=0) == 0


def test_decode_workspace_bytes_formula():
    lib = api.load()
    N, Hq, Hkv, d = 256, 32, 8, 128
    G = Hq // Hkv
    assert lib.lizard_attn_decode_workspace_bytes(N, Hq, Hkv, d, 1) == 4 * (N * Hkv * (1 + G) * d + N)
    assert lib.lizard_attn_decode_workspace_bytes(0, Hq, Hkv, d, 1) == 0
    assert lib.lizard_attn_decode_workspace_bytes(N, 3, 2, d, 1) == 0
    need = lib.lizard_attn_decode_workspace_bytes(4, 2, 2, 128, 1)
    assert _dec(lib, wsb=need - 1) == 3


def _fwd_ext(lib, **kw):
    a = dict(q=16, k=16, v=16, lg=16, wq=16, wk=16, stride=0, tk=16, tv=16, out=16, B=1, Hq=2, Hkv=2,
             L=64, d=128, W=64, M=4, mix=0.5, scale=0.1, dtype=1, sin=None, rkin=None, rvin=None, pos=None,
             sout=None, rkout=None, rvout=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.lizard_attn_fwd_ext(P(a["q"]), P(a["k"]), P(a["v"]), P(a["lg"]), P(a["wq"]), P(a["wk"]),
                                   a["stride"], P(a["tk"]), P(a["tv"]), P(a["out"]), a["B"], a["Hq"],
                                   a["Hkv"], a["L"], a["d"], a["W"], a["M"], a["mix"], a["scale"],
                                   a["dtype"], P(a["sin"]), P(a["rkin"]), P(a["rvin"]), P(a["pos"]),
                                   P(a["sout"]), P(a["rkout"]), P(a["rvout"]), P(a["ws"]), a["wsb"],
                                   P(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(rkin=32, rvin=32), 1),                      # a ring in needs pos
    (dict(rkin=32, pos=64), 1),                       # keys without values
    (dict(rkout=32), 1),                              # keys out without values
    (dict(sin=48, sout=48), 1),                       # state_out must not be state_in
    (dict(pos=66), 1),                                # pos misaligned
    (dict(sout=40), 1),                               # misaligned state
    (dict(rkin=32, rvin=32, pos=64, ws=None), 3),     # history needs workspace
    (dict(d=96), 2),
])
def test_fwd_ext_validation_codes(kw, code):
    lib = api.load()
    assert _fwd_ext(lib, **kw) == code
    assert lib.lizard_last_error()


def test_fwd_ext_workspace_bytes():
    lib = api.load()
    B, Hkv, L, d, W = 2, 4, 256, 128, 100
    plain = lib.lizard_attn_fwd_workspace_bytes(B, Hkv, Hkv, L, d, W, 1)
    ext = lib.lizard_attn_fwd_ext_workspace_bytes(B, Hkv, Hkv, L, d, W, 1)
    hist = B * Hkv * 128 * d * 2            # W - 1 = 99 rows rounded up to 128, bf16
    assert ext >= plain + 2 * hist
    # (a separate query-side W_phi uses the whole size: its copy sits before the history rows)
    assert _fwd_ext(lib, B=B, Hq=Hkv, Hkv=Hkv, L=L, W=W, wk=32, rkin=32, rvin=32, pos=64, ws=4096,
                    wsb=ext - 1) == 3
    assert _fwd_ext(lib, L=0) == 0          # empty problem


def test_mix_range_accepts_zero_and_above_one():
    """mix = 0 (window only) and mix > 1 (negative window weight) pass validation: an empty
    problem returns OK without launching anything."""
    lib = api.load()
    assert _fwd(lib, mix=0.0, B=0) == 0
    assert _fwd(lib, mix=1.5, B=0) == 0
    assert _dec(lib, mix=0.0, N=0) == 0


def test_options_set_get_and_reject():
    lib = api.load()
    saved = {n: lib.lizard_get_option(n.encode()) for n in ("fwd_kernel", "fwd_segments", "fwd_split_shift")}
    try:
        assert lib.lizard_set_option(b"fwd_segments", 3) == 0
        assert lib.lizard_get_option(b"fwd_segments") == 3
        assert lib.lizard_set_option(b"fwd_kernel", 2) == 0
        assert lib.lizard_get_option(b"fwd_kernel") == 2
        assert lib.lizard_set_option(b"fwd_kernel", 3) == 1
        assert lib.lizard_set_option(b"fwd_segments", -1) == 1
        assert lib.lizard_set_option(b"no_such_option", 1) == 1
        assert lib.lizard_set_option(None, 1) == 1
        assert lib.lizard_get_option(b"no_such_option") == 0
    finally:
        for n, v in saved.items():
            assert lib.lizard_set_option(n.encode(), v) == 0


def test_segment_option_changes_the_plan():
    """A 4 x 32 x 4096 forward is planned in two segments on the whole-head path, whose state
    pass (when the second segment does not start itself) needs workspace; one forced segment
    needs none.  Both two and three segments keep 256 state-pass pieces of one 128 x 128 fp32
    state and 128 log-gate sums each.  Every size also covers the query-side W_phi copies
    (128 x 128 bf16 per query head) that a separate W_phi needs."""
    lib = api.load()
    saved = lib.lizard_get_option(b"fwd_segments")
    wq_copies = 32 * 128 * 128 * 2
    try:
        lib.lizard_set_option(b"fwd_segments", 0)
        base = lib.lizard_attn_fwd_workspace_bytes(4, 32, 32, 4096, 128, 64, 1)
        lib.lizard_set_option(b"fwd_segments", 1)
        assert lib.lizard_attn_fwd_workspace_bytes(4, 32, 32, 4096, 128, 64, 1) == wq_copies
        lib.lizard_set_option(b"fwd_segments", 3)
        more = lib.lizard_attn_fwd_workspace_bytes(4, 32, 32, 4096, 128, 64, 1)
        assert base == more == 256 * (128 * 128 * 4 + 128 * 4) + wq_copies
    finally:
        lib.lizard_set_option(b"fwd_segments", saved)


def _dec_noalloc(lib, **kw):
    a = dict(state=16, wk=16, wv=16, pos=16, q=16, k=16, v=16, lg=16, wq=16, wkm=16, stride=0, tk=16,
             tv=16, out=16, N=4, Hq=2, Hkv=2, d=128, W=64, M=4, mix=0.5, scale=0.1, dtype=1, stream=None)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.lizard_attn_decode_noalloc(P(a["state"]), P(a["wk"]), P(a["wv"]), P(a["pos"]), P(a["q"]),
                                          P(a["k"]), P(a["v"]), P(a["lg"]), P(a["wq"]), P(a["wkm"]),
                                          a["stride"], P(a["tk"]), P(a["tv"]), P(a["out"]), a["N"], a["Hq"],
                                          a["Hkv"], a["d"], a["W"], a["M"], a["mix"], a["scale"], a["dtype"],
                                          P(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), 1), (dict(Hq=3), 1), (dict(d=32), 2), (dict(W=257), 2), (dict(mix=-1.0), 1),
    (dict(N=4100, Hq=8, Hkv=8), 2),          # 4100 * 8 * 2 * 128 floats exceed the 32 MiB scratch
    (dict(N=32641, Hq=1, Hkv=1, d=128), 2),  # 4 * 32641 * (2 * 128 + 1) bytes: just over 32 MiB
])
def test_decode_noalloc_validation_codes(kw, code):
    """Host-side checks of the workspace-free decode step, all before any HIP call."""
    lib = api.load()
    assert _dec_noalloc(lib, **kw) == code
    assert lib.lizard_last_error()


def test_decode_noalloc_empty_is_ok():
    assert _dec_noalloc(api.load(), N=0) == 0


def _gla(lib, **kw):
    a = dict(q=16, k=16, v=16, lg=16, w=16, out=16, B=1, Hq=2, Hkv=2, L=64, d=128, mode=0, dtype=1, stream=None)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.lizard_gla_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["lg"]), P(a["w"]), P(a["out"]), a["B"],
                              a["Hq"], a["Hkv"], a["L"], a["d"], a["mode"], a["dtype"], P(a["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(w=None), 1), (dict(out=24), 1), (dict(Hq=3), 1), (dict(Hkv=0), 1),
    (dict(L=-1), 1), (dict(mode=2), 1), (dict(mode=-1), 1), (dict(dtype=5), 1),
    (dict(d=64), 2), (dict(dtype=0), 2),      # bf16, d = 128 only
    (dict(mode=7, B=0), 1),                   # checked before the empty case
])
def test_gla_fwd_validation_codes(kw, code):
    lib = api.load()
    assert _gla(lib, **kw) == code
    assert lib.lizard_last_error()


def test_gla_fwd_empty_is_ok():
    lib = api.load()
    assert _gla(lib, B=0) == 0
    assert _gla(lib, L=0, q=None) == 0
