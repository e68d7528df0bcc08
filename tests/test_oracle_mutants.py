"""The pins must catch plausible mistakes: build mutated copies of the oracle's
C source (on the CPU, in a temp dir), point the oracle binding at each, and
check that at least one pin fails for every mutant."""
import ctypes
import os
import subprocess

import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "lizard_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("gate after add",
     "row[e] = gam * row[e] + phk[f] * vi[e];",
     "row[e] = gam * (row[e] + phk[f] * vi[e]);"),
    ("gate of previous token",
     "const double gam = exp(gi[f]);",
     "const double gam = exp(i > 0 ? gi[f - df] : gi[f]);"),
    ("readout with phi_k",
     "for (int e = 0; e < d; ++e) yg[e] += phq[f] * row[e];",
     "for (int e = 0; e < d; ++e) yg[e] += phk[f] * row[e];"),
    ("window one key too many",
     "const int lo = i - W + 1 > 0 ? i - W + 1 : 0;",
     "const int lo = i - W > 0 ? i - W : 0;"),
    ("window excludes current token",
     "for (int j = lo; j <= i; ++j) {\n        logit[n]",
     "for (int j = lo; j < i; ++j) {\n        logit[n]"),
    ("no softmax scale",
     "logit[n] = scale * dot(qi, kh + (int64_t)j * d, d);",
     "logit[n] = dot(qi, kh + (int64_t)j * d, d);"),
    ("meta tokens dropped from normaliser",
     "zsum += logit[a];\n      }\n      for (int e = 0; e < d; ++e) yw[e] = 0.0;\n      n = 0;",
     "if (a >= M) zsum += logit[a];\n      }\n      for (int e = 0; e < d; ++e) yw[e] = 0.0;\n      n = 0;"),
    ("merge weights swapped",
     "y[o + e] = mix * yg[e] + (1.0 - mix) * yw[e];",
     "y[o + e] = (1.0 - mix) * yg[e] + mix * yw[e];"),
    ("feature map normalised wrongly",
     "for (int f = 0; f < df; ++f) phi[f] /= sum;",
     "for (int f = 0; f < df; ++f) phi[f] /= (sum + 1.0);"),
    ("gqa maps heads round-robin",
     "const int b = bh / Hq, hq = bh % Hq, hk = hq / G;",
     "const int b = bh / Hq, hq = bh % Hq, hk = hq % Hkv;"),
    ("decode writes the slot after pos",
     "const int slot = p % W;",
     "const int slot = (p + 1) % W;"),
    ("decode decays after adding",
     "S[(int64_t)f * d + e] = gam * S[(int64_t)f * d + e] + phi[f] * vt[e];",
     "S[(int64_t)f * d + e] = gam * (S[(int64_t)f * d + e] + phi[f] * vt[e]);"),
    ("decode window one slot short",
     "const int nvalid = p + 1 < W ? p + 1 : W;",
     "const int nvalid = p + 1 < W ? p + 1 : W - 1;"),
]

PIN_FUNCS = [
    pins.test_hand_worked_example,
    pins.test_gamma_one_is_causal_linear_attention,
    pins.test_gamma_zero_keeps_only_current_token,
    pins.test_per_dim_gate_brute_force_products,
    pins.test_window_covering_sequence_is_causal_softmax_attention,
    lambda: pins.test_window_with_meta_tokens_matches_masked_sdpa(3, 4),
    pins.test_mix_isolates_branches,
    pins.test_gqa_equals_repeated_heads,
    pins.test_decode_from_empty_equals_forward,
    pins.test_decode_window_reads_ring_by_position,
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, mut, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for {name!r} not found"
    msrc = src.replace(orig, mut, 1)
    cpath = tmp_path / "mut.c"
    cpath.write_text(msrc)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(cpath),
                    "-o", str(so), "-lm"], check=True)
    real = oracle._load()
    lib = ctypes.CDLL(str(so))
    for fn in ("oracle_lizard_fwd", "oracle_lizard_decode", "oracle_num_threads"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", lib)
    failures = 0
    for fn in PIN_FUNCS:
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught mutant {name!r}"


# Mutants of the Hedgehog feature map, against its own pins.
import tests.test_oracle_hedgehog as hh_pins  # noqa: E402

HH_MUTANTS = [
    ("hedgehog halves swapped",
     "phi[j] = exp(acc);\n      phi[h + j] = exp(-acc);",
     "phi[j] = exp(-acc);\n      phi[h + j] = exp(acc);"),
    ("hedgehog second half not negated",
     "phi[h + j] = exp(-acc);",
     "phi[h + j] = exp(acc);"),
    ("hedgehog weights read transposed",
     "acc += x[i] * w[(int64_t)i * h + j];",
     "acc += x[i] * w[(int64_t)j * d + i];"),
    ("hedgehog normalised like softmax",
     "phi[h + j] = exp(-acc);\n    }\n    return;",
     "phi[h + j] = exp(-acc);\n    }\n    for (int f = 0; f < df; ++f) phi[f] /= df;\n    return;"),
]

HH_PIN_FUNCS = [
    lambda: hh_pins.test_gamma_one_is_a_causal_cosh_kernel_sum(False),
    lambda: hh_pins.test_gamma_one_is_a_causal_cosh_kernel_sum(True),
    hh_pins.test_zero_weights_give_unit_features_and_a_geometric_gate,
    hh_pins.test_sign_flip_swaps_the_halves,
    hh_pins.test_gate_halves_fix_the_order_of_the_halves,
]


@pytest.mark.parametrize("name,orig,mut", HH_MUTANTS, ids=[m[0] for m in HH_MUTANTS])
def test_hedgehog_pins_catch_mutant(name, orig, mut, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for {name!r} not found"
    cpath = tmp_path / "mut.c"
    cpath.write_text(src.replace(orig, mut, 1))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(cpath),
                    "-o", str(so), "-lm"], check=True)
    real = oracle._load()
    lib = ctypes.CDLL(str(so))
    for fn in ("oracle_lizard_fwd", "oracle_lizard_decode", "oracle_num_threads"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", lib)
    failures = 0
    for fn in HH_PIN_FUNCS:
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught mutant {name!r}"


# Mutants of the backward pass, against its pins (finite differences, autograd).
import tests.test_oracle_bwd as bwd_pins  # noqa: E402

BWD_MUTANTS = [
    ("bwd gate gradient without gamma",
     "dgh[(int64_t)i * df + f] += gam * c;",
     "dgh[(int64_t)i * df + f] += c;"),
    ("bwd state gradient not decayed",
     "for (int e = 0; e < d; ++e) Gr[(int64_t)f * d + e] *= gam;",
     "for (int e = 0; e < d; ++e) Gr[(int64_t)f * d + e] *= 1.0;"),
    ("bwd query features read the previous state",
     "a += Si[(int64_t)f * d + e] * ydg[e];",
     "a += Sp[(int64_t)f * d + e] * ydg[e];"),
    ("bwd softmax map without its inner product",
     "for (int f = 0; f < df; ++f) dz[f] = phi[f] * (dphi[f] - inner);",
     "for (int f = 0; f < df; ++f) dz[f] = phi[f] * dphi[f];"),
    ("bwd window dq without the scale",
     "dqh[(int64_t)i * d + e] += scale * ds * kh[(int64_t)j * d + e];",
     "dqh[(int64_t)i * d + e] += ds * kh[(int64_t)j * d + e];"),
    ("bwd window dv without the merge weight",
     "dvh[(int64_t)j * d + e] += p[n] * (1.0 - mix) * dyi[e];",
     "dvh[(int64_t)j * d + e] += p[n] * dyi[e];"),
    ("bwd hedgehog halves added",
     "dz[j] = phi[j] * dphi[j] - phi[cols + j] * dphi[cols + j];",
     "dz[j] = phi[j] * dphi[j] + phi[cols + j] * dphi[cols + j];"),
    ("bwd weight gradient transposed",
     "dw[(int64_t)i * cols + c] += x[i] * dz[c];",
     "dw[(int64_t)c * d + i] += x[i] * dz[c];"),
    ("bwd value gradient with the query features",
     "for (int f = 0; f < df; ++f) a += Gr[(int64_t)f * d + e] * pk[f];",
     "for (int f = 0; f < df; ++f) a += Gr[(int64_t)f * d + e] * pq[f];"),
    ("bwd window ignores the meta-token mean",
     "for (int m = 0; m < M; ++m, ++n) {\n          p[n] /= zsum;\n          dp[n] = (1.0 - mix) * dot(dyi, tvh + (int64_t)m * d, d);\n          inner += p[n] * dp[n];",
     "for (int m = 0; m < M; ++m, ++n) {\n          p[n] /= zsum;\n          dp[n] = (1.0 - mix) * dot(dyi, tvh + (int64_t)m * d, d);"),
]

BWD_PIN_FUNCS = [
    lambda: bwd_pins.check_fd(*bwd_pins.FD_CASES[0]),
    lambda: bwd_pins.check_fd(*bwd_pins.FD_CASES[4]),
    lambda: bwd_pins.test_bwd_matches_autograd_of_explicit_products(*bwd_pins.AG_CASES[0]),
]


@pytest.mark.parametrize("name,orig,mut", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_pins_catch_mutant(name, orig, mut, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for {name!r} not found"
    cpath = tmp_path / "mut.c"
    cpath.write_text(src.replace(orig, mut, 1))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(cpath),
                    "-o", str(so), "-lm"], check=True)
    real = oracle._load()
    lib = ctypes.CDLL(str(so))
    for fn in ("oracle_lizard_fwd", "oracle_lizard_decode", "oracle_lizard_bwd", "oracle_num_threads"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", lib)
    failures = 0
    for fn in BWD_PIN_FUNCS:
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught mutant {name!r}"
