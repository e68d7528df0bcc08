"""Benchmark: Lizard attention forward on one MI355X (plus the decode step).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one forward pass (feature maps, chunk-local gate sums, intra- and
inter-chunk products, state scan, anchor window, merge) over the
Llama-3-8B-shaped layer: B=4, H=32, L=4096, d=128, W=64, M=4, bf16 inputs with
fp32 accumulation, seeded synthetic data.  Inputs are resident in HBM before
the timed region.

Timing.  After the W requested warm-up calls, warm-up continues until at least
CLOCK_WARMUP_MS of back-to-back forward calls have run (the GPU's clocks take
some 50-100 ms of steady work to settle); the line states the warm-up actually
run.  Then K calls are timed back to back, bracketed by two synchronisations
(`ms_per_step`, `value`).  Each of those launches is also timed on its own
with HIP events on the launch stream; `roofline.achieved` divides the
algorithmic bytes by their mean (the average launch duration, the figure a
rocprofv3 kernel trace of the same launches averages to).  A second pass of K
calls, each preceded by a 512 MB read that flushes the 256 MB MALL, is
reported beside it (`mall_flushed_launches`): across runs it came out from 1%
faster to 20% slower than the back-to-back launches, with the same spread when
the flush was replaced by an idle gap or by compute-only work, so what it
measures is the clock state after a pause, not inputs left in the MALL (the
inputs and output, 671 MB, are 2.6 times its size).

The JSON line also carries, on the same layer shape: the forward with the
Hedgehog feature map, the forward with per-head separate W_phi, the global
branch alone in its standard and reparameterized forms, and the backward pass
(each the median of per-launch HIP-event times after a clock warm-up); the
decode step (N=256 sequences, H=32, d=128, fp32 state, W=64, M=4; 128
consecutive steps captured once in a HIP graph and replayed, with the same
steps launched one by one beside it) with its own HBM roofline; and the fp64
oracle timed on the
host cores over the whole forward workload (about 1.5 s of wall time on 16
threads).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linearized_attention_amd import api  # noqa: E402
from linearized_attention_amd.synthetic import (WORKLOADS, WORKLOAD_NAMES, make_fwd_inputs,  # noqa: E402
                                                workload_decode_inputs, workload_fwd_inputs)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_full_workload1.json")
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters_fwd_full_workload{}.json")
CLOCK_WARMUP_MS = 400.0        # minimum of steady forward calls before the timed region
FLUSH_BYTES = 512 << 20        # read before each flushed launch (MALL is 256 MB)
KERNEL_SOURCES = ["linearized_attention_amd/csrc/fwd_full.hip", "linearized_attention_amd/csrc/fwd_full.hpp",
                  "linearized_attention_amd/csrc/fwd_common.hpp", "linearized_attention_amd/csrc/common.hpp",
                  "linearized_attention_amd/csrc/api.hip"]
# The forward call on this workload launches one whole-head kernel (two segments per head, the
# second walking its own start state); timings, rooflines and traffic refer to the call.
FWD_KERNEL = "fwd_full_kernel"
FWD_KERNEL_SYMBOL = "fwd_full"
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def fwd_algorithmic(c) -> tuple[float, float]:
    """Algorithmic bytes and flops of one forward over workload c.

    Bytes: q, k, v, log gamma read once and out written once (per-KV tensors
    counted once); weights and meta tokens are negligible.  Flops: per query
    token-head the query feature map 2 d d_f, intra-chunk (C+1)(d_f+d_v),
    inter-chunk read-out 2 d_f d_v and window 2 (M + W) (d + d_v); per key
    token-head (once per key/value head) the key feature map 2 d d_f and the
    state update 2 d_f d_v."""
    B, Hq, Hkv, L, d, W, M = c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["W"], c["M"]
    e = 2 if c["dtype"] == "bf16" else 4
    nbytes = e * d * (2 * B * Hq * L + 3 * B * Hkv * L)
    C = 64
    per_q = 2 * d * d + (C + 1) * (2 * d) + 2 * d * d + 2 * (M + W) * (2 * d)
    per_k = 2 * d * d + 2 * d * d
    return float(nbytes), float(per_q) * B * Hq * L + float(per_k) * B * Hkv * L


def decode_bytes_per_step(c) -> float:
    """HBM bytes of one decode step: fp32 state read+written, ring K/V read,
    the new k/v written into the ring, q/k/v/log gamma read and out written."""
    N, Hq, Hkv, d, W = c["N"], c["Hq"], c["Hkv"], c["d"], c["W"]
    e = 2
    per_kv = 2 * d * d * 4 + 2 * W * d * e + 2 * d * e + 3 * d * e
    per_q = 2 * d * e
    return float(N * (Hkv * per_kv + Hq * per_q))


def clock_warmup(fn, calls: int, min_ms: float = CLOCK_WARMUP_MS):
    """Run fn `calls` times, then on until at least min_ms of wall time of back-to-back calls
    has passed.  Returns (calls run, ms)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    for _ in range(calls):
        fn()
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def time_launches_flushed(fn, steps: int, flush: torch.Tensor):
    """Per-launch HIP-event durations of `steps` calls of fn, each after a read of the whole
    flush buffer (out of the timed interval) so that no input is left in the MALL.  A read, not
    a write: a written buffer leaves dirty lines whose write-back would fall into the timed
    launch."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        flush.sum()  # fp32 reduction: reads the buffer, writes one value
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def launch_stats(per):
    return {"median_ms": statistics.median(per), "mean_ms": sum(per) / len(per), "min_ms": min(per),
            "max_ms": max(per), "launches": len(per)}


def time_launches(fn, steps: int):
    """Time `steps` calls of fn on the current stream with HIP events: per-launch
    durations and the bracketed total."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(st)
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    t_end.record(st)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return t_start.elapsed_time(t_end), per


def bench_forward(steps: int, warmup: int, idx: int = 1, min_warm_ms: float = CLOCK_WARMUP_MS,
                  flushed: bool = True):
    c = WORKLOADS[idx]
    log("[bench] generating forward workload:", WORKLOAD_NAMES[idx])
    inp = workload_fwd_inputs(idx)
    g = inp.to("cuda")
    out = torch.empty_like(g.q)
    need = api.lizard_attn_fwd_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["W"], g.q.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def step():
        api.lizard_attn_fwd(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, g.w_phi_k, g.t_k, g.t_v, W=inp.W,
                            M=inp.M, mix=inp.mix, scale=inp.scale, out=out, workspace=ws)

    wcalls, wms = clock_warmup(step, warmup, min_warm_ms)
    log(f"[bench] forward: {wcalls} warm-up calls in {wms:.0f} ms, timing {steps} steps")
    total_ms, per = time_launches(step, steps)
    per_flushed = None
    if flushed:
        flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        per_flushed = time_launches_flushed(step, steps, flush)
        del flush
    return c, inp, total_ms, per, per_flushed, (wcalls, wms)


def bench_forward_hedgehog(steps: int, warmup: int):
    """The same layer shape with the Hedgehog feature map (W_phi [d, d/2])."""
    c = WORKLOADS[1]
    log("[bench] generating the forward workload with the Hedgehog map")
    inp = make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"], M=c["M"],
                          dtype=c["dtype"], seed=1001, gate=c["gate"], phi_cols=c["d"] // 2)
    g = inp.to("cuda")
    out = torch.empty_like(g.q)
    need = api.lizard_attn_fwd_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["W"], g.q.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def step():
        api.lizard_attn_fwd_hedgehog(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, g.w_phi_k, g.t_k, g.t_v,
                                     W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale, out=out, workspace=ws)

    wcalls, wms = clock_warmup(step, warmup)
    log(f"[bench] hedgehog forward: {wcalls} warm-up calls in {wms:.0f} ms, timing {steps} steps")
    total_ms, per = time_launches(step, steps)
    return c, total_ms, per


def bench_forward_separate_w(steps: int, warmup: int):
    """The same layer with a W_phi per query head and per key/value head (separate matrices for
    the two sides): the query feature maps come from a pass of their own."""
    c = WORKLOADS[1]
    log("[bench] generating the forward workload with per-head, separate W_phi")
    inp = make_fwd_inputs(B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], L=c["L"], d=c["d"], W=c["W"], M=c["M"],
                          dtype=c["dtype"], seed=1001, gate=c["gate"], per_head_w=True, separate_wk=True)
    g = inp.to("cuda")
    out = torch.empty_like(g.q)
    need = api.lizard_attn_fwd_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["W"], g.q.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def step():
        api.lizard_attn_fwd(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, g.w_phi_k, g.t_k, g.t_v, W=inp.W,
                            M=inp.M, mix=inp.mix, scale=inp.scale, out=out, workspace=ws)

    wcalls, wms = clock_warmup(step, warmup)
    log(f"[bench] separate-W forward: {wcalls} warm-up calls in {wms:.0f} ms, timing {steps} steps")
    total_ms, per = time_launches(step, steps)
    return total_ms, per


def bench_decode(steps: int, warmup: int):
    c = WORKLOADS[3]
    log("[bench] generating decode workload:", WORKLOAD_NAMES[3])
    dec = workload_decode_inputs(3, steps=steps)
    st = dec.state.cuda()
    rk, rv, pos = dec.ring_k.cuda(), dec.ring_v.cuda(), dec.pos.cuda()
    w = [t.cuda() for t in (dec.w_phi_q, dec.w_phi_k, dec.t_k, dec.t_v)]
    xs = [tuple(t.cuda() for t in s) for s in dec.steps]
    out = torch.empty_like(xs[0][0])
    wsb = api.lizard_attn_decode_workspace_bytes(c["N"], c["Hq"], c["Hkv"], c["d"], out.dtype)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    it = [0]

    def step():
        q, k, v, lg = xs[it[0] % len(xs)]
        it[0] += 1
        api.lizard_attn_decode(st, rk, rv, pos, q, k, v, lg, *w, M=dec.M, mix=dec.mix, scale=dec.scale,
                               out=out, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    it[0] = 0
    log(f"[bench] decode: timing {steps} consecutive steps")
    total_ms, per = time_launches(step, steps)
    # The same steps captured once in a HIP graph and replayed whole: the timing a serving loop
    # that replays its decode steps sees (no host launch work between the steps).
    graph = torch.cuda.CUDAGraph()
    it[0] = 0
    with torch.cuda.graph(graph):
        for _ in range(steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    reps = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        reps.append(a.elapsed_time(b))
    log(f"[bench] decode: graph of {steps} steps replayed in {statistics.median(reps):.3f} ms (median of 5)")
    return c, total_ms, per, reps


def bwd_algorithmic_bytes(c) -> float:
    """Algorithmic HBM bytes of one backward call: q, dy (per query head) and k, v, log gamma (per
    key/value head) read once; dq and dk, dv, dlog gamma written once.  Weights, meta tokens and
    their fp32 gradients are negligible."""
    B, Hq, Hkv, L, d = c["B"], c["Hq"], c["Hkv"], c["L"], c["d"]
    e = 2 if c["dtype"] == "bf16" else 4
    return float(e * d * L * B * (3 * Hq + 6 * Hkv))


def bench_backward(steps: int, warmup: int, idx: int = 1):
    """The backward pass over the same layer shape (dy seeded N(0, 1) in bf16)."""
    c = WORKLOADS[idx]
    log("[bench] generating the backward workload:", WORKLOAD_NAMES[idx])
    inp = workload_fwd_inputs(idx)
    g = inp.to("cuda")
    dy = torch.randn(g.q.shape, generator=torch.Generator().manual_seed(7)).to(g.q.dtype).to("cuda")
    need = api.lizard_attn_bwd_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["M"], g.q.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def step():
        api.lizard_attn_bwd(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, g.w_phi_k, g.t_k, g.t_v, dy, W=inp.W,
                            M=inp.M, mix=inp.mix, scale=inp.scale, workspace=ws)

    wcalls, wms = clock_warmup(step, warmup)
    log(f"[bench] backward: {wcalls} warm-up calls in {wms:.0f} ms, timing {steps} steps")
    total_ms, per = time_launches(step, steps)
    return c, total_ms, per, need


def bench_gla(steps: int, warmup: int, idx: int = 1):
    """The global branch alone (lizard_gla_fwd) over the same layer shape in both intra-chunk
    forms: the standard secondary-chunked one with fp32 diagonal blocks and the reparameterized
    one.  Returns per-mode (total ms, per-launch ms)."""
    c = WORKLOADS[idx]
    log("[bench] generating the GLA-only workload:", WORKLOAD_NAMES[idx])
    inp = workload_fwd_inputs(idx)
    g = inp.to("cuda")
    out = torch.empty_like(g.q)
    res = {}
    for mode in ("standard", "reparam"):
        def step(mode=mode):
            api.lizard_gla_fwd(g.q, g.k, g.v, g.log_gamma, g.w_phi_q, mode=mode, out=out)

        wcalls, wms = clock_warmup(step, warmup)
        log(f"[bench] gla {mode}: {wcalls} warm-up calls in {wms:.0f} ms, timing {steps} steps")
        res[mode] = time_launches(step, steps)
    return c, res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The fp64 oracle on the host cores over the whole forward workload (128
    heads x 4096 tokens; about 20 thread-seconds of fp64 work, 1-2 s of wall
    time on 16 threads)."""
    import oracle
    c = WORKLOADS[1]
    inp = workload_fwd_inputs(1)
    threads = oracle.num_threads()
    heads = c["B"] * c["Hq"]
    log(f"[bench] cpu baseline: oracle on the full forward workload ({heads} heads x {c['L']} tokens), "
        f"{threads} threads")
    t0 = time.perf_counter()
    oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix, scale=inp.scale)
    dt = time.perf_counter() - t0
    tokens = c["B"] * c["L"]
    return {"value": tokens / dt, "unit": "tokens/s", "cores": min(threads, heads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"the whole forward workload ({c['B']} x {c['Hq']} heads x {c['L']} tokens), fp64, "
                      f"{dt:.2f} s wall"}


def _counter_dispatches(path: str):
    """Per-dispatch values of each (kernel, counter) in a rocprofv3 counter_collection.csv
    (rows of one dispatch and counter summed over their dimensions)."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            key = (row["Kernel_Name"], row["Counter_Name"])
            d = per.setdefault(key, {})
            d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    return per


def _counter_means(path: str):
    """Per-dispatch mean of each (kernel, counter) in a rocprofv3 counter_collection.csv."""
    return {k: sum(v.values()) / len(v) for k, v in _counter_dispatches(path).items()}


def _copy_value(path: str, counter: str):
    """The counter of the largest copyBuffer dispatch: the plain copy of COPY_BYTES (input
    uploads are copies too, and much smaller)."""
    vals = [max(v.values()) for (k, c), v in _counter_dispatches(path).items() if c == counter and "copyBuffer" in k]
    if not vals:
        raise SystemExit(f"no copyBuffer dispatch for {counter}")
    return max(vals)


def _pick(means, counter, symbol, exclude=()):
    vals = [v for (k, c), v in means.items() if c == counter and symbol in k and not any(x in k for x in exclude)]
    if not vals:
        raise SystemExit(f"no kernel matching {symbol!r} for {counter}")
    return sum(vals)  # every kernel of one forward call


def write_traffic(fetch_csv: str, write_csv: str, idx: int):
    """Turn two counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) over
    `bench.py --pmc-run --workload idx` into HBM bytes per forward call.  Each
    counter is scaled by what it reads for the plain copy of COPY_BYTES in the
    same run."""
    fetch, write = _counter_means(fetch_csv), _counter_means(write_csv)
    kf, kw = _pick(fetch, "FETCH_SIZE", FWD_KERNEL_SYMBOL), _pick(write, "WRITE_SIZE", FWD_KERNEL_SYMBOL)
    cf, cw = _copy_value(fetch_csv, "FETCH_SIZE"), _copy_value(write_csv, "WRITE_SIZE")
    sf, sw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    c = WORKLOADS[idx]
    nbytes, _ = fwd_algorithmic(c)
    traffic = kf * 1024.0 * sf + kw * 1024.0 * sw
    out = {"kernel": FWD_KERNEL, "workload": WORKLOAD_NAMES[idx], "kernel_source_sha": kernel_source_sha(),
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes_each_way": COPY_BYTES,
           "fetch_scale": sf, "write_scale": sw,
           "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": nbytes,
           "traffic_over_algorithmic": traffic / nbytes,
           "commands": [f"rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_fetch -o pmc -- python3 bench.py "
                        f"--pmc-run --workload {idx}",
                        f"rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_write -o pmc -- python3 bench.py "
                        f"--pmc-run --workload {idx}",
                        f"python3 bench.py --workload {idx} --write-traffic "
                        "gpurun_out/pmc_fetch/pmc_counter_collection.csv "
                        "gpurun_out/pmc_write/pmc_counter_collection.csv"]}
    path = TRAFFIC_FILE if idx == 1 else TRAFFIC_FILE.replace("workload1", f"workload{idx}")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


GEMM_N = 8192  # the bf16 GEMM of --pmc-run: 2 N^3 flops, calibrates the MFMA counter


def write_counters(csvs, idx: int):
    """Per-call means of every SQ/GRBM counter collected over `bench.py --pmc-run --workload idx`
    (one counter pass per file), summed over the kernels of one forward call, with the executed
    bf16 MFMA flops: SQ_INSTS_VALU_MFMA_MOPS_BF16 scaled by 2 N^3 / (its value for the N^3 bf16
    GEMM of the same run)."""
    means = {}
    for p in csvs:
        means.update(_counter_means(p))
    names = sorted({cn for (_, cn) in means})
    fwd = {}
    for cn in names:
        try:
            fwd[cn] = _pick(means, cn, FWD_KERNEL_SYMBOL)
        except SystemExit:
            pass
    out = {"kernel": FWD_KERNEL, "workload": WORKLOAD_NAMES[idx], "kernel_source_sha": kernel_source_sha(),
           "per_call": fwd}
    mops = "SQ_INSTS_VALU_MFMA_MOPS_BF16"
    if mops in fwd:
        gemm = [v for (k, cn), v in means.items() if cn == mops and "lz::" not in k and "fwd_full" not in k]
        g = max(gemm) if gemm else 0.0
        if g > 0:
            per_mop = 2.0 * GEMM_N ** 3 / g
            _, algo = fwd_algorithmic(WORKLOADS[idx])
            out["mfma_flops_per_mop"] = per_mop
            out["executed_mfma_flops_per_call"] = fwd[mops] * per_mop
            out["algorithmic_flops_per_call"] = algo
            out["executed_over_algorithmic"] = fwd[mops] * per_mop / algo
    out["commands"] = [f"rocprofv3 --pmc <counters> -f csv -d gpurun_out/pmc_<pass> -o pmc -- python3 bench.py "
                       f"--pmc-run --workload {idx}", f"python3 bench.py --workload {idx} --write-counters <csv files>"]
    with open(COUNTER_FILE.format(idx), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def load_counters(idx: int):
    try:
        with open(COUNTER_FILE.format(idx)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t


def load_traffic(idx: int = 1):
    path = TRAFFIC_FILE if idx == 1 else TRAFFIC_FILE.replace("workload1", f"workload{idx}")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Warm-up calls before the timed ones; the warm-up then continues until CLOCK_WARMUP_MS of
    # steady calls have run (with 3 warm-up calls the timed calls of workload 1 ran about 15%
    # slower than with 200 or more: the clocks had not settled).
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--workload", type=int, default=1, choices=(1, 2, 4),
                    help="forward workload to time (2: 32K stress, 4: GQA); other than 1, only that "
                         "forward is timed and reported")
    ap.add_argument("--no-hedgehog", action="store_true",
                    help="skip the Hedgehog-map forward on the same shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward pass on the same shape")
    ap.add_argument("--no-separate-w", action="store_true",
                    help="skip the forward with per-head, separate W_phi on the same shape")
    ap.add_argument("--no-gla", action="store_true",
                    help="skip the standard / reparameterized GLA-only forwards on the same shape")
    ap.add_argument("--pmc-run", action="store_true",
                    help="a few forward calls, a plain copy of known size and a bf16 GEMM of known flops, "
                         "for rocprofv3 counter passes")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="(no GPU) turn the two counter_collection.csv files of the --pmc-run passes "
                         "into profiles/traffic_fwd_full_workload<N>.json")
    ap.add_argument("--write-counters", nargs="+", metavar="CSV",
                    help="(no GPU) turn counter_collection.csv files of --pmc-run passes into "
                         "profiles/counters_fwd_full_workload<N>.json")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.workload)
        return
    if args.write_counters:
        write_counters(args.write_counters, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards by batch/head with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    api.load()

    if args.pmc_run:
        bench_forward(2, 1, args.workload, min_warm_ms=0.0, flushed=False)
        nbytes = COPY_BYTES
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        del src, dst
        a = torch.full((GEMM_N, GEMM_N), 0.5, dtype=torch.bfloat16, device="cuda")
        b = torch.full((GEMM_N, GEMM_N), 0.25, dtype=torch.bfloat16, device="cuda")
        torch.matmul(a, b)
        torch.cuda.synchronize()
        log(f"[bench] pmc run: forward calls, then a copy of {nbytes} bytes each way, then a "
            f"{GEMM_N}^3 bf16 GEMM")
        return

    c, inp, total_ms, per, per_fl, (wcalls, wms) = bench_forward(args.steps, args.warmup, args.workload)
    ms_per_step = total_ms / args.steps
    tokens = c["B"] * c["L"]
    value = tokens / (ms_per_step * 1e-3)
    nbytes, flops = fwd_algorithmic(c)
    st = launch_stats(per)
    kern_ms = st["mean_ms"]  # the average launch duration (the kernel-trace summary's figure)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    mfma_tflops = flops / (kern_ms * 1e-3) / 1e12
    traffic = load_traffic(args.workload)
    counters = load_counters(args.workload)
    mfma = {"algorithmic_flops_per_launch": flops, "achieved_tflops": mfma_tflops,
            "peak_tflops": BF16_PEAK_TFLOPS, "frac": mfma_tflops / BF16_PEAK_TFLOPS,
            "executed_flops_per_launch": None, "executed_tflops": None, "executed_frac": None}
    if counters and counters.get("executed_mfma_flops_per_call"):
        ex = counters["executed_mfma_flops_per_call"]
        mfma.update(executed_flops_per_launch=ex, executed_tflops=ex / (kern_ms * 1e-3) / 1e12,
                    executed_frac=ex / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                    executed_source=os.path.relpath(COUNTER_FILE.format(args.workload), ROOT))
    result = {
        "metric": "Lizard-attn fwd tokens/sec at L=4096,H=32,d=128; % MFMA peak; decode % HBM BW",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup": {"calls": wcalls, "ms": wms, "min_ms": CLOCK_WARMUP_MS},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "B": c["B"], "H": c["Hq"], "Hkv": c["Hkv"],
                   "L": c["L"], "d": c["d"], "W": c["W"], "M": c["M"], "chunk": 64, "accumulation": "fp32"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": FWD_KERNEL if args.workload == 1 else "fwd_full_state_kernel + fwd_full_kernel",
                     "kernel_ms": kern_ms, "launches": {**st, "mall_flushed": False},
                     "mall_flushed_launches": launch_stats(per_fl),
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": mfma,
    }
    del inp
    torch.cuda.empty_cache()
    if args.workload != 1:
        print(json.dumps(result), flush=True)
        return
    if not args.no_hedgehog:
        hc, htot, hper = bench_forward_hedgehog(max(args.steps // 2, 1), args.warmup)
        hms = statistics.median(hper)
        hach = nbytes / (hms * 1e-3) / 1e9
        result["hedgehog"] = {
            "workload": WORKLOAD_NAMES[1] + " hedgehog-map W_phi[128,64]",
            "steps": len(hper), "ms_per_step": htot / len(hper),
            "tokens_per_s": tokens / (htot / len(hper) * 1e-3),
            "roofline": {"bound": "hbm", "achieved": hach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": hach / HBM_PEAK_GBS, "kernel_ms": hms,
                         "algorithmic_bytes_per_launch": nbytes},
        }
        torch.cuda.empty_cache()
    if not args.no_separate_w:
        stot, sper = bench_forward_separate_w(max(args.steps // 2, 1), args.warmup)
        sms = statistics.median(sper)
        result["separate_w"] = {
            "workload": WORKLOAD_NAMES[1] + " with W_phi per query head and per key/value head",
            "steps": len(sper), "ms_per_step": stot / len(sper), "kernel_ms": sms,
            "tokens_per_s": tokens / (stot / len(sper) * 1e-3),
            "over_shared_w": sms / statistics.median(per),
        }
        torch.cuda.empty_cache()
    if not args.no_gla:
        gc, gres = bench_gla(max(args.steps // 2, 1), args.warmup)
        fwd_ms = statistics.median(per)
        gms = {m: statistics.median(p) for m, (t, p) in gres.items()}
        result["gla"] = {
            "workload": WORKLOAD_NAMES[1] + " global branch only (mix = 1, no window)",
            "steps": len(gres["standard"][1]),
            "standard_ms": gms["standard"], "reparam_ms": gms["reparam"], "lizard_fwd_ms": fwd_ms,
            "standard_tokens_per_s": tokens / (gms["standard"] * 1e-3),
            "reparam_tokens_per_s": tokens / (gms["reparam"] * 1e-3),
            "standard_over_reparam": gms["standard"] / gms["reparam"],
            "standard_over_lizard_fwd": gms["standard"] / fwd_ms,
            "timing": "median per-launch HIP-event time, inputs resident, after a clock warm-up",
        }
        torch.cuda.empty_cache()
    if not args.no_backward:
        bc, btot, bper, bws = bench_backward(max(args.steps // 2, 1), args.warmup)
        bms = statistics.median(bper)
        bbytes = bwd_algorithmic_bytes(bc)
        result["backward"] = {
            "workload": WORKLOAD_NAMES[1] + " backward (dq, dk, dv, dlog_gamma, dW_phi, dT)",
            "steps": len(bper), "ms_per_step": btot / len(bper),
            "tokens_per_s": tokens / (btot / len(bper) * 1e-3),
            "workspace_bytes": bws,
            "roofline": {"bound": "hbm", "achieved": bbytes / (bms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": bbytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, "kernel_ms": bms,
                         "algorithmic_bytes_per_launch": bbytes},
        }
        torch.cuda.empty_cache()
    if not args.no_decode:
        dc, dtot, dper, dreps = bench_decode(args.decode_steps, 4)
        dbytes = decode_bytes_per_step(dc)
        dms = statistics.median(dper)
        gms = statistics.median(dreps) / args.decode_steps
        dach = dbytes / (gms * 1e-3) / 1e9
        result["decode"] = {
            "workload": WORKLOAD_NAMES[3], "steps": args.decode_steps,
            "ms_per_step": gms, "tokens_per_s": dc["N"] / (gms * 1e-3),
            "timing": f"{args.decode_steps} consecutive steps captured in one HIP graph, median of 5 replays",
            "eager": {"ms_per_step": dtot / args.decode_steps, "step_ms_median": dms,
                      "frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "roofline": {"bound": "hbm", "achieved": dach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dach / HBM_PEAK_GBS, "bytes_per_step": dbytes, "step_ms": gms},
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
