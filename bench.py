#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default: the decode step at B = 64 (H_qk 16, H_v 32, d_k = d_v = 128,
bfloat16 q/k/v/gates, float32 state updated in place) is the headline: one
step = one gdn_decode_step over the whole batch; the state rotates over 4
buffers (4 x 128 MiB, more than the 256 MB Infinity Cache) so each step
streams its state from HBM; W untimed steps, then K steps timed back to back
between HIP events on the stream the kernel runs on.  After the timed region,
min(K, 200) steps each between their own events give the median and p90, and
as many steps on one state buffer give the cache-assisted figure (128 MiB
fits the Infinity Cache), each labelled as such.  The same line then
carries, under "workloads", every prefill workload (tiny_prefill,
prefill_t4096_fused_gates, varlen_prefill_8seq, wide_prefill_t32768_d256):
min(K, 10) launches of gdn_prefill as the library's AUTO plan takes it (with a
workspace, so the chunked forms run in two passes), each between its own
events after a 1 GiB read that flushes the L2 and the Infinity Cache.  Each
entry has its mean and median time, tokens/s, the plan the library reports,
its own roofline and the oracle's CPU baseline.  Prints ONE JSON line.

The line also carries the block's neighbouring operations fused into the
recurrence against their unfused pairs: "output_norm" (the gated RMSNorm
epilogue) and "decode_conv" (the conv step as the decode step's prologue).

--workload NAME times one workload alone (any prefill workload, the block's
neighbouring operations conv_step_b64, conv_varlen_8seq, gated_rmsnorm_t33173,
or the fused pairs output_norm and decode_conv), for profiling.

CPU baseline: the oracle's float32 build (the same C source with a float32
working state, gcc -O3 -march=native, OpenMP over independent (sequence,
head) units, built on the host that runs it) on a bounded sample of each
workload: median of 3 runs on the host's threads, plus one run on a single
thread; nproc and the CPU model are reported.

Inputs are synthetic and seeded (gated_delta_rule_serial_amd.synth); they are
resident in device memory before the timed region starts.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_delta_rule_serial_amd import gdn, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
# FP32 vector FMA without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz.
FP32_VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12  # 78.64
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
DECODE_STATE_BUFFERS = 4
PREFILL_WORKLOADS = ["tiny_prefill", "prefill_t4096_fused_gates", "varlen_prefill_8seq", "wide_prefill_t32768_d256"]
METRIC = "GDN prefill tokens/s + decode-step \u00b5s (B=64), % of HBM peak on 1 MI355X"


def algorithmic_bytes(shape: synth.Shape, inp: synth.Inputs) -> int:
    """Inputs read once, outputs written once, state read (if given) and written once."""
    es = 2 if shape.io_dtype == torch.bfloat16 else 4
    T = inp.total_tokens
    n = len(inp.seqlens)
    qk = 2 * T * shape.h_qk * shape.d_k * es
    v = T * shape.h_v * shape.d_v * es
    o = T * shape.h_v * shape.d_v * es
    gates = 2 * T * shape.h_v * es
    params = 2 * shape.h_v * 4 if shape.gate_mode == "raw" else 0
    state = n * shape.h_v * shape.d_k * shape.d_v * 4
    state_io = state * (2 if inp.initial_state is not None else 1)
    cu = (n + 1) * 4 if shape.kind == "prefill" else 0
    return qk + v + o + gates + params + state_io + cu


def flops_serial(shape: synth.Shape, T: int) -> int:
    """decay 1 + retrieval 2 + update 2 + readout 2 flops per state element per token."""
    return 7 * T * shape.h_v * shape.d_k * shape.d_v


def chunked_flops(shape, T, chunk=64):
    """MFMA flops of the chunked form per launch: per token and value head,
    K K^T and Q K^T over the lower triangle (2 C d_k), W = T' K (C d_k),
    U = T'' V (C d_v), X = W S, Y = Q S and the state update (6 d_k d_v), M D (C d_v)."""
    dk, dv = shape.d_k, shape.d_v
    return T * shape.h_v * (3 * chunk * dk + 2 * chunk * dv + 6 * dk * dv)


def _manifest():
    try:
        from gated_delta_rule_serial_amd import build as libbuild
        return libbuild.load_manifest()
    except (OSError, ValueError):
        return None


def _record(name: str):
    """The rocprofv3 counter record profiles/<name>_traffic.json, or None when
    there is none or when the machine code of a kernel it measured differs
    from the built one (the record lists each kernel's code digest, from the
    build's manifest)."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    code = rec.get("kernels_code")
    man = _manifest()
    if not code or man is None:
        return None
    for kname, digest in code.items():
        if man.get(kname, {}).get("code_sha256_16") != digest:
            return None
    return rec


def _traffic(name: str):
    """HBM bytes per launch from the counter record (None when stale or absent)."""
    rec = _record(name)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def _counters(name: str):
    """Per-kernel utilisation counters of the record (MfmaUtil, VALUBusy,
    VALUUtilization, LDSBankConflict, in percent), keyed by kernel template
    name; None when the record is stale or absent."""
    rec = _record(name)
    if rec is None or not rec.get("utilisation_pct"):
        return None
    out = {}
    for k, v in rec["utilisation_pct"].items():
        short = k.replace("gdn::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        out[short] = v
    return out


# ---------------------------------------------------------------- CPU baseline (the oracle)
def _cpu_env(orc):
    import oracle
    cpu = oracle.host_cpu()
    return {"cpu_model": cpu["model"], "nproc": cpu["logical_cpus"], "threads_available": orc.max_threads(),
            "build": "oracle float32 working state, gcc -O3 -march=native, OpenMP over (sequence, head) units"}


def _median_runs(fn, runs=3):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2], ts


def cpu_baseline_decode(shape, inp, budget_s=1.5):
    """The oracle's float32 build on a bounded sample of the decode workload:
    k whole B = 64 decode steps (all heads), k sized from a probe so that one
    run takes about budget_s; median of 3 runs, then a single-thread run."""
    import numpy as np

    import oracle
    orc = oracle.float32_baseline()
    q, k, v = inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy()
    gg, bb = oracle.default().gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    st0 = inp.initial_state.double().numpy()
    threads = orc.max_threads()

    def steps_fn(nsteps):
        def run():
            st = st0.copy()
            for _ in range(nsteps):
                orc.decode_step(q, k, v, gg, bb, st)
            assert np.isfinite(st).all()
        return run

    _median_runs(steps_fn(1), runs=1)  # first touch of the inputs
    t1, _ = _median_runs(steps_fn(1), runs=1)
    nsteps = max(1, int(budget_s / max(t1, 1e-6)))
    med, ts = _median_runs(steps_fn(nsteps))
    orc.set_threads(1)
    try:
        n1 = max(1, int(budget_s / max(t1 * threads, 1e-6)))
        one, _ = _median_runs(steps_fn(n1), runs=1)
    finally:
        orc.set_threads(threads)
    B = shape.num_seqs
    res = {"value": round(B * nsteps / med, 3), "unit": "tokens/s", "cores": min(threads, B * shape.h_v),
           "kind": "oracle",
           "sample": f"{nsteps} whole decode steps (B={B}, all {shape.h_v} heads) per run, median of 3 runs "
                     f"({', '.join(f'{t:.2f}' for t in ts)} s)",
           "one_thread_value": round(B * n1 / one, 3),
           "one_thread_sample": f"{n1} decode steps in {one:.2f} s on 1 thread"}
    res.update(_cpu_env(orc))
    return res


def cpu_baseline_prefill(shape, inp, budget_s=1.5):
    """The oracle's float32 build on a bounded sample of a prefill workload:
    the first m tokens of every sequence, all heads, m sized from a probe so
    that one run takes about budget_s (the whole workload when it fits);
    median of 3 runs, then a single-thread run on its own sample."""
    import oracle
    orc = oracle.float32_baseline()
    threads = orc.max_threads()
    max_len = max(inp.seqlens)

    def sample(m):
        lens = [min(l, m) for l in inp.seqlens]
        idx = torch.cat([torch.arange(int(inp.cu_seqlens[i]), int(inp.cu_seqlens[i]) + lens[i])
                         for i in range(len(lens))])
        cu = [0]
        for l in lens:
            cu.append(cu[-1] + l)
        gg, bb = oracle.default().gates(inp.a[idx], inp.b[idx], inp.A_log, inp.dt_bias)
        s0 = None if inp.initial_state is None else inp.initial_state.double().numpy()
        args = (inp.q[idx].double().numpy(), inp.k[idx].double().numpy(), inp.v[idx].double().numpy(), gg, bb,
                cu, s0)
        return (lambda: orc.prefill(*args)), cu[-1]

    m0 = min(64, max_len)
    fn, tok0 = sample(m0)
    _median_runs(fn, runs=1)  # first touch of the inputs
    t0, _ = _median_runs(fn, runs=1)
    per_tok = t0 / max(tok0, 1)
    m = max(m0, min(max_len, int(m0 * budget_s / max(t0, 1e-6))))
    fn, tok = sample(m)
    med, ts = _median_runs(fn)
    units = len(inp.seqlens) * shape.h_v
    used = min(threads, units)
    orc.set_threads(1)
    try:
        m1 = max(1, min(max_len, int(budget_s / max(per_tok * used, 1e-9) / max(len(inp.seqlens), 1))))
        fn1, tok1 = sample(m1)
        one, _ = _median_runs(fn1, runs=1)
    finally:
        orc.set_threads(threads)
    whole = m >= max_len
    res = {"value": round(tok / med, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": (("the whole workload" if whole else f"the first {m} tokens of each sequence") +
                      f" ({tok} tokens, all {shape.h_v} value heads) per run, median of 3 runs "
                      f"({', '.join(f'{t:.2f}' for t in ts)} s)"),
           "one_thread_value": round(tok1 / one, 3),
           "one_thread_sample": f"{tok1} tokens (all heads) in {one:.2f} s on 1 thread"}
    res.update(_cpu_env(orc))
    return res


# ---------------------------------------------------------------- GPU
def bench_decode(shape, steps, warmup, want_cpu):
    dev = "cuda"
    inp = synth.generate(shape)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    # gates: the library's own gate prologue (bf16 g, beta from the raw draws)
    g, beta = gdn.gate_prologue(inp.a.to(dev), inp.b.to(dev), inp.A_log.to(dev), inp.dt_bias.to(dev))
    states = [inp.initial_state.to(dev).clone() for _ in range(DECODE_STATE_BUFFERS)]
    out = torch.empty(shape.num_seqs, shape.h_v, shape.d_v, dtype=shape.io_dtype, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        gdn.gdn_decode_step(q, k, v, states[i % len(states)], out, g=g, beta=beta)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        gdn.gdn_decode_step(q, k, v, states[i % len(states)], out, g=g, beta=beta)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    assert torch.isfinite(out.float()).all()
    nbytes = algorithmic_bytes(shape, inp)
    achieved = nbytes / (ms * 1e-3) / 1e9
    # outside the timed region: each step between its own events (median and
    # p90), and back-to-back steps on one state buffer, which the 256 MB
    # Infinity Cache can hold (cache-assisted, so not the headline)
    n_ev = min(steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        gdn.gdn_decode_step(q, k, v, states[i % len(states)], out, g=g, beta=beta)
        b.record(stream)
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    for _ in range(10):
        gdn.gdn_decode_step(q, k, v, states[0], out, g=g, beta=beta)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_ev):
        gdn.gdn_decode_step(q, k, v, states[0], out, g=g, beta=beta)
    e1.record(stream)
    torch.cuda.synchronize()
    line = {
        "metric": METRIC,
        "value": round(shape.num_seqs / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "decode_step_us": round(ms * 1e3, 3),
        "decode_step_us_per_step_events": {"steps": n_ev, "median": round(per_step[n_ev // 2], 3),
                                           "p90": round(per_step[min(n_ev - 1, (9 * n_ev) // 10)], 3)},
        "decode_step_us_one_state_buffer_cache_assisted": round(e0.elapsed_time(e1) * 1e3 / n_ev, 3),
        "ms_per_step": round(ms, 6),
        "wall_s": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic(shape.name),
                     "kernel": "decode_kernel<bf16, d_k 128, 128 columns per workgroup, precomputed gates>",
                     "algorithmic_bytes_per_launch": nbytes, "counters_pct": _counters(shape.name)},
        "config": {"workload": shape.name, "batch": shape.num_seqs, "h_qk": shape.h_qk, "h_v": shape.h_v,
                   "d_k": shape.d_k, "d_v": shape.d_v, "io_dtype": "bf16", "state_dtype": "f32",
                   "gates": "precomputed bf16", "state_buffers_rotated": DECODE_STATE_BUFFERS},
    }
    if want_cpu:
        line["cpu_baseline"] = cpu_baseline_decode(shape, inp)
    return line


def _flush(buf):
    """Evict L2 and the 256 MB Infinity Cache before a timed launch by reading a
    1 GiB buffer.  A read leaves clean lines behind; a write-based flush leaves
    dirty ones, and their write-back to HBM then runs inside the timed launch
    (about 40 us on a 272 MB x 3 elementwise kernel)."""
    buf.sum()


def prefill_roofline(shape, T, ms, nbytes, plan, ws_bytes):
    """The roofline of the form the library took: HBM for the chunked forms
    (their ~180 flop/B at d = 128 sit below the bf16 MFMA ridge of
    2.5 PFLOP/s / 8 TB/s ~ 312 flop/B), with the MFMA rate beside it; the
    vector ALUs for the serial scan (7 d_k d_v flops per token and head), with
    the HBM fraction beside it."""
    hbm_gbs = nbytes / (ms * 1e-3) / 1e9
    form = plan["form"]
    traffic = _traffic(f"{shape.name}_{form}")
    counters = _counters(f"{shape.name}_{form}")
    if form.startswith("chunked"):
        # float32 I/O: three bf16 MFMA products (hi.hi + hi.lo + lo.hi) per product
        fl = chunked_flops(shape, T) * (3 if form == "chunked_f32" else 1)
        tf = fl / (ms * 1e-3) / 1e12
        return {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": plan["kernels"],
                "algorithmic_bytes_per_launch": nbytes, "workspace_bytes": ws_bytes,
                "mfma_tflops": round(tf, 2), "mfma_frac_of_bf16_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                "counters_pct": counters}
    fl = flops_serial(shape, T)
    tf = fl / (ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(tf, 2), "peak": round(FP32_VALU_PEAK_TFLOPS, 2), "unit": "TFLOP/s",
            "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": plan["kernels"],
            "flops_per_launch": fl, "algorithmic_bytes_per_launch": nbytes,
            "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "counters_pct": counters}


def bench_prefill(shape, steps, warmup, want_cpu, algorithm="auto", two_pass=True, flush=None):
    dev = "cuda"
    inp = synth.generate(shape)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cu = inp.cu_seqlens.to(dev)
    cu_host = inp.cu_seqlens.tolist()
    raw = shape.gate_mode == "raw"
    if raw:
        gates = dict(a=inp.a.to(dev), b=inp.b.to(dev), A_log=inp.A_log.to(dev), dt_bias=inp.dt_bias.to(dev))
    else:
        g, beta = gdn.gate_prologue(inp.a.to(dev), inp.b.to(dev), inp.A_log.to(dev), inp.dt_bias.to(dev))
        gates = dict(g=g, beta=beta)
    s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
    T = inp.total_tokens
    n = len(inp.seqlens)
    out = torch.empty(T, shape.h_v, shape.d_v, dtype=shape.io_dtype, device=dev)
    fin = torch.empty(n, shape.h_v, shape.d_k, shape.d_v, dtype=torch.float32, device=dev)
    if flush is None:
        flush = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device=dev)  # 1 GiB
    # the chunked form's workspace (two passes), allocated before the timed region
    ws_bytes = gdn.prefill_workspace_size(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T,
                                          algorithm=algorithm) if two_pass else 0
    if ws_bytes:
        gates["workspace"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    plan = gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T,
                                  algorithm=algorithm, raw_gates=raw, workspace_bytes=ws_bytes)

    def one():
        gdn.gdn_prefill(q, k, v, cu, out=out, final_state=fin, initial_state=s0, cu_seqlens_host=cu_host,
                        algorithm=algorithm, **gates)

    ms, med, wall = _timed(one, steps, warmup, flush)
    assert torch.isfinite(out.float()).all()
    nbytes = algorithmic_bytes(shape, inp)
    entry = {
        "ms": round(ms, 6),
        "ms_median": round(med, 6),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "steps": steps,
        "warmup": warmup,
        "wall_s": round(wall, 3),
        "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "plan": plan,
        "roofline": prefill_roofline(shape, T, ms, nbytes, plan, ws_bytes),
        "config": {"workload": shape.name, "num_seqs": n, "total_tokens": T, "seqlens": inp.seqlens,
                   "h_qk": shape.h_qk, "h_v": shape.h_v, "d_k": shape.d_k, "d_v": shape.d_v,
                   "io_dtype": "bf16" if shape.io_dtype == torch.bfloat16 else "f32", "state_dtype": "f32",
                   "gates": shape.gate_mode, "initial_state": inp.initial_state is not None},
    }
    if want_cpu:
        entry["cpu_baseline"] = cpu_baseline_prefill(shape, inp)
    return entry


def _timed(one, steps, warmup, flush=None):
    """Mean and median ms of `one` over `steps` launches, each between its own
    events on the current stream (after a cache flush when given)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            _flush(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        one()
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_list = sorted(a.elapsed_time(b) for a, b in times)
    return sum(ms_list) / len(ms_list), ms_list[len(ms_list) // 2], wall


def _timed_ab(one_a, one_b, steps, warmup, flush=None):
    """_timed for two variants of the same work, their steps interleaved (a, b,
    a, b, ...) so that clock and cache drift over the run falls on both alike."""
    for _ in range(warmup):
        one_a()
        one_b()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = ([], [])
    for _ in range(steps):
        for i, one in enumerate((one_a, one_b)):
            if flush is not None:
                _flush(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one()
            e1.record(stream)
            times[i].append((e0, e1))
    torch.cuda.synchronize()
    out = []
    for t in times:
        ms_list = sorted(a.elapsed_time(b) for a, b in t)
        out.append((sum(ms_list) / len(ms_list), ms_list[len(ms_list) // 2]))
    return out


def bench_conv(shape, steps, warmup, want_cpu):
    """gdn_causal_conv over packed sequences, or gdn_causal_conv_step for the
    one-token workload.  HBM-bound: x and y once, the states in and out once,
    the weights and bias once."""
    dev = "cuda"
    inp = synth.generate_conv(shape)
    es = inp.x.element_size()
    C, K = inp.weight.shape
    carry = (K - 1) * shape.dilation
    x, w, b = inp.x.to(dev), inp.weight.to(dev), inp.bias.to(dev)
    n = len(inp.seqlens)
    T = sum(inp.seqlens)
    y = torch.empty_like(x)
    step = shape.seqlen == 1
    s0 = inp.initial_state.to(dev)
    fin = s0 if step else torch.empty_like(s0)
    cu = inp.cu_seqlens.to(dev)
    cu_host = inp.cu_seqlens.tolist()
    flush = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device=dev)

    def one():
        if step:
            gdn.gdn_causal_conv_step(x, w, fin, y=y, bias=b, dilation=shape.dilation)
        else:
            gdn.gdn_causal_conv(x, w, cu, y=y, bias=b, initial_state=s0, final_state=fin,
                                dilation=shape.dilation, cu_seqlens_host=cu_host)

    ms, med, wall = _timed(one, steps, warmup, flush)
    nbytes = 2 * T * C * es + 2 * n * carry * C * es + C * K * es + C * es + (0 if step else (n + 1) * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    line = {"metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 6),
            "ms_median": round(med, 6), "wall_s": round(wall, 3), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": _traffic(shape.name),
                         "kernel": "conv_step_kernel" if step else "conv_window_kernel + conv_state_kernel",
                         "algorithmic_bytes_per_launch": nbytes},
            "config": {"workload": shape.name, "num_seqs": n, "total_tokens": T, "channels": C, "kernel_size": K,
                       "dilation": shape.dilation, "io_dtype": "bf16", "activation": "silu"}}
    if want_cpu:
        import oracle
        orc = oracle.default()
        cols = min(C, 64)
        t0 = time.perf_counter()
        orc.causal_conv(inp.x[:, :cols], inp.weight[:cols], cu_host, inp.bias[:cols], inp.initial_state[:, :, :cols],
                        dilation=shape.dilation, silu=True)
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(T * cols / C / el, 3), "unit": "tokens/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"channels 0-{cols - 1} of {C}, every token ({T}), in {el:.2f} s on one "
                                          f"thread; rate scaled to all channels"}
    return line


def bench_norm(shape, steps, warmup, want_cpu):
    """gdn_gated_rmsnorm over [rows, width]: x and gate read once, y written once."""
    dev = "cuda"
    inp = synth.generate_norm(shape)
    es = inp.x.element_size()
    x, g, sc = inp.x.to(dev), inp.gate.to(dev), inp.scale.to(dev)
    y = torch.empty_like(x)
    flush = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    ms, med, wall = _timed(lambda: gdn.gdn_gated_rmsnorm(x, g, sc, y=y), steps, warmup, flush)
    nbytes = 3 * x.numel() * es + sc.numel() * es
    gbs = nbytes / (ms * 1e-3) / 1e9
    line = {"metric": METRIC, "value": round(shape.rows / (ms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 6), "ms_median": round(med, 6), "wall_s": round(wall, 3),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": _traffic(shape.name),
                         "kernel": "rmsnorm_kernel", "algorithmic_bytes_per_launch": nbytes},
            "config": {"workload": shape.name, "rows": shape.rows, "width": shape.width, "group": shape.group,
                       "io_dtype": "bf16", "activation": "silu", "eps": 1e-5}}
    if want_cpu:
        import oracle
        orc = oracle.default()
        rows = min(shape.rows, 2048)
        t0 = time.perf_counter()
        orc.gated_rmsnorm(inp.x[:rows], inp.gate[:rows], inp.scale)
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(rows / el, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                "sample": f"rows 0-{rows - 1} of {shape.rows} in {el:.2f} s on one thread"}
    return line


# Shapes of the output-norm comparison: the decode step, the packed 8-sequence
# workload (its state pass runs 64-column blocks, so AUTO keeps the norm a
# separate pass), and the same geometry at 16 sequences of 2048 tokens (512
# units: 128-column blocks, where AUTO fuses the norm into the state pass).
NORM_SHAPES = {
    "decode_b64": synth.BY_NAME["decode_b64"],
    "varlen_prefill_8seq": synth.BY_NAME["varlen_prefill_8seq"],
    "packed_16x2048": dataclasses.replace(synth.BY_NAME["varlen_prefill_8seq"], name="packed_16x2048", num_seqs=16,
                                          seqlen=2048, len_range=None),
}


def bench_output_norm(name, steps, warmup, flush):
    """The recurrence with its gated RMSNorm epilogue (one group per value head),
    fused into the output store where the plan fuses it, against the unfused
    pair: the recurrence writing o, then gdn_gated_rmsnorm over o in place.
    Algorithmic bytes: the fused call replaces the write of o by the read of
    the gate and the write of y; the pair adds to the recurrence's bytes a
    read of o and of the gate and a write of y.  The prefill shapes are timed
    launch by launch after a cache flush, interleaved; the decode step in
    alternating blocks of back-to-back steps, as the headline."""
    dev = "cuda"
    shape = NORM_SHAPES[name]
    inp = synth.generate(shape)
    T = inp.total_tokens
    n = len(inp.seqlens)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    raw = shape.gate_mode == "raw"
    decode = shape.kind == "decode"
    if raw:
        gates = dict(a=inp.a.to(dev), b=inp.b.to(dev), A_log=inp.A_log.to(dev), dt_bias=inp.dt_bias.to(dev))
    else:
        g, beta = gdn.gate_prologue(inp.a.to(dev), inp.b.to(dev), inp.A_log.to(dev), inp.dt_bias.to(dev))
        gates = dict(g=g, beta=beta)
    gate, scale = synth.output_norm_inputs(T, shape.h_v, shape.d_v, seed=1234 + 30, io_dtype=shape.io_dtype)
    gate, scale = gate.to(dev), scale.to(dev)
    out = torch.empty(T, shape.h_v, shape.d_v, dtype=shape.io_dtype, device=dev)
    es = out.element_size()
    if decode:
        states = [inp.initial_state.to(dev).clone() for _ in range(DECODE_STATE_BUFFERS)]
        it = [0]

        def rec(**kw):
            it[0] += 1
            gdn.gdn_decode_step(q, k, v, states[it[0] % len(states)], out, **gates, **kw)
        plan_norm = "fused"
        fl = None
    else:
        cu = inp.cu_seqlens.to(dev)
        cu_host = inp.cu_seqlens.tolist()
        s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
        fin = torch.empty(n, shape.h_v, shape.d_k, shape.d_v, dtype=torch.float32, device=dev)
        ws_bytes = gdn.prefill_workspace_size(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        plan_norm = gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T,
                                           raw_gates=raw, workspace_bytes=ws_bytes, norm=True)
        fl = flush

        def rec(**kw):
            gdn.gdn_prefill(q, k, v, cu, out=out, final_state=fin, initial_state=s0, cu_seqlens_host=cu_host,
                            **gates, **({"workspace": ws} if ws is not None else {}), **kw)
    nbytes = algorithmic_bytes(shape, inp)
    o_bytes = out.numel() * es
    fused_bytes = nbytes + o_bytes + scale.numel() * es          # + gate read (y replaces o)
    pair_bytes = nbytes + 3 * o_bytes + scale.numel() * es        # + o read, gate read, y write
    if plan_norm != "fused" and plan_norm.get("norm") != "fused":
        fused_bytes = pair_bytes  # the plan runs the norm as its own pass: the pair's traffic
    o2 = out.view(T, -1)

    def pair():
        rec()
        gdn.gdn_gated_rmsnorm(o2, gate.view(T, -1), scale, y=o2)
    if decode:  # back-to-back blocks, as the headline decode (no median then)
        ms_f, ms_p = _timed_blocks(lambda: rec(norm_gate=gate, norm_scale=scale), pair, steps, warmup)
        med_f, med_p = ms_f, ms_p
    else:
        (ms_f, med_f), (ms_p, med_p) = _timed_ab(lambda: rec(norm_gate=gate, norm_scale=scale), pair, steps,
                                                 warmup, fl)
    return {"tokens": T, "fused": {"ms": round(ms_f, 6), "ms_median": round(med_f, 6), "plan": plan_norm,
                      "algorithmic_bytes": fused_bytes,
                      "hbm_frac": round(fused_bytes / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "unfused_pair": {"ms": round(ms_p, 6), "ms_median": round(med_p, 6), "algorithmic_bytes": pair_bytes,
                             "hbm_frac": round(pair_bytes / (ms_p * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "saved_ms": round(ms_p - ms_f, 6), "saved_bytes": pair_bytes - fused_bytes}


def _timed_blocks(one_a, one_b, steps, warmup, blocks=4):
    """Mean ms per step of two variants of the same step, each timed as
    `steps` back-to-back launches between events, in `blocks` alternating
    blocks (a, b, a, b, ...).  Back to back, as the headline decode is timed:
    events around each launch would add a fixed launch gap to both and hide
    a difference of a few microseconds."""
    def block(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    for fn in (one_a, one_b):
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    ta, tb = [], []
    for _ in range(blocks):
        ta.append(block(one_a))
        tb.append(block(one_b))
    return sum(ta) / len(ta), sum(tb) / len(tb)


def bench_decode_conv(steps, warmup):
    """The decode step fed by the block's conv (gdn_decode_step_conv: the conv
    step and the decode step in one launch) against the unfused pair
    (gdn_causal_conv_step writing y, then gdn_decode_step), at the decode
    workload (B = 64, H 16/32, d 128, bf16) and its conv (8192 channels, 4
    taps, silu).  The pair's decode reads q, k, v buffers of y's size: the
    split of y into them is not charged to it.  Each form runs `steps` steps
    back to back between events, in four alternating blocks, and the
    recurrent state rotates over 4 buffers as in the headline; the fused form
    alternates its two conv-state buffers.  Algorithmic bytes: the fused call
    reads x, the carried inputs, taps and bias in place of q, k and v; the
    pair adds y's write and its read as q, k, v."""
    dev = "cuda"
    shape = synth.BY_NAME["decode_b64"]
    inp = synth.generate(shape)
    cin = synth.generate_conv(synth.CONV_BY_NAME["conv_step_b64"])
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    g, beta = gdn.gate_prologue(inp.a.to(dev), inp.b.to(dev), inp.A_log.to(dev), inp.dt_bias.to(dev))
    states = [inp.initial_state.to(dev).clone() for _ in range(DECODE_STATE_BUFFERS)]
    out = torch.empty(shape.num_seqs, shape.h_v, shape.d_v, dtype=shape.io_dtype, device=dev)
    x, w, bias = cin.x.to(dev), cin.weight.to(dev), cin.bias.to(dev)
    cs = [cin.initial_state.to(dev).clone() for _ in range(2)]
    y = torch.empty_like(x)
    it = [0]

    def fused():
        i = it[0] = it[0] + 1
        gdn.gdn_decode_step_conv(x, w, cs[i % 2], cs[1 - i % 2], states[i % len(states)], out, h_qk=shape.h_qk,
                                 d_k=shape.d_k, conv_bias=bias, g=g, beta=beta)

    def pair():
        i = it[0] = it[0] + 1
        gdn.gdn_causal_conv_step(x, w, cs[0], y=y, bias=bias)
        gdn.gdn_decode_step(q, k, v, states[i % len(states)], out, g=g, beta=beta)

    ms_f, ms_p = _timed_blocks(fused, pair, steps, warmup)
    es = x.element_size()
    rec = algorithmic_bytes(shape, inp)                   # state in/out, q, k, v, gates, out
    qkv = x.numel() * es
    conv_extra = 2 * cs[0].numel() * es + (w.numel() + bias.numel()) * es   # carried inputs in/out, taps
    fused_bytes = rec + conv_extra                        # x (the size of q, k, v) read in their place
    pair_bytes = rec + 2 * qkv + conv_extra               # + the conv's x read and y write
    return {"fused": {"us": round(ms_f * 1e3, 3), "algorithmic_bytes": fused_bytes,
                      "hbm_frac": round(fused_bytes / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "unfused_pair": {"us": round(ms_p * 1e3, 3), "algorithmic_bytes": pair_bytes,
                             "hbm_frac": round(pair_bytes / (ms_p * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "saved_us": round((ms_p - ms_f) * 1e3, 3), "saved_bytes": pair_bytes - fused_bytes,
            "steps_per_block": steps, "blocks": 4}


def bench_copy(mib, steps, warmup):
    """A plain device copy of known size (dst.copy_(src), mib MiB each way): the
    reference kernel that scales the rocprofv3 HBM byte counters."""
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"metric": "device copy", "value": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 6), "bytes_read": n * 4, "bytes_written": n * 4}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all",
                    choices=["all", "output_norm", "decode_conv"] + sorted(synth.BY_NAME) + sorted(synth.CONV_BY_NAME) +
                    sorted(synth.NORM_BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--algorithm", default="auto", choices=["auto", "serial", "chunked"],
                    help="prefill formulation (prefill workloads only)")
    ap.add_argument("--one-pass", action="store_true",
                    help="chunked prefill: no workspace, one pass per sequence")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="time a plain device copy of this many MiB instead (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the gated delta-rule path here runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported; per-GPU sharding is by heads or sequences, "
              f"with no exchange inside the op)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        print(json.dumps(bench_copy(args.copy_mib, args.steps or 50, args.warmup or 5)), flush=True)
        return
    want_cpu = not args.no_cpu_baseline
    if args.workload in synth.CONV_BY_NAME or args.workload in synth.NORM_BY_NAME:
        steps = args.steps if args.steps is not None else 20
        warmup = args.warmup if args.warmup is not None else 3
        if args.workload in synth.CONV_BY_NAME:
            line = bench_conv(synth.CONV_BY_NAME[args.workload], steps, warmup, want_cpu)
        else:
            line = bench_norm(synth.NORM_BY_NAME[args.workload], steps, warmup, want_cpu)
    elif args.workload == "output_norm":
        steps = args.steps if args.steps is not None else 10
        warmup = args.warmup if args.warmup is not None else 3
        flush = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
        res = {name: bench_output_norm(name, steps, warmup, flush) for name in NORM_SHAPES}
        e = res["packed_16x2048"]
        line = {"metric": METRIC, "value": round(e["tokens"] / (e["fused"]["ms"] * 1e-3), 1),
                "unit": "tokens/s", "ms_per_step": e["fused"]["ms"], "output_norm": res}
    elif args.workload == "decode_conv":
        steps = args.steps if args.steps is not None else 250
        warmup = args.warmup if args.warmup is not None else 20
        e = bench_decode_conv(steps, warmup)
        line = {"metric": METRIC, "value": round(64 / (e["fused"]["us"] * 1e-6), 1), "unit": "tokens/s",
                "ms_per_step": round(e["fused"]["us"] * 1e-3, 6), "decode_conv": e}
    elif args.workload in ("all", "decode_b64"):
        steps = args.steps if args.steps is not None else 1000
        warmup = args.warmup if args.warmup is not None else 50
        line = bench_decode(synth.BY_NAME["decode_b64"], steps, warmup, want_cpu)
        print(f"decode_b64: {line['decode_step_us']} us/step", file=sys.stderr, flush=True)
        if args.workload == "all":
            psteps, pwarm = max(3, min(steps, 10)), max(1, min(warmup, 3))
            flush = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
            line["workloads"] = {}
            for name in PREFILL_WORKLOADS:
                e = bench_prefill(synth.BY_NAME[name], psteps, pwarm, want_cpu, args.algorithm, not args.one_pass,
                                  flush=flush)
                line["workloads"][name] = e
                print(f"{name}: {e['ms']} ms ({e['plan']['form']}), HBM {100 * e['hbm_frac']:.1f} %",
                      file=sys.stderr, flush=True)
            # the block's output norm: fused epilogue against the unfused pair
            line["output_norm"] = {}
            for name in NORM_SHAPES:
                e = bench_output_norm(name, psteps if name != "decode_b64" else min(steps, 200), pwarm, flush)
                line["output_norm"][name] = e
                print(f"{name} + norm: fused {e['fused']['ms']} ms, pair {e['unfused_pair']['ms']} ms",
                      file=sys.stderr, flush=True)
            # the block's conv feeding the decode step: fused prologue against the unfused pair
            e = bench_decode_conv(min(steps, 250), min(warmup, 20))
            line["decode_conv"] = e
            print(f"decode_b64 + conv: fused {e['fused']['us']} us, pair {e['unfused_pair']['us']} us",
                  file=sys.stderr, flush=True)
    else:
        shape = synth.BY_NAME[args.workload]
        steps = args.steps if args.steps is not None else 10
        warmup = args.warmup if args.warmup is not None else 3
        e = bench_prefill(shape, steps, warmup, want_cpu, args.algorithm, not args.one_pass)
        line = {"metric": METRIC, "value": e.pop("tokens_per_s"), "unit": "tokens/s", "ms_per_step": e.pop("ms")}
        line.update(e)
    head = {"metric": line.pop("metric"), "value": line.pop("value"), "unit": line.pop("unit"), "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    head.update(line)
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
