#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: the decode step at B = 64 (H_qk 16, H_v 32, d_k = d_v = 128,
bfloat16 q/k/v/gates, float32 state updated in place).  One step = one
gdn_decode_step over the whole batch.  The state rotates over 4 buffers
(4 x 128 MiB, more than the 256 MB Infinity Cache) so each step streams its
state from HBM.  W untimed steps, then K steps timed back to back between HIP
events on the stream the kernel runs on.  Prints ONE JSON line.

Other workloads (--workload prefill_t4096_fused_gates, varlen_prefill_8seq,
wide_prefill_t32768_d256, tiny_prefill) time one gdn_prefill per step, each
between its own events, with a 1 GiB read in between that flushes the L2 and
the Infinity Cache (clean lines only, so no write-back lands in the timed
launch).  The block's neighbouring operations are timed the same
way: conv_step_b64 (gdn_causal_conv_step), conv_varlen_8seq (gdn_causal_conv)
and gated_rmsnorm_t33173 (gdn_gated_rmsnorm).

Inputs are synthetic and seeded (gated_delta_rule_serial_amd.synth); they are
resident in device memory before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
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


def _kernel_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_serial_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(name: str, kernel_files) -> float | None:
    """HBM bytes per launch measured with rocprofv3 counters (profiles/<name>_traffic.json),
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256_16") != _kernel_hash(kernel_files):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline_decode(shape, inp, budget_s=10.0):
    """The oracle (as it stands) on a bounded sample of the decode workload:
    whole B = 64 decode steps on the host cores until ~budget_s has passed."""
    import numpy as np

    import oracle
    orc = oracle.default()
    q, k, v = inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy()
    gg, bb = orc.gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    st = inp.initial_state.double().numpy().copy()
    steps = 0
    t0 = time.perf_counter()
    while True:
        orc.decode_step(q, k, v, gg, bb, st)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s and steps >= 2:
            break
    assert np.isfinite(st).all()
    return dict(value=round(shape.num_seqs * steps / el, 3), unit="tokens/s", cores=orc.max_threads(),
                kind="oracle", sample=f"{steps} full decode steps (B={shape.num_seqs}, all heads) in {el:.1f} s")


def cpu_baseline_prefill(shape, inp, budget_s=10.0):
    """The oracle on a bounded sample of a prefill workload: the first m tokens of
    every sequence for the first k q/k head groups (all their value heads), with
    (k, m) sized from a short probe so that the run takes about budget_s.  The
    rate is scaled to all heads: tokens x (sampled value heads / h_v) / seconds."""
    import oracle
    orc = oracle.default()
    ratio = shape.h_v // shape.h_qk

    def run(groups, ntok):
        lens = [min(l, ntok) for l in inp.seqlens]
        idx = torch.cat([torch.arange(int(inp.cu_seqlens[i]), int(inp.cu_seqlens[i]) + lens[i])
                         for i in range(len(lens))])
        cu = [0]
        for l in lens:
            cu.append(cu[-1] + l)
        hv = slice(0, groups * ratio)
        gg, bb = orc.gates(inp.a[idx][:, hv], inp.b[idx][:, hv], inp.A_log[hv], inp.dt_bias[hv])
        s0 = None if inp.initial_state is None else inp.initial_state[:, hv].double().numpy()
        args = (inp.q[idx][:, :groups].double().numpy(), inp.k[idx][:, :groups].double().numpy(),
                inp.v[idx][:, hv].double().numpy(), gg, bb, cu, s0)
        t0 = time.perf_counter()
        orc.prefill(*args)
        return time.perf_counter() - t0, cu[-1]

    max_len = max(inp.seqlens)
    el, tok = run(1, min(128, max_len))
    per_unit = el / max(tok, 1)                     # seconds per token per head group (one thread's share)
    budget_units = budget_s / max(per_unit, 1e-9)   # token x group units that fit the budget
    groups = max(1, min(shape.h_qk, int(budget_units // max(inp.total_tokens, 1))))
    ntok = max_len if groups > 1 else max(128, min(max_len, int(budget_units / max(len(inp.seqlens), 1))))
    el, tok = run(groups, ntok)
    heads = groups * ratio
    return dict(value=round(tok * heads / shape.h_v / el, 3), unit="tokens/s", cores=orc.max_threads(),
                kind="oracle",
                sample=f"value heads 0-{heads - 1} of {shape.h_v} ({groups} q/k head groups), first {min(ntok, max_len)} "
                       f"tokens of each sequence ({tok} tokens) in {el:.1f} s; rate scaled to all heads")


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
    kernel_files = ["decode_step.hip", "gdn_device.hpp"]
    traffic = _traffic(shape.name, kernel_files)
    line = {
        "metric": METRIC,
        "value": round(shape.num_seqs / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "decode_step_us": round(ms * 1e3, 3),
        "ms_per_step": round(ms, 6),
        "wall_s": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_kernel<bf16, d_k 128, 128 columns per workgroup, precomputed gates>",
                     "algorithmic_bytes_per_launch": nbytes},
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


def chunked_flops(shape, T, chunk=64):
    """MFMA flops of the chunked form per launch: per token and value head,
    K K^T and Q K^T over the lower triangle (2 C d_k), W = T' K (C d_k),
    U = T'' V (C d_v), X = W S, Y = Q S and the state update (6 d_k d_v), M D (C d_v)."""
    dk, dv = shape.d_k, shape.d_v
    return T * shape.h_v * (3 * chunk * dk + 2 * chunk * dv + 6 * dk * dv)


def bench_prefill(shape, steps, warmup, want_cpu, algorithm="auto", two_pass=True):
    dev = "cuda"
    inp = synth.generate(shape)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    cu = inp.cu_seqlens.to(dev)
    cu_host = inp.cu_seqlens.tolist()
    raw = shape.gate_mode == "raw"
    if raw:
        gates = dict(a=inp.a.to(dev), b=inp.b.to(dev), A_log=inp.A_log.to(dev), dt_bias=inp.dt_bias.to(dev))
        g = beta = None
    else:
        g, beta = gdn.gate_prologue(inp.a.to(dev), inp.b.to(dev), inp.A_log.to(dev), inp.dt_bias.to(dev))
        gates = dict(g=g, beta=beta)
    s0 = None if inp.initial_state is None else inp.initial_state.to(dev)
    T = inp.total_tokens
    n = len(inp.seqlens)
    out = torch.empty(T, shape.h_v, shape.d_v, dtype=shape.io_dtype, device=dev)
    fin = torch.empty(n, shape.h_v, shape.d_k, shape.d_v, dtype=torch.float32, device=dev)
    flush = torch.zeros(256 * 1024 * 1024, dtype=torch.float32, device=dev)  # 1 GiB
    stream = torch.cuda.current_stream()
    # the chunked form's workspace (two passes), allocated before the timed region
    ws_bytes = gdn.prefill_workspace_size(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T,
                                          algorithm=algorithm) if two_pass else 0
    if ws_bytes:
        gates["workspace"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def one():
        gdn.gdn_prefill(q, k, v, cu, out=out, final_state=fin, initial_state=s0, cu_seqlens_host=cu_host,
                        algorithm=algorithm, **gates)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(steps):
        _flush(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        one()
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_list = sorted(a.elapsed_time(b) for a, b in times)
    ms = sum(ms_list) / len(ms_list)
    assert torch.isfinite(out.float()).all()
    nbytes = algorithmic_bytes(shape, inp)
    hbm_gbs = nbytes / (ms * 1e-3) / 1e9
    # the float32 chunked form (two passes, products on split bf16 operands) runs
    # whenever the workspace is given for float32 I/O
    wide = shape.io_dtype == torch.float32 and ws_bytes > 0
    chunked = wide or algorithm == "chunked" or (
        algorithm == "auto" and shape.io_dtype == torch.bfloat16 and shape.d_k in (64, 128)
        and shape.d_v % 8 == 0 and T >= 64 * n)
    if wide:
        # three bf16 MFMA products (hi.hi + hi.lo + lo.hi) per float32-class product
        fl = 3 * chunked_flops(shape, T)
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                "traffic": _traffic(shape.name + "_chunked_f32",
                                    ["prefill_wide.hip", "prefill_split.hip", "chunk_mfma.hpp", "gdn_device.hpp"]),
                "kernel": "wide_prep_kernel + wide_state_kernel (float32 I/O, chunked in two passes, split-bf16 MFMA)",
                "algorithmic_bytes_per_launch": nbytes, "workspace_bytes": ws_bytes,
                "mfma_tflops": round(fl / (ms * 1e-3) / 1e12, 2), "mfma_frac_of_bf16_peak":
                    round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    elif chunked:
        # the chunked form's intensity (~180 flop/B at d = 128) is below the bf16 MFMA
        # ridge (2.5 PFLOP/s / 8 TB/s ~ 312 flop/B): HBM bounds it
        fl = chunked_flops(shape, T)
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                "traffic": (_traffic(shape.name + "_two_pass", ["prefill_split.hip", "chunk_mfma.hpp", "gdn_device.hpp"])
                            if ws_bytes else
                            _traffic(shape.name + "_chunked", ["prefill_chunked.hip", "chunk_mfma.hpp", "gdn_device.hpp"])),
                "kernel": ("chunk_prep_kernel + chunk_state_kernel (chunked in two passes, bf16 MFMA)" if ws_bytes
                           else "chunk_kernel (chunked, bf16 MFMA)"),
                "algorithmic_bytes_per_launch": nbytes, "workspace_bytes": ws_bytes,
                "mfma_tflops": round(fl / (ms * 1e-3) / 1e12, 2), "mfma_frac_of_bf16_peak":
                    round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    else:
        # the serial form does 7 d_k d_v flops per token and head on the vector ALUs
        fl = flops_serial(shape, T)
        tf = fl / (ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(tf, 2), "peak": round(FP32_VALU_PEAK_TFLOPS, 2),
                "unit": "TFLOP/s", "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4),
                "traffic": _traffic(shape.name + "_serial", ["prefill_scan.hip", "gdn_device.hpp"]),
                "kernel": ("scan_plain_kernel (serial scan, d_k 256, two columns per wave)" if shape.d_k == 256
                           else "scan_plain_kernel or scan_kernel (serial scan)"), "flops_per_launch": fl,
                "algorithmic_bytes_per_launch": nbytes}
    line = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms, 6),
        "ms_median": round(ms_list[len(ms_list) // 2], 6),
        "wall_s": round(wall, 3),
        "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "roofline": roof,
        "config": {"workload": shape.name,
                   "algorithm": (("chunked, two passes, split-bf16 products" if wide else "chunked, two passes")
                                 if ws_bytes else "chunked") if chunked else "serial",
                   "num_seqs": n,
                   "total_tokens": T, "seqlens": inp.seqlens, "h_qk": shape.h_qk, "h_v": shape.h_v,
                   "d_k": shape.d_k, "d_v": shape.d_v,
                   "io_dtype": "bf16" if shape.io_dtype == torch.bfloat16 else "f32", "state_dtype": "f32",
                   "gates": shape.gate_mode},
    }
    if want_cpu:
        line["cpu_baseline"] = cpu_baseline_prefill(shape, inp)
    return line


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
                         "traffic": _traffic(shape.name, ["causal_conv.hip", "gdn_device.hpp"]),
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
                         "traffic": _traffic(shape.name, ["gated_rmsnorm.hip", "gdn_device.hpp"]),
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
    ap.add_argument("--workload", default="decode_b64",
                    choices=sorted(synth.BY_NAME) + sorted(synth.CONV_BY_NAME) + sorted(synth.NORM_BY_NAME))
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
    else:
        shape = synth.BY_NAME[args.workload]
        decode = shape.kind == "decode"
        steps = args.steps if args.steps is not None else (1000 if decode else 10)
        warmup = args.warmup if args.warmup is not None else (50 if decode else 3)
        if decode:
            line = bench_decode(shape, steps, warmup, want_cpu)
        else:
            line = bench_prefill(shape, steps, warmup, want_cpu, args.algorithm, not args.one_pass)
    head = {"metric": line.pop("metric"), "value": line.pop("value"), "unit": line.pop("unit"), "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": line.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    head.update(line)
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
