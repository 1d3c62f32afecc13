"""GPU parity outside the workloads' input domain, through GDN_ALGO_AUTO.

The workloads feed L2-normalised keys and gates from the gate prologue (a
true decay, g <= 0).  The pages keep unnormalised keys legal on every route and
decline a chunked fast path because neither a bounded decay nor normalised keys
follows from a node's shape ([P1] onnxruntime-ep-mlx, src/ops/ssm.rs, module
doc and the scan kernel's comment).  The library's chunked forms are the same
recurrence regrouped, exact in real arithmetic for any gates; here they are
held to the oracle on:
  - keys whose norms spread over [0.3, 1.4] (beta |k|^2 up to about 1.9, so
    the delta step's transition I - beta k k^T has eigenvalues in (-1, 1]);
  - precomputed log-decays with every 13th (token, head) entry positive, up to
    +0.3 (the state grows at those steps).
The plan query confirms that AUTO took the chunked form being tested.
Tolerances as everywhere: |d| <= tol (1 + |ref|) elementwise, plus
||d||_F <= tol ||ref||_F for bfloat16 I/O.
"""
import dataclasses

import pytest
import torch

from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, gates_for, gpu_prefill, oracle_prefill, say, workspace_for

pytestmark = pytest.mark.gpu

W = synth.BY_NAME


def _inputs(base, seqlens, *, seed, norms=(0.3, 1.4), positive_every=13, positive_hi=0.3, **over):
    shape = dataclasses.replace(W[base], **over)
    inp = synth.generate(shape, seqlens=seqlens, seed=seed)
    inp.k = synth.rescale_rows(inp.k, *norms, seed=seed + 1)
    if shape.gate_mode == "raw":
        return shape, inp, None, None
    g, beta = gates_for(inp)
    if positive_every:
        g = synth.positive_log_decays(g, positive_every, positive_hi, seed=seed + 2)
    return shape, inp, g, beta


def _plan(shape, inp, two_pass):
    ws = workspace_for(inp) if two_pass else None
    return gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, len(inp.seqlens),
                                  inp.total_tokens, raw_gates=shape.gate_mode == "raw",
                                  workspace_bytes=0 if ws is None else ws.numel())


BF16_CASES = [
    # (workload, seqlens, two_pass, form AUTO must take)
    ("varlen_prefill_8seq", [300, 129, 70], False, "chunked_one_pass"),
    ("varlen_prefill_8seq", [300, 129, 70], True, "chunked_two_pass"),
    ("prefill_t4096_fused_gates", [600], True, "chunked_two_pass"),
    ("prefill_t4096_fused_gates", [600], False, "chunked_one_pass"),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=[f"{c[0]}_{'two' if c[2] else 'one'}_pass" for c in BF16_CASES])
def test_bf16_chunked_unnormalised_keys_growing_gates(case):
    name, lens, two_pass, form = case
    shape, inp, g, beta = _inputs(name, lens, seed=501)
    raw = shape.gate_mode == "raw"
    plan = _plan(shape, inp, two_pass)
    say(f"[domain bf16] {name} {lens} two_pass={two_pass} plan={plan}")
    assert plan["form"] == form, plan
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm="auto", two_pass=two_pass)
    ro, rf = oracle_prefill(inp, g, beta, raw=raw)
    check(out, ro, TOL[torch.bfloat16], "out")
    check(fin, rf, TOL[torch.bfloat16], "final state")


F32_CASES = [
    # (h_qk, h_v, d_k, d_v, seqlens, initial state)
    (2, 2, 256, 256, [400], False),
    (4, 4, 128, 128, [300, 65], True),
    (1, 2, 256, 64, [1, 260], True),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: f"hq{c[0]}_hv{c[1]}_dk{c[2]}_dv{c[3]}_T{sum(c[4])}")
def test_f32_chunked_unnormalised_keys_growing_gates(case):
    h_qk, h_v, d_k, d_v, lens, init = case
    shape, inp, g, beta = _inputs("wide_prefill_t32768_d256", lens, seed=502, h_qk=h_qk, h_v=h_v, d_k=d_k,
                                  d_v=d_v, init_state=init)
    plan = _plan(shape, inp, True)
    say(f"[domain f32] {case} plan={plan}")
    assert plan["form"] == "chunked_f32", plan
    out, fin = gpu_prefill(inp, g, beta, algorithm="auto", two_pass=True)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, TOL[torch.float32], "out")
    check(fin, rf, TOL[torch.float32], "final state")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_serial_unnormalised_keys_growing_gates(dtype):
    """The serial scan on the same kind of inputs (short sequences: AUTO keeps it)."""
    shape, inp, g, beta = _inputs("varlen_prefill_8seq", [40, 17, 3], seed=503, io_dtype=dtype, h_qk=2, h_v=4,
                                  d_k=128, d_v=64)
    plan = _plan(shape, inp, False)
    assert plan["form"] == "serial", plan
    out, fin = gpu_prefill(inp, g, beta, algorithm="auto")
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, TOL[dtype], "out")
    check(fin, rf, TOL[dtype], "final state")
