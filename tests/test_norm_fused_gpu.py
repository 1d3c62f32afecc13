"""GPU parity of the recurrence with its gated RMSNorm epilogue (the output
norm of the block, [P1] onnxruntime-ep-mlx, src/ops/ssm.rs,
`gated_rms_norm_op`, one group per value head).

Reference: the oracle's recurrence (double) followed by the oracle's gated
RMSNorm of its outputs (double), both pinned on the CPU.  The fused forms
normalise the float32 readout in the kernel; the separate pass normalises
the narrowed output, as a caller running the two operations would.  Both are
held to the I/O dtype's tolerance normwise, and elementwise against each
element's gain (check_normed); the plan query says which form ran."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, gates_for, say, to_dev, workspace_for

pytestmark = pytest.mark.gpu
W = synth.BY_NAME


# The elementwise bound on normed outputs is a guard against gross errors (a
# wrong row's norm or a wrong gate element is off by O(gain)), at 5 tol: the
# norm maps each row of o to unit RMS, so the elementwise error of o relative
# to its row's RMS, which for the bf16 chunked forms has a tail (about 3e-3
# normwise, up to 2e-2 for the worst of 10^5 elements, the same with and
# without the fused epilogue), becomes the error of y.  The criterion proper
# is the normwise bound at tol.
GROSS = 5.0


def check_normed(gpu, ref, gate, scale, act, tol, what):
    """Normwise ||d||_F <= tol ||ref||_F, and elementwise |d| <= GROSS tol
    (|gain| + |ref|) with gain = scale act(gate): the norm multiplies element
    j of the unit-RMS row by its gain (up to about 6 for silu of N(0, 2^2)
    gates), so an element's error follows its gain, where 1 + |ref| would not."""
    from gpu_harness import rel_errors
    g = gate.double()
    gain = (scale.double() * (g * torch.sigmoid(g) if act == "silu" else torch.sigmoid(g))).abs()
    d = (gpu.double() - ref.double()).abs()
    assert torch.isfinite(gpu.double()).all(), f"{what}: non-finite values"
    e = float((d / (gain + ref.double().abs() + 1e-30)).max())
    fro, mrel = rel_errors(gpu, ref)
    say(f"    {what}: max |d|/(|gain|+|ref|) = {e:.3e} (bound {GROSS * tol:.0e}), ||d||/||ref|| = {fro:.3e} "
        f"(tol {tol:.0e}), max |d|/|ref| over |ref|>=1e-3 = {mrel:.3e}")
    assert fro <= tol, f"{what}: normwise {fro:.3e} > {tol:.0e}"
    assert e <= GROSS * tol, f"{what}: {e:.3e} > {GROSS * tol:.0e}"


def _ref(o, gate, scale, act):
    T, h_v, d_v = o.shape
    y = oracle.default().gated_rmsnorm(o.reshape(T, h_v * d_v), gate.double().reshape(T, h_v * d_v),
                                       scale.double(), eps=1e-5, activation=act)
    return torch.from_numpy(y.reshape(T, h_v, d_v))


PREFILL_CASES = [
    # (workload, overrides, seqlens, two_pass, expected norm form); the fused
    # two-pass epilogue runs from 512 (sequence, head) units (16 x 32 here)
    ("varlen_prefill_8seq", dict(), [70, 65, 130, 0, 64, 99, 71, 66, 200, 64, 80, 65, 64, 64, 90, 64, 3], True,
     "fused"),
    ("varlen_prefill_8seq", dict(h_qk=32, h_v=64, d_v=96), [150, 65, 70, 66, 64, 81, 64, 90], True, "fused"),
    ("varlen_prefill_8seq", dict(h_qk=2, h_v=4, d_v=48), [200, 65], True, "separate pass"),
    ("varlen_prefill_8seq", dict(), [300, 129, 0, 70], True, "separate pass"),
    ("prefill_t4096_fused_gates", dict(), [600], True, "separate pass"),
    ("varlen_prefill_8seq", dict(), [300, 129, 70], False, "separate pass"),
    ("varlen_prefill_8seq", dict(d_v=256, h_qk=2, h_v=4), [130, 70], True, "separate pass"),
    ("wide_prefill_t32768_d256", dict(h_qk=2, h_v=2), [300], True, "separate pass"),
    ("varlen_prefill_8seq", dict(h_qk=2, h_v=4), [20, 5], False, "separate pass"),   # serial
]


@pytest.mark.parametrize("act", ["silu", "sigmoid"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"{c[0]}_{i}" for i, c in enumerate(PREFILL_CASES)])
def test_prefill_with_output_norm(case, act):
    name, over, lens, two_pass, form = case
    shape = dataclasses.replace(W[name], **over)
    inp = synth.generate(shape, seqlens=lens, seed=611)
    raw = shape.gate_mode == "raw"
    g, beta = (None, None) if raw else gates_for(inp)
    T = inp.total_tokens
    gate, scale = synth.output_norm_inputs(T, shape.h_v, shape.d_v, seed=612, io_dtype=shape.io_dtype)
    ws = workspace_for(inp) if two_pass else None
    plan = gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, len(lens), T,
                                  raw_gates=raw, workspace_bytes=0 if ws is None else ws.numel(), norm=True)
    say(f"[norm prefill] {name} {over} {lens} {act}: {plan}")
    assert plan["norm"] == form, plan
    out = torch.full((T, shape.h_v, shape.d_v), float("nan"), dtype=shape.io_dtype, device="cuda")
    fin = torch.empty(len(lens), shape.h_v, shape.d_k, shape.d_v, dtype=torch.float32, device="cuda")
    gates = (dict(a=to_dev(inp.a), b=to_dev(inp.b), A_log=to_dev(inp.A_log), dt_bias=to_dev(inp.dt_bias))
             if raw else dict(g=to_dev(g), beta=to_dev(beta)))
    if ws is not None:
        gates["workspace"] = ws
    gdn.gdn_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), out=out, final_state=fin,
                    initial_state=to_dev(inp.initial_state), cu_seqlens_host=inp.cu_seqlens.tolist(),
                    norm_gate=to_dev(gate), norm_scale=to_dev(scale), norm_activation=act, **gates)
    torch.cuda.synchronize()
    orc = oracle.default()
    if raw:
        g64, b64 = orc.gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    else:
        g64, b64 = g.double().numpy(), beta.double().numpy()
    ro, rf = orc.prefill(inp.q, inp.k, inp.v, g64, b64, inp.cu_seqlens.numpy(),
                         None if inp.initial_state is None else inp.initial_state)
    tol = TOL[shape.io_dtype]
    check_normed(out.double().cpu(), _ref(ro, gate, scale, act), gate, scale, act, tol, "normed out")
    check(fin.double().cpu(), torch.from_numpy(rf), tol, "final state")


@pytest.mark.parametrize("d_v,form", [(128, True), (64, True), (256, False)], ids=["dv128_fused", "dv64_fused",
                                                                                   "dv256_pass"])
def test_decode_with_output_norm(d_v, form):
    """The decode step at its batch of 64 (d_v 128 and 64: the workgroup owns
    the row, fused; 256: a separate pass), two chained steps."""
    shape = dataclasses.replace(W["decode_b64"], d_v=d_v)
    say(f"[norm decode] d_v={d_v}")
    st = None
    ref_state = None
    for step in range(2):
        inp = synth.generate(shape, seed=620 + step)
        g, beta = gates_for(inp)
        if st is None:
            st = to_dev(inp.initial_state).clone()
            ref_state = inp.initial_state.double().numpy().copy()
        gate, scale = synth.output_norm_inputs(64, shape.h_v, d_v, seed=630 + step, io_dtype=torch.bfloat16)
        out = torch.full((64, shape.h_v, d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
        gdn.gdn_decode_step(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), st, out, g=to_dev(g), beta=to_dev(beta),
                            norm_gate=to_dev(gate), norm_scale=to_dev(scale))
        torch.cuda.synchronize()
        ro = oracle.default().decode_step(inp.q, inp.k, inp.v, g.double().numpy(), beta.double().numpy(), ref_state)
        check_normed(out.double().cpu(), _ref(ro, gate, scale, "silu"), gate, scale, "silu", TOL[torch.bfloat16],
                     f"normed out step {step}")
        check(st.double().cpu(), torch.from_numpy(ref_state), TOL[torch.bfloat16], f"state step {step}")


def test_fused_matches_separate_pair():
    """The fused two-pass prefill against the library's unfused pair (prefill,
    then gdn_gated_rmsnorm over its output): same inputs, the pair narrows o
    before normalising, so they agree to the bf16 tolerance."""
    shape = W["varlen_prefill_8seq"]
    inp = synth.generate(shape, seqlens=[400, 257], seed=641)
    g, beta = gates_for(inp)
    T = inp.total_tokens
    gate, scale = synth.output_norm_inputs(T, shape.h_v, shape.d_v, seed=642, io_dtype=torch.bfloat16)
    args = (to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens))
    kw = dict(initial_state=to_dev(inp.initial_state), g=to_dev(g), beta=to_dev(beta),
              cu_seqlens_host=inp.cu_seqlens.tolist(), workspace=workspace_for(inp))
    fused = torch.empty(T, shape.h_v, shape.d_v, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill(*args, out=fused, final_state=None, norm_gate=to_dev(gate), norm_scale=to_dev(scale), **kw)
    o = torch.empty_like(fused)
    gdn.gdn_prefill(*args, out=o, final_state=None, **kw)
    pair = gdn.gated_rmsnorm(o.reshape(T, -1), to_dev(gate).reshape(T, -1), to_dev(scale)).reshape(fused.shape)
    torch.cuda.synchronize()
    check_normed(fused.double().cpu(), pair.double().cpu(), gate, scale, "silu", TOL[torch.bfloat16], "fused vs pair")


@pytest.mark.parametrize("rule,seqlens,form", [
    ("gated", [70, 65, 130, 0, 64, 99, 71, 66, 200, 64, 80, 65, 64, 64, 90, 64, 3], "fused"),
    ("linear", [70, 65, 130, 0, 64, 99, 71, 66, 200, 64, 80, 65, 64, 64, 90, 64, 3], "fused"),
    ("gated", [300, 129, 70], "separate pass"),
    ("linear", [300, 129, 70], "separate pass"),
], ids=["gated_fused", "linear_fused", "gated_pass", "linear_pass"])
def test_plain_rules_with_output_norm(rule, seqlens, form):
    """The gated and linear rules (no delta correction) in the bf16 two-pass
    form with the output norm: from 512 (sequence, head) units the state pass
    runs its 128-column blocks and normalises in its stores, over the records
    of the plain rules (T'' = I, T' = 0); below that, the separate pass."""
    shape = W["varlen_prefill_8seq"]
    inp = synth.generate(shape, seqlens=seqlens, seed=651)
    T, n = inp.total_tokens, len(seqlens)
    g, _ = gates_for(inp)
    gate, scale = synth.output_norm_inputs(T, shape.h_v, shape.d_v, seed=652, io_dtype=torch.bfloat16)
    ws = workspace_for(inp, rule=rule)
    plan = gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T,
                                  workspace_bytes=ws.numel(), rule=rule, norm=True)
    say(f"[norm prefill plain] {rule} {seqlens}: {plan}")
    assert plan["form"] == "chunked_two_pass" and plan["norm"] == form, plan
    out = torch.full((T, shape.h_v, shape.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty(n, shape.h_v, shape.d_k, shape.d_v, dtype=torch.float32, device="cuda")
    gates = dict(g=to_dev(g)) if rule == "gated" else {}
    gdn.gdn_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), out=out, final_state=fin,
                    initial_state=to_dev(inp.initial_state), cu_seqlens_host=inp.cu_seqlens.tolist(), rule=rule,
                    workspace=ws, norm_gate=to_dev(gate), norm_scale=to_dev(scale), **gates)
    torch.cuda.synchronize()
    ro, rf = oracle.default().prefill(inp.q, inp.k, inp.v, g.double().numpy() if rule == "gated" else None, None,
                                      inp.cu_seqlens.numpy(), inp.initial_state, rule=rule)
    tol = TOL[torch.bfloat16]
    check_normed(out.double().cpu(), _ref(ro, gate, scale, "silu"), gate, scale, "silu", tol, "normed out")
    check(fin.double().cpu(), torch.from_numpy(rf), tol, "final state")


def test_slot_pool_with_output_norm():
    """The output norm through the slot-pool entry points: a two-pass prefill of
    17 sequences (544 units: the fused state pass) into a pool of 20 slots,
    one of them padding, then one decode step over the same slots (fused)."""
    shape = W["varlen_prefill_8seq"]
    lens = [70, 65, 130, 0, 64, 99, 71, 66, 200, 64, 80, 65, 64, 64, 90, 64, 3]
    slots = [19, 0, 7, 3, -1, 12, 1, 18, 5, 9, 2, 16, 11, 4, 14, 8, 6]
    n, num_slots = len(lens), 20
    inp = synth.generate(dataclasses.replace(shape, init_state=False), seqlens=lens, seed=661)
    T = inp.total_tokens
    g, beta = gates_for(inp)
    gen = torch.Generator().manual_seed(662)
    pool = torch.randn(num_slots, shape.h_v, shape.d_k, shape.d_v, generator=gen) * 0.05
    pool_gpu = pool.cuda()
    slots_dev = torch.tensor(slots, dtype=torch.int32, device="cuda")
    gate, scale = synth.output_norm_inputs(T, shape.h_v, shape.d_v, seed=663, io_dtype=torch.bfloat16)
    ws = workspace_for(inp)
    plan = gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, n, T,
                                  workspace_bytes=ws.numel(), norm=True)
    say(f"[norm slots] prefill {plan}")
    assert plan["norm"] == "fused", plan
    out = torch.full((T, shape.h_v, shape.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_slots(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), pool_gpu, slots_dev,
                          out=out, g=to_dev(g), beta=to_dev(beta), cu_seqlens_host=inp.cu_seqlens.tolist(),
                          slots_host=slots, workspace=ws, norm_gate=to_dev(gate), norm_scale=to_dev(scale))
    torch.cuda.synchronize()
    s0 = torch.stack([pool[s] if s >= 0 else torch.zeros(pool.shape[1:]) for s in slots])
    ro, rf = oracle.default().prefill(inp.q, inp.k, inp.v, g.double().numpy(), beta.double().numpy(),
                                      inp.cu_seqlens.numpy(), s0)
    ref_pool = pool.double().clone()
    for i, s in enumerate(slots):
        if s >= 0:
            ref_pool[s] = torch.from_numpy(rf[i])
    tol = TOL[torch.bfloat16]
    check_normed(out.double().cpu(), _ref(ro, gate, scale, "silu"), gate, scale, "silu", tol, "prefill normed out")
    check(pool_gpu.double().cpu(), ref_pool, tol, "pool after prefill")
    for s in (10, 13, 15, 17):
        assert torch.equal(pool_gpu[s].cpu(), pool[s]), f"untouched slot {s} changed"
    # one decode token per sequence over the same slots, the norm fused in the step
    dinp = synth.generate(dataclasses.replace(W["decode_b64"], num_seqs=n), seed=664)
    dg, db = gates_for(dinp)
    dgate, dscale = synth.output_norm_inputs(n, shape.h_v, shape.d_v, seed=665, io_dtype=torch.bfloat16)
    before = pool_gpu.double().cpu()
    dout = torch.full((n, shape.h_v, shape.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_step_slots(to_dev(dinp.q), to_dev(dinp.k), to_dev(dinp.v), pool_gpu, slots_dev, dout,
                              g=to_dev(dg), beta=to_dev(db), slots_host=slots, norm_gate=to_dev(dgate),
                              norm_scale=to_dev(dscale))
    torch.cuda.synchronize()
    st = torch.stack([before[s] if s >= 0 else torch.zeros(pool.shape[1:], dtype=torch.float64)
                      for s in slots]).numpy().copy()
    do = oracle.default().decode_step(dinp.q, dinp.k, dinp.v, dg.double().numpy(), db.double().numpy(), st)
    ref_pool = before.clone()
    for i, s in enumerate(slots):
        if s >= 0:
            ref_pool[s] = torch.from_numpy(st[i])
    check_normed(dout.double().cpu(), _ref(do, dgate, dscale, "silu"), dgate, dscale, "silu", tol,
                 "decode normed out")
    check(pool_gpu.double().cpu(), ref_pool, tol, "pool after decode")
