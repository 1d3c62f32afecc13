"""GPU parity of the variants the pages define, against the oracle: the update
rules (linear / gated / delta / gated delta), per-key-dim decay, one beta per
token shared by the heads, and the per-step state history -- through the
serial scan, the decode step and (where it applies) the chunked prefill."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, say, to_dev

pytestmark = pytest.mark.gpu

RULES = ["gated_delta", "delta", "gated", "linear"]


def _setup(h_qk, h_v, d_k, d_v, dt, lens, *, seed, per_key=False, shared=False, init=True):
    shape = dataclasses.replace(synth.BY_NAME["tiny_prefill"], h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v,
                                io_dtype=dt, init_state=init)
    inp = synth.generate(shape, seqlens=lens, seed=seed)
    vg = synth.variant_gates(inp.total_tokens, h_v, d_k, seed=seed + 1, io_dtype=dt)
    orc = oracle.default()
    T = inp.total_tokens
    # raw inputs of each layout, and the oracle's gates from exactly those values
    a = vg.a_key if per_key else inp.a
    A_log = vg.A_log_key if per_key else inp.A_log
    dt_bias = vg.dt_bias_key if per_key else inp.dt_bias
    b = vg.b_shared if shared else inp.b
    if per_key:
        g64, _ = orc.gates(a.reshape(T, h_v * d_k), a.reshape(T, h_v * d_k), A_log.reshape(-1),
                           dt_bias.reshape(-1))
        g64 = g64.reshape(T, h_v, d_k)
    else:
        g64, _ = orc.gates(a, a, A_log, dt_bias)
    _, b64 = orc.gates(b.reshape(-1, 1), b.reshape(-1, 1), torch.zeros(1), torch.zeros(1))
    b64 = b64.reshape(b.shape)
    return inp, dict(a=a, b=b, A_log=A_log, dt_bias=dt_bias), g64, b64


def _oracle(inp, g, beta, *, rule, per_key, shared, window=0):
    orc = oracle.default()
    uses_g = rule in ("gated", "gated_delta")
    uses_b = rule in ("delta", "gated_delta")
    return orc.prefill(inp.q, inp.k, inp.v, g if uses_g else None, beta if uses_b else None,
                       inp.cu_seqlens.numpy(), inp.initial_state, rule=rule, decay_per_key=per_key,
                       beta_shared=shared, window=window)


def _gpu_prefill(inp, gates, *, raw, rule, per_key, shared, window=0, algorithm="serial", two_pass=False):
    dev = "cuda"
    T, n = inp.total_tokens, len(inp.seqlens)
    h_v, d_k, d_v = inp.shape.h_v, inp.shape.d_k, inp.shape.d_v
    out = torch.full((T, h_v, d_v), float("nan"), dtype=inp.shape.io_dtype, device=dev)
    fin = torch.full((n, h_v, d_k, d_v), float("nan"), device=dev)
    hist = torch.full((n, window, h_v, d_k, d_v), float("nan"), device=dev) if window else None
    kw = {k: to_dev(v) for k, v in gates.items()}
    if two_pass:
        sh = inp.shape
        nbytes = gdn.prefill_workspace_size(sh.h_qk, sh.h_v, sh.d_k, sh.d_v, sh.io_dtype, n, T, algorithm=algorithm,
                                            rule=rule, decay_per_key=per_key, beta_shared=shared)
        assert nbytes > 0
        kw["workspace"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    gdn.gdn_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), out=out, final_state=fin,
                    initial_state=to_dev(inp.initial_state), cu_seqlens_host=inp.cu_seqlens.tolist(),
                    algorithm=algorithm, rule=rule, decay_per_key=per_key, beta_shared=shared,
                    state_history=hist, **kw)
    torch.cuda.synchronize()
    return out.double().cpu(), fin.double().cpu(), (None if hist is None else hist.double().cpu())


def _gate_kwargs(raw, raw_in, g64, b64, dt):
    if raw:
        return dict(raw_in)
    return dict(g=torch.from_numpy(g64).to(dt), beta=torch.from_numpy(b64).to(dt))


CASES = [
    # (h_qk, h_v, d_k, d_v, dtype, seqlens)
    (2, 4, 48, 40, torch.float32, [70, 0, 13]),
    (16, 32, 128, 128, torch.bfloat16, [150, 66]),
    (1, 2, 256, 64, torch.float32, [33]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"dk{c[2]}_dv{c[3]}_{str(c[4])[6:]}")
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_rules_serial(case, rule, raw):
    h_qk, h_v, d_k, d_v, dt, lens = case
    say(f"[rule] {rule} raw={raw} {case}")
    inp, raw_in, g64, b64 = _setup(h_qk, h_v, d_k, d_v, dt, lens, seed=200)
    gates = _gate_kwargs(raw, raw_in, g64, b64, dt)
    # the oracle sees the gates the kernel reads: rounded to the I/O dtype when precomputed
    if not raw:
        g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    out, fin, _ = _gpu_prefill(inp, gates, raw=raw, rule=rule, per_key=False, shared=False)
    ro, rf = _oracle(inp, g64, b64, rule=rule, per_key=False, shared=False)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"dk{c[2]}_dv{c[3]}_{str(c[4])[6:]}")
@pytest.mark.parametrize("per_key,shared", [(True, False), (False, True), (True, True)],
                         ids=["perkey", "sharedbeta", "both"])
@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_layouts_serial(case, per_key, shared, raw):
    h_qk, h_v, d_k, d_v, dt, lens = case
    say(f"[layout] per_key={per_key} shared={shared} raw={raw} {case}")
    inp, raw_in, g64, b64 = _setup(h_qk, h_v, d_k, d_v, dt, lens, seed=300, per_key=per_key, shared=shared)
    gates = _gate_kwargs(raw, raw_in, g64, b64, dt)
    if not raw:
        g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    out, fin, _ = _gpu_prefill(inp, gates, raw=raw, rule="gated_delta", per_key=per_key, shared=shared)
    ro, rf = _oracle(inp, g64, b64, rule="gated_delta", per_key=per_key, shared=shared)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")


@pytest.mark.parametrize("window", [1, 4, 80])
def test_state_history(window):
    dt = torch.float32
    say(f"[history] W={window}")
    inp, raw_in, g64, b64 = _setup(2, 4, 32, 24, dt, [70, 0, 3, 9], seed=400)
    gates = _gate_kwargs(False, raw_in, g64, b64, dt)
    g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    out, fin, hist = _gpu_prefill(inp, gates, raw=False, rule="gated_delta", per_key=False, shared=False,
                                  window=window)
    ro, rf, rh = _oracle(inp, g64, b64, rule="gated_delta", per_key=False, shared=False, window=window)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")
    check(hist, torch.from_numpy(rh), TOL[dt], "history")


@pytest.mark.parametrize("shared", [False, True], ids=["perhead", "sharedbeta"])
@pytest.mark.parametrize("rule", ["gated_delta", "delta"])
@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "two_pass"])
def test_chunked_rules_and_shared_beta(rule, shared, two_pass):
    dt = torch.bfloat16
    say(f"[chunked-variant] {rule} shared={shared} two_pass={two_pass}")
    inp, raw_in, g64, b64 = _setup(16, 32, 128, 128, dt, [150, 70, 1], seed=500, shared=shared)
    gates = _gate_kwargs(True, raw_in, g64, b64, dt)
    out, fin, _ = _gpu_prefill(inp, gates, raw=True, rule=rule, per_key=False, shared=shared, algorithm="chunked",
                               two_pass=two_pass)
    ro, rf = _oracle(inp, g64, b64, rule=rule, per_key=False, shared=shared)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")


PLAIN_GEOMS = [
    # (h_qk, h_v, d_k, d_v, seqlens, raw gates): head ratio 2 (paired preparation units), 3 (one head
    # per unit), d_v 256 (four 64-column state blocks), a ragged d_v, a long sequence (the linear
    # rule's state grows with it)
    (16, 32, 128, 128, [150, 70, 1], True),
    (2, 6, 64, 64, [200, 0, 65], False),
    (1, 1, 128, 256, [300], False),
    (2, 2, 64, 40, [129, 64], True),
    (4, 8, 128, 128, [2048], False),
]


@pytest.mark.parametrize("geom", PLAIN_GEOMS, ids=lambda g: f"h{g[0]}x{g[1]}_dk{g[2]}_dv{g[3]}_T{sum(g[4])}")
@pytest.mark.parametrize("rule", ["gated", "linear"])
def test_chunked_two_pass_plain_rules(rule, geom):
    """The gated and linear rules (no delta correction) in the bfloat16 two-pass chunked form,
    as AUTO plans it with a workspace: the preparation pass writes T'' = I and T' = 0, so the
    state pass takes D = V."""
    h_qk, h_v, d_k, d_v, lens, raw = geom
    dt = torch.bfloat16
    say(f"[chunked-plain] {rule} {geom}")
    inp, raw_in, g64, b64 = _setup(h_qk, h_v, d_k, d_v, dt, lens, seed=540)
    gates = _gate_kwargs(raw, raw_in, g64, b64, dt)
    if not raw:
        g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    n, T = len(lens), inp.total_tokens
    ws = gdn.prefill_workspace_size(h_qk, h_v, d_k, d_v, dt, n, T, rule=rule)
    plan = gdn.prefill_query_plan(h_qk, h_v, d_k, d_v, dt, n, T, raw_gates=raw, workspace_bytes=ws, rule=rule)
    assert plan["form"] == "chunked_two_pass" and "chunk_trec_kernel" in plan["kernels"], plan
    out, fin, _ = _gpu_prefill(inp, gates, raw=raw, rule=rule, per_key=False, shared=False, algorithm="auto",
                               two_pass=True)
    ro, rf = _oracle(inp, g64, b64, rule=rule, per_key=False, shared=False)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")


@pytest.mark.parametrize("rule", ["gated", "linear", "delta"])
def test_rules_through_slot_pool(rule):
    """The rules other than gated delta through the slot pool: the two-pass
    prefill (plain rules: the small plain record) and then one decode step
    over the same pool.  Slot -1 is padding; untouched slots stay
    bit-identical."""
    h_qk, h_v, d_k, d_v, dt = 16, 32, 128, 128, torch.bfloat16
    lens, slots = [70, 0, 33, 129], [5, -1, 2, 0]
    inp, raw_in, g64, b64 = _setup(h_qk, h_v, d_k, d_v, dt, lens, seed=560, init=False)
    gates = _gate_kwargs(False, raw_in, g64, b64, dt)
    g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    uses_g, uses_b = rule == "gated", rule == "delta"
    kw = {k: to_dev(v) for k, v in gates.items() if (k == "g" and uses_g) or (k == "beta" and uses_b)}
    n, T = len(lens), inp.total_tokens
    gen = torch.Generator().manual_seed(561)
    pool = torch.randn(6, h_v, d_k, d_v, generator=gen) * 0.05
    pool_gpu = pool.cuda()
    ws = gdn.prefill_workspace_size(h_qk, h_v, d_k, d_v, dt, n, T, rule=rule)
    say(f"[rules-slots] {rule} slots={slots} workspace={ws}")
    out = torch.full((T, h_v, d_v), float("nan"), dtype=dt, device="cuda")
    gdn.gdn_prefill_slots(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), pool_gpu,
                          torch.tensor(slots, dtype=torch.int32, device="cuda"), out=out,
                          cu_seqlens_host=inp.cu_seqlens.tolist(), slots_host=slots, rule=rule,
                          workspace=torch.empty(ws, dtype=torch.uint8, device="cuda"), **kw)
    torch.cuda.synchronize()
    s0 = torch.stack([pool[s] if s >= 0 else torch.zeros(pool.shape[1:]) for s in slots])
    ro, rf = _oracle(dataclasses.replace(inp, initial_state=s0), g64, b64, rule=rule, per_key=False, shared=False)
    ref_pool = pool.double().clone()
    for i, s in enumerate(slots):
        if s >= 0:
            ref_pool[s] = torch.from_numpy(rf[i])
    check(out.double().cpu(), torch.from_numpy(ro), TOL[dt], "prefill out")
    check(pool_gpu.double().cpu(), ref_pool, TOL[dt], "pool after prefill")
    for s in (1, 3, 4):
        assert torch.equal(pool_gpu[s].cpu(), pool[s]), f"untouched slot {s} changed"
    # one decode token per sequence over the pool the prefill left
    dinp, draw, dg, db = _setup(h_qk, h_v, d_k, d_v, dt, [1] * n, seed=562, init=False)
    dgates = _gate_kwargs(False, draw, dg, db, dt)
    dg, db = dgates["g"].double().numpy(), dgates["beta"].double().numpy()
    dkw = {k: to_dev(v) for k, v in dgates.items() if (k == "g" and uses_g) or (k == "beta" and uses_b)}
    before = pool_gpu.double().cpu()
    dout = torch.full((n, h_v, d_v), float("nan"), dtype=dt, device="cuda")
    gdn.gdn_decode_step_slots(to_dev(dinp.q), to_dev(dinp.k), to_dev(dinp.v), pool_gpu,
                              torch.tensor(slots, dtype=torch.int32, device="cuda"), dout, slots_host=slots,
                              rule=rule, **dkw)
    torch.cuda.synchronize()
    s1 = torch.stack([before[s] if s >= 0 else torch.zeros(pool.shape[1:], dtype=torch.float64) for s in slots])
    do, df = _oracle(dataclasses.replace(dinp, initial_state=s1), dg, db, rule=rule, per_key=False, shared=False)
    ref_pool = before.clone()
    for i, s in enumerate(slots):
        if s >= 0:
            ref_pool[s] = torch.from_numpy(df[i])
    check(dout.double().cpu(), torch.from_numpy(do), TOL[dt], "decode out")
    check(pool_gpu.double().cpu(), ref_pool, TOL[dt], "pool after decode")


F32_PLAIN_GEOMS = [
    # (h_qk, h_v, d_k, d_v, seqlens, raw gates): d_k 128 and 256, d_v 32 to 256, ragged tails, an
    # empty and a one-token sequence
    (2, 4, 128, 32, [200, 0, 70, 1], False),
    (1, 2, 256, 64, [300], True),
    (2, 2, 256, 256, [200, 64], False),
]


@pytest.mark.parametrize("geom", F32_PLAIN_GEOMS, ids=lambda g: f"h{g[0]}x{g[1]}_dk{g[2]}_dv{g[3]}_T{sum(g[4])}")
@pytest.mark.parametrize("rule", ["gated", "linear"])
def test_chunked_f32_plain_rules(rule, geom):
    """The gated and linear rules in the float32 two-pass chunked form, as AUTO plans it with a
    workspace: the preparation pass forms A = 0, so T = I, W = 0 and U = V, and the state pass
    takes D = V."""
    h_qk, h_v, d_k, d_v, lens, raw = geom
    dt = torch.float32
    say(f"[chunked-f32-plain] {rule} {geom}")
    inp, raw_in, g64, b64 = _setup(h_qk, h_v, d_k, d_v, dt, lens, seed=570)
    gates = _gate_kwargs(raw, raw_in, g64, b64, dt)
    if not raw:
        g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    n, T = len(lens), inp.total_tokens
    ws = gdn.prefill_workspace_size(h_qk, h_v, d_k, d_v, dt, n, T, rule=rule)
    plan = gdn.prefill_query_plan(h_qk, h_v, d_k, d_v, dt, n, T, raw_gates=raw, workspace_bytes=ws, rule=rule)
    assert plan["form"] == "chunked_f32", plan
    out, fin, _ = _gpu_prefill(inp, gates, raw=raw, rule=rule, per_key=False, shared=False, algorithm="auto",
                               two_pass=True)
    ro, rf = _oracle(inp, g64, b64, rule=rule, per_key=False, shared=False)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")


@pytest.mark.parametrize("geom", [(16, 32, 128, 128, [300, 0, 70, 1], True), (2, 6, 64, 40, [200, 65], False)],
                         ids=["h16x32_dk128_dv128", "h2x6_dk64_dv40"])
@pytest.mark.parametrize("rule", ["gated", "linear"])
def test_chunked_one_pass_plain_rules(rule, geom):
    """Without a workspace the gated and linear rules take the one-pass chunked form, as AUTO
    plans it: A = 0, so T = I, T' = 0 and T'' = I, and D = V."""
    h_qk, h_v, d_k, d_v, lens, raw = geom
    dt = torch.bfloat16
    say(f"[chunked-one-pass-plain] {rule} {geom}")
    inp, raw_in, g64, b64 = _setup(h_qk, h_v, d_k, d_v, dt, lens, seed=580)
    gates = _gate_kwargs(raw, raw_in, g64, b64, dt)
    if not raw:
        g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    n, T = len(lens), inp.total_tokens
    plan = gdn.prefill_query_plan(h_qk, h_v, d_k, d_v, dt, n, T, raw_gates=raw, rule=rule)
    assert plan["form"] == "chunked_one_pass", plan
    out, fin, _ = _gpu_prefill(inp, gates, raw=raw, rule=rule, per_key=False, shared=False, algorithm="auto")
    ro, rf = _oracle(inp, g64, b64, rule=rule, per_key=False, shared=False)
    check(out, torch.from_numpy(ro), TOL[dt], "out")
    check(fin, torch.from_numpy(rf), TOL[dt], "final state")


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("per_key,shared", [(False, False), (True, False), (False, True), (True, True)],
                         ids=["plain", "perkey", "sharedbeta", "both"])
@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_decode_variants(rule, per_key, shared, raw):
    dt = torch.bfloat16
    say(f"[decode-variant] {rule} per_key={per_key} shared={shared} raw={raw}")
    inp, raw_in, g64, b64 = _setup(2, 4, 64, 80, dt, [1] * 5, seed=600, per_key=per_key, shared=shared)
    gates = _gate_kwargs(raw, raw_in, g64, b64, dt)
    if not raw:
        g64, b64 = gates["g"].double().numpy(), gates["beta"].double().numpy()
    st = to_dev(inp.initial_state).clone()
    out = gdn.decode_step(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), st, rule=rule, decay_per_key=per_key,
                          beta_shared=shared, **{k: to_dev(v) for k, v in gates.items()})
    torch.cuda.synchronize()
    ro, rf = _oracle(inp, g64, b64, rule=rule, per_key=per_key, shared=shared)
    check(out.double().cpu(), torch.from_numpy(ro), TOL[dt], "out")
    check(st.double().cpu(), torch.from_numpy(rf), TOL[dt], "state")
