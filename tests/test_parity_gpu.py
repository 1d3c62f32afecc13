"""GPU parity: the HIP library (through its C ABI) against the oracle, element
by element, on seeded synthetic inputs.

Reduced sizes cover every workload's geometry with ragged tails (token counts
that are not multiples of the 4-token prefetch ring or the 64-token gate
block, column counts that are not multiples of a wave's column block).  The
full-size cases run the library exactly as the benchmark launches it and
compare sampled (q/k head group) slices that the oracle computes alone.

Tolerance: |gpu - ref| <= tol (1 + |ref|) elementwise, tol = 1e-4 for float32
I/O, 1e-2 for bfloat16 I/O and 1e-3 for float16 I/O.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, gates_for, gpu_prefill, oracle_prefill, say, to_dev, workspace_for

pytestmark = pytest.mark.gpu

W = synth.BY_NAME


def _shape(base="tiny_prefill", **kw):
    return dataclasses.replace(W[base], **kw)


# ------------------------------------------------------------------ prefill, reduced sizes
PREFILL_CASES = [
    ("tiny_prefill", {}),
    ("prefill_t4096_fused_gates", dict(seqlen=200)),
    ("varlen_prefill_8seq", dict(seqlens=[37, 0, 129, 64, 1, 250, 3])),
    ("wide_prefill_t32768_d256", dict(seqlen=97)),
]


@pytest.mark.parametrize("algorithm", ["serial", "auto"])
@pytest.mark.parametrize("name,over", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_workload_geometry(name, over, algorithm):
    shape = W[name]
    say(f"[prefill] {name} {over} {algorithm}")
    inp = synth.generate(shape, **over)
    raw = shape.gate_mode == "raw"
    g, beta = (None, None) if raw else gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm=algorithm)
    ro, rf = oracle_prefill(inp, g, beta, raw=raw)
    tol = TOL[shape.io_dtype]
    check(out, ro, tol, "out")
    check(fin, rf, tol, "final state")


GEOMETRIES = [
    # (h_qk, h_v, d_k, d_v, dtype, seqlens)
    (1, 1, 1, 1, torch.float32, [5, 9]),
    (1, 4, 48, 40, torch.bfloat16, [70, 0, 13]),
    (2, 2, 100, 130, torch.float32, [66]),
    (3, 6, 256, 256, torch.bfloat16, [21, 2]),
    (1, 1, 16, 3, torch.float32, [130]),
    (4, 8, 64, 64, torch.bfloat16, [65, 64, 63]),
    (1, 2, 32, 200, torch.float32, [9, 17]),
    (2, 4, 128, 128, torch.float32, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]),
    (2, 4, 128, 128, torch.float16, [70, 0, 13]),
    (1, 1, 16, 3, torch.float16, [130]),
    (3, 6, 256, 256, torch.float16, [21, 2]),
]


@pytest.mark.parametrize("geom", GEOMETRIES, ids=lambda g: f"hq{g[0]}_hv{g[1]}_dk{g[2]}_dv{g[3]}_{str(g[4])[6:]}")
@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_prefill_geometry(geom, raw):
    h_qk, h_v, d_k, d_v, dt, lens = geom
    shape = _shape(h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, io_dtype=dt, init_state=True,
                   gate_mode="raw" if raw else "precomputed")
    say(f"[prefill-geom] {geom} raw={raw}")
    inp = synth.generate(shape, seqlens=lens, seed=77)
    g, beta = (None, None) if raw else gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm="serial")
    ro, rf = oracle_prefill(inp, g, beta, raw=raw)
    check(out, ro, TOL[dt], "out")
    check(fin, rf, TOL[dt], "final state")


# ------------------------------------------------------------------ the d_k = 256 wide scan
# The plain rule at d_k = 256 runs its own kernel: two columns per wave, whole
# 64-token blocks unguarded while the 16-token ring stays inside the sequence
# (from 64 + 16 = 80 tokens on), a guarded tail in groups of 16.  Lengths
# around those edges, an odd d_v (the second column of the last wave is
# padding), every I/O dtype, precomputed and raw gates.
WIDE_CASES = [
    (torch.float32, 255, [1, 15, 16, 79, 80, 81, 200]),
    (torch.bfloat16, 256, [81, 145, 0, 17]),
    (torch.float16, 33, [96, 97, 5]),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: f"dv{c[1]}_{str(c[0])[6:]}")
@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_wide_scan_blocks_and_tails(case, raw):
    dt, d_v, lens = case
    shape = _shape("wide_prefill_t32768_d256", h_qk=2, h_v=4, d_v=d_v, io_dtype=dt, init_state=True,
                   gate_mode="raw" if raw else "precomputed")
    say(f"[wide] d_v={d_v} {dt} lens={lens} raw={raw}")
    inp = synth.generate(shape, seqlens=lens, seed=11)
    g, beta = (None, None) if raw else gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm="serial")
    ro, rf = oracle_prefill(inp, g, beta, raw=raw)
    check(out, ro, TOL[dt], "out")
    check(fin, rf, TOL[dt], "final state")


def test_prefill_options():
    """Explicit scale, in-place state, out or state omitted, no host cu_seqlens."""
    shape = _shape("varlen_prefill_8seq", init_state=True)
    inp = synth.generate(shape, seqlens=[40, 3, 0, 77])
    g, beta = gates_for(inp)
    ro, rf = oracle_prefill(inp, g, beta, scale=0.3)
    tol = TOL[shape.io_dtype]
    say("[prefill-options] scale 0.3 + in place")
    out, fin = gpu_prefill(inp, g, beta, scale=0.3, in_place=True)
    check(out, ro, tol, "out (in place)")
    check(fin, rf, tol, "state (in place)")
    say("[prefill-options] state only, no host cu")
    out, fin = gpu_prefill(inp, g, beta, scale=0.3, want_out=False, use_host_cu=False)
    assert out is None
    check(fin, rf, tol, "state only")
    say("[prefill-options] out only")
    out, fin = gpu_prefill(inp, g, beta, scale=0.3, want_state=False)
    assert fin is None
    check(out, ro, tol, "out only")


def test_prefill_no_tokens_returns_initial_state():
    shape = _shape(init_state=True)
    inp = synth.generate(shape, seqlens=[0, 0, 0])
    g, beta = gates_for(inp)
    say("[prefill-empty] three empty sequences")
    out, fin = gpu_prefill(inp, g, beta)
    assert out.shape[0] == 0
    assert torch.equal(fin, inp.initial_state.double())
    shape0 = _shape(init_state=False)
    inp0 = synth.generate(shape0, seqlens=[0, 4, 0])
    g0, b0 = gates_for(inp0)
    out0, fin0 = gpu_prefill(inp0, g0, b0)
    assert torch.equal(fin0[0], torch.zeros_like(fin0[0])) and torch.equal(fin0[2], torch.zeros_like(fin0[2]))


def test_rounding_tie_to_even():
    """q = k = e0, g = 0, beta = 1/2, S0 = e0 e0^T, v = 1.0078125, scale 1, bf16 I/O:
    the exact outputs 1.00390625 (a bf16 tie) and 1.005859375 round to 1.0 and
    1.0078125.  Prefill and two decode steps."""
    d = 16
    q = torch.zeros(2, 1, d)
    q[:, 0, 0] = 1.0
    v = torch.zeros(2, 1, d)
    v[:, 0, 0] = 1.0078125
    s0 = torch.zeros(1, 1, d, d)
    s0[0, 0, 0, 0] = 1.0
    bf = torch.bfloat16
    dev = "cuda"
    g = torch.zeros(2, 1, dtype=bf, device=dev)
    beta = torch.full((2, 1), 0.5, dtype=bf, device=dev)
    qd = q.to(bf).to(dev)
    say("[rounding] prefill")
    out, fin = gdn.prefill(qd, qd, v.to(bf).to(dev), torch.tensor([0, 2], dtype=torch.int32, device=dev),
                           initial_state=s0.to(dev), g=g, beta=beta, scale=1.0)
    torch.cuda.synchronize()
    assert out[:, 0, 0].float().tolist() == [1.0, 1.0078125]
    assert fin[0, 0, 0, 0].item() == 1.005859375
    say("[rounding] decode")
    st = s0.to(dev).clone()
    outs = [gdn.decode_step(qd[t:t + 1], qd[t:t + 1], v[t:t + 1].to(bf).to(dev), st, g=g[t:t + 1],
                            beta=beta[t:t + 1], scale=1.0) for t in range(2)]
    torch.cuda.synchronize()
    assert [o[0, 0, 0].item() for o in outs] == [1.0, 1.0078125]
    assert st[0, 0, 0, 0].item() == 1.005859375


def test_rounding_tie_to_even_f16():
    """The float16 form of the same question: v = 1 + 2^-10 gives the exact
    outputs 1 + 2^-11 (a float16 tie, to 1.0) and 1 + 3 2^-12 (to 1 + 2^-10)."""
    d = 16
    q = torch.zeros(2, 1, d)
    q[:, 0, 0] = 1.0
    v = torch.zeros(2, 1, d)
    v[:, 0, 0] = 1.0 + 2.0 ** -10
    s0 = torch.zeros(1, 1, d, d)
    s0[0, 0, 0, 0] = 1.0
    hf = torch.float16
    dev = "cuda"
    g = torch.zeros(2, 1, dtype=hf, device=dev)
    beta = torch.full((2, 1), 0.5, dtype=hf, device=dev)
    qd = q.to(hf).to(dev)
    say("[rounding-f16] prefill")
    out, fin = gdn.prefill(qd, qd, v.to(hf).to(dev), torch.tensor([0, 2], dtype=torch.int32, device=dev),
                           initial_state=s0.to(dev), g=g, beta=beta, scale=1.0)
    torch.cuda.synchronize()
    assert out[:, 0, 0].float().tolist() == [1.0, 1.0 + 2.0 ** -10]
    assert fin[0, 0, 0, 0].item() == 1.0 + 3 * 2.0 ** -12
    say("[rounding-f16] decode")
    st = s0.to(dev).clone()
    outs = [gdn.decode_step(qd[t:t + 1], qd[t:t + 1], v[t:t + 1].to(hf).to(dev), st, g=g[t:t + 1],
                            beta=beta[t:t + 1], scale=1.0) for t in range(2)]
    torch.cuda.synchronize()
    assert [o[0, 0, 0].item() for o in outs] == [1.0, 1.0 + 2.0 ** -10]
    assert st[0, 0, 0, 0].item() == 1.0 + 3 * 2.0 ** -12


# ------------------------------------------------------------------ decode
def _decode_inputs(shape, seed):
    inp = synth.generate(shape, seed=seed)
    g, beta = gates_for(inp)
    return inp, g, beta


@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_decode_b64_full(raw):
    """The decode workload at its full size (B = 64), three chained steps."""
    shape = W["decode_b64"]
    say(f"[decode] B=64 full, raw={raw}")
    inp0 = synth.generate(shape)
    st_gpu = to_dev(inp0.initial_state).clone()
    st_ref = inp0.initial_state.double().numpy().copy()
    orc = oracle.default()
    tol = TOL[shape.io_dtype]
    for step in range(3):
        inp = synth.generate(shape, seed=5000 + step)
        if raw:
            gates = dict(a=to_dev(inp.a), b=to_dev(inp.b), A_log=to_dev(inp.A_log), dt_bias=to_dev(inp.dt_bias))
            gr, br = orc.gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
        else:
            g, beta = gates_for(inp)
            gates = dict(g=to_dev(g), beta=to_dev(beta))
            gr, br = g.double().numpy(), beta.double().numpy()
        out = gdn.decode_step(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), st_gpu, **gates)
        torch.cuda.synchronize()
        ro = orc.decode_step(inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy(), gr, br, st_ref)
        check(out.double().cpu(), torch.from_numpy(ro), tol, f"out step {step}")
        check(st_gpu.double().cpu(), torch.from_numpy(st_ref), tol, f"state step {step}")


DECODE_GEOMS = [
    (1, 1, 16, 16, torch.float32, 3),
    (2, 4, 48, 40, torch.bfloat16, 5),
    (1, 1, 256, 256, torch.float32, 2),
    (3, 6, 100, 130, torch.bfloat16, 4),
    (1, 2, 1, 1, torch.float32, 7),
    (2, 2, 128, 66, torch.float32, 3),
    (16, 32, 128, 128, torch.float16, 8),
    (1, 1, 48, 40, torch.float16, 3),
]


@pytest.mark.parametrize("geom", DECODE_GEOMS, ids=lambda g: f"hq{g[0]}_hv{g[1]}_dk{g[2]}_dv{g[3]}_B{g[5]}")
def test_decode_geometry(geom):
    h_qk, h_v, d_k, d_v, dt, B = geom
    shape = _shape("decode_b64", h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, io_dtype=dt, num_seqs=B)
    say(f"[decode-geom] {geom}")
    inp, g, beta = _decode_inputs(shape, 91)
    st = to_dev(inp.initial_state).clone()
    out = gdn.decode_step(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), st, g=to_dev(g), beta=to_dev(beta))
    torch.cuda.synchronize()
    ref_state = inp.initial_state.double().numpy().copy()
    ro = oracle.default().decode_step(inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy(),
                                      g.double().numpy(), beta.double().numpy(), ref_state)
    check(out.double().cpu(), torch.from_numpy(ro), TOL[dt], "out")
    check(st.double().cpu(), torch.from_numpy(ref_state), TOL[dt], "state")


def test_decode_steps_equal_prefill():
    """T decode steps of one sequence reproduce a T-token prefill."""
    shape = _shape("varlen_prefill_8seq", init_state=True)
    inp = synth.generate(shape, seqlens=[6])
    g, beta = gates_for(inp)
    say("[decode-vs-prefill] 6 steps")
    out_p, fin_p = gpu_prefill(inp, g, beta)
    st = to_dev(inp.initial_state).clone()
    outs = []
    for t in range(6):
        outs.append(gdn.decode_step(to_dev(inp.q[t:t + 1]), to_dev(inp.k[t:t + 1]), to_dev(inp.v[t:t + 1]), st,
                                    g=to_dev(g[t:t + 1]), beta=to_dev(beta[t:t + 1])))
    torch.cuda.synchronize()
    tol = TOL[shape.io_dtype]
    check(torch.cat(outs).double().cpu(), out_p, tol, "decode vs prefill out")
    check(st.double().cpu(), fin_p, tol, "decode vs prefill state")


# ------------------------------------------------------------------ gate prologue
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16], ids=["f32", "bf16", "f16"])
def test_gate_prologue(dt):
    shape = _shape("prefill_t4096_fused_gates", io_dtype=dt)
    inp = synth.generate(shape, seqlen=333)
    say(f"[gates] {dt}")
    g, beta = gdn.gate_prologue(to_dev(inp.a), to_dev(inp.b), to_dev(inp.A_log), to_dev(inp.dt_bias))
    torch.cuda.synchronize()
    rg, rb = oracle.default().gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    check(g.double().cpu(), torch.from_numpy(rg), TOL[dt], "g")
    check(beta.double().cpu(), torch.from_numpy(rb), TOL[dt], "beta")


# ------------------------------------------------------------------ chunked (matrix-core) prefill
CHUNKED = [
    # (h_qk, h_v, d_k, d_v, seqlens, raw gates, initial state)
    (16, 32, 128, 128, [200], True, False),
    (16, 32, 128, 128, [37, 0, 129, 64, 1, 250, 3], False, True),
    (2, 4, 64, 40, [70, 0, 13, 64], False, True),
    (1, 2, 128, 200, [130], True, True),
    (4, 4, 64, 64, [1, 2, 65, 128], True, False),
    (1, 1, 128, 8, [300], False, True),
    # head ratio 4: value heads in pairs, 544 units, so the two pairs of a q/k
    # head are placed on one XCD; head ratio 3: one value head per unit
    (8, 32, 128, 64, [1500, 600], False, True),
    (1, 3, 64, 32, [100, 37], True, False),
]


@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "two_pass"])
@pytest.mark.parametrize("case", CHUNKED, ids=lambda c: f"hq{c[0]}_hv{c[1]}_dk{c[2]}_dv{c[3]}_T{sum(c[4])}")
def test_chunked_prefill(case, two_pass):
    h_qk, h_v, d_k, d_v, lens, raw, init = case
    shape = _shape("varlen_prefill_8seq", h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, init_state=init,
                   gate_mode="raw" if raw else "precomputed")
    say(f"[chunked] {case} two_pass={two_pass}")
    inp = synth.generate(shape, seqlens=lens, seed=99)
    g, beta = (None, None) if raw else gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm="chunked", two_pass=two_pass)
    ro, rf = oracle_prefill(inp, g, beta, raw=raw)
    check(out, ro, TOL[shape.io_dtype], "out")
    check(fin, rf, TOL[shape.io_dtype], "final state")


# The bf16 two-pass state pass at d_k = 128 runs 16-column tiles with the
# state rows split over four waves while those tiles take one round of the
# compute units or less (256 on an MI355X), and blocks of 64 or 128 columns
# otherwise.  Both forms against the oracle, on either side of that rule.
TWO_PASS_FORMS = [
    # (h_qk, h_v, d_v, seqlens, initial state updated in place)
    (16, 32, 128, [300], False),         # 32 units x 8 tiles: row-split
    (16, 32, 128, [300, 5], False),      # 64 units x 8 tiles: column blocks
    (2, 4, 40, [2000, 1, 64], True),     # row-split, a ragged last tile, the state in place
]


@pytest.mark.parametrize("case", TWO_PASS_FORMS, ids=["rows_one_round", "columns_two_rounds", "rows_ragged_in_place"])
def test_two_pass_state_forms(case):
    h_qk, h_v, d_v, lens, in_place = case
    shape = _shape("varlen_prefill_8seq", h_qk=h_qk, h_v=h_v, d_v=d_v, init_state=True)
    say(f"[two-pass forms] {case}")
    inp = synth.generate(shape, seqlens=lens, seed=21)
    g, beta = gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True, in_place=in_place)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, TOL[shape.io_dtype], "out")
    check(fin, rf, TOL[shape.io_dtype], "final state")


@pytest.mark.parametrize("two_pass", [False, True], ids=["one_pass", "two_pass"])
def test_chunked_prefill_resets_and_weak_decay(two_pass):
    """Log-decays of -inf (a reset), of 0 (no decay) and tiny beta in one sequence."""
    shape = _shape("varlen_prefill_8seq", init_state=True)
    inp = synth.generate(shape, seqlens=[150, 70])
    g, beta = gates_for(inp)
    g = g.float()
    g[5::37] = float("-inf")
    g[100:140] = 0.0
    g = g.to(torch.bfloat16)
    beta = beta.float()
    beta[60:70] = 1e-3
    beta = beta.to(torch.bfloat16)
    say(f"[chunked] resets / no decay / tiny beta, two_pass={two_pass}")
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=two_pass)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, TOL[torch.bfloat16], "out")
    check(fin, rf, TOL[torch.bfloat16], "final state")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_two_pass_chunk_table_many_long_sequences(dtype):
    """The two-pass workspace's chunk table: a block-wide pass writes the
    entries of sequences longer than 16 chunks, up to 256 of them; the rest
    (here 14 more long ones) and the short ones are written per thread."""
    lens = [1100 if i % 10 else 70 for i in range(300)]  # 270 long, 30 short, interleaved
    d_k = 64 if dtype == torch.bfloat16 else 128
    shape = _shape("varlen_prefill_8seq", h_qk=1, h_v=1, d_k=d_k, d_v=16, io_dtype=dtype, init_state=True)
    inp = synth.generate(shape, seqlens=lens, seed=21)
    g, beta = gates_for(inp)
    say(f"[chunk table] {len(lens)} sequences, {inp.total_tokens} tokens, {dtype}")
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, TOL[dtype], "out")
    check(fin, rf, TOL[dtype], "final state")


def test_two_pass_chunk_table_more_sequences_than_threads():
    """More sequences than the table kernel's 1024 threads: each thread sums
    and writes two or three sequences, empty and 1-token ones among them."""
    gen = torch.Generator().manual_seed(33)
    lens = torch.randint(0, 90, (2300,), generator=gen).tolist()
    lens[5], lens[6], lens[2299] = 0, 1, 2000  # empty, 1 token, one long sequence at the end
    shape = _shape("varlen_prefill_8seq", h_qk=1, h_v=1, d_k=64, d_v=16, io_dtype=torch.bfloat16, init_state=True)
    inp = synth.generate(shape, seqlens=lens, seed=22)
    g, beta = gates_for(inp)
    say(f"[chunk table] {len(lens)} sequences, {inp.total_tokens} tokens")
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, TOL[torch.bfloat16], "out")
    check(fin, rf, TOL[torch.bfloat16], "final state")


def test_chunked_unsupported_is_reported():
    shape = _shape(init_state=False)  # float32 I/O, d_k 16
    inp = synth.generate(shape, seqlens=[64])
    g, beta = gates_for(inp)
    with pytest.raises(gdn.GdnError, match="chunked algorithm needs"):
        gpu_prefill(inp, g, beta, algorithm="chunked")


# ------------------------------------------------------------------ full sizes, sampled
FULL = [
    ("prefill_t4096_fused_gates", [0, 15], "auto"),
    ("prefill_t4096_fused_gates", [5, 9], "two_pass"),
    ("prefill_t4096_fused_gates", [3], "serial"),
    ("varlen_prefill_8seq", [0, 7, 15], "auto"),
    ("varlen_prefill_8seq", [2, 11], "two_pass"),
    ("varlen_prefill_8seq", [4], "serial"),
    ("wide_prefill_t32768_d256", [0, 5], "auto"),
]


@pytest.mark.parametrize("name,heads,algorithm", FULL, ids=[f"{f[0]}-{f[2]}" for f in FULL])
def test_prefill_full_size_sampled(name, heads, algorithm):
    """The full workload as the benchmark runs it; the oracle recomputes the
    listed q/k head groups (all their value heads, every token) on their own."""
    shape = W[name]
    inp = synth.generate(shape)
    say(f"[full] {name} ({algorithm}): {len(inp.seqlens)} seqs, {inp.total_tokens} tokens; "
        f"oracle on head groups {heads}")
    raw = shape.gate_mode == "raw"
    g, beta = (None, None) if raw else gates_for(inp)
    two_pass = algorithm == "two_pass"
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm="auto" if two_pass else algorithm, two_pass=two_pass)
    ref = oracle_prefill(inp, g, beta, raw=raw, heads=heads)
    ratio = shape.h_v // shape.h_qk
    tol = TOL[shape.io_dtype]
    for hq, (ro, rf) in ref.items():
        hv = slice(hq * ratio, (hq + 1) * ratio)
        check(out[:, hv], ro, tol, f"out head group {hq}")
        check(fin[:, hv], rf, tol, f"state head group {hq}")
    assert torch.isfinite(out).all() and torch.isfinite(fin).all()


# ------------------------------------------------------------------ slot-indexed state pool
def _pool(num_slots, shape, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(num_slots, shape.h_v, shape.d_k, shape.d_v, generator=gen) * 0.05


@pytest.mark.parametrize("raw", [False, True], ids=["gates", "rawgates"])
def test_decode_slots(raw):
    """Decode over a pool: sequence i updates pool[slots[i]]; slot -1 and 99 are
    padding (zero state, nothing written); untouched slots stay bit-identical."""
    shape = _shape("decode_b64", num_seqs=6)
    inp, g, beta = _decode_inputs(shape, 123)
    slots = [3, 7, 0, -1, 9, 99]
    pool = _pool(10, shape, 5)
    say(f"[decode-slots] raw={raw} slots={slots}")
    pool_gpu = pool.cuda()
    slots_d = torch.tensor(slots, dtype=torch.int32, device="cuda")
    out = torch.empty(6, shape.h_v, shape.d_v, dtype=shape.io_dtype, device="cuda")
    orc = oracle.default()
    if raw:
        gates = dict(a=to_dev(inp.a), b=to_dev(inp.b), A_log=to_dev(inp.A_log), dt_bias=to_dev(inp.dt_bias))
        gr, br = orc.gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    else:
        gates = dict(g=to_dev(g), beta=to_dev(beta))
        gr, br = g.double().numpy(), beta.double().numpy()
    gdn.gdn_decode_step_slots(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), pool_gpu, slots_d, out,
                              slots_host=slots, **gates)
    torch.cuda.synchronize()
    # oracle: gather (padding -> zeros), step, scatter back
    st = np.stack([pool[s].double().numpy() if 0 <= s < 10 else np.zeros(pool.shape[1:]) for s in slots])
    ro = orc.decode_step(inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy(), gr, br, st)
    ref_pool = pool.double().clone()
    for i, s in enumerate(slots):
        if 0 <= s < 10:
            ref_pool[s] = torch.from_numpy(st[i])
    check(out.double().cpu(), torch.from_numpy(ro), TOL[shape.io_dtype], "out")
    check(pool_gpu.double().cpu(), ref_pool, TOL[shape.io_dtype], "pool")
    for s in (1, 2, 4, 5, 6, 8):
        assert torch.equal(pool_gpu[s].cpu(), pool[s]), f"untouched slot {s} changed"


@pytest.mark.parametrize("algorithm", ["serial", "chunked", "two_pass", "two_pass_f32"])
def test_prefill_slots(algorithm):
    if algorithm == "two_pass_f32":  # the float32 chunked form (d_k 256)
        shape = _shape("wide_prefill_t32768_d256", h_qk=2, h_v=2, d_v=32, init_state=False)
        algorithm = "two_pass"
    else:
        shape = _shape("varlen_prefill_8seq", init_state=False)
    inp = synth.generate(shape, seqlens=[70, 0, 33, 129])
    g, beta = gates_for(inp)
    slots = [5, -1, 2, 0]
    pool = _pool(6, shape, 9)
    say(f"[prefill-slots] {algorithm} slots={slots}")
    pool_gpu = pool.cuda()
    out = torch.full((inp.total_tokens, shape.h_v, shape.d_v), float("nan"), dtype=shape.io_dtype, device="cuda")
    two_pass = algorithm == "two_pass"
    gdn.gdn_prefill_slots(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), pool_gpu,
                          torch.tensor(slots, dtype=torch.int32, device="cuda"), out=out, g=to_dev(g),
                          beta=to_dev(beta), cu_seqlens_host=inp.cu_seqlens.tolist(), slots_host=slots,
                          algorithm="chunked" if two_pass else algorithm,
                          workspace=workspace_for(inp, "chunked") if two_pass else None)
    torch.cuda.synchronize()
    s0 = torch.stack([pool[s] if 0 <= s < 6 else torch.zeros(pool.shape[1:]) for s in slots])
    ref_inp = dataclasses.replace(inp, initial_state=s0)
    ro, rf = oracle_prefill(ref_inp, g, beta)
    ref_pool = pool.double().clone()
    for i, s in enumerate(slots):
        if 0 <= s < 6:
            ref_pool[s] = rf[i]
    check(out.double().cpu(), ro, TOL[shape.io_dtype], "out")
    check(pool_gpu.double().cpu(), ref_pool, TOL[shape.io_dtype], "pool")
    for s in (1, 3, 4):
        assert torch.equal(pool_gpu[s].cpu(), pool[s]), f"untouched slot {s} changed"


def test_slots_identity_equals_plain():
    """slots = 0..N-1 over a pool is the plain call with the pool as in/out state (bitwise)."""
    shape = _shape("varlen_prefill_8seq", init_state=True)
    inp = synth.generate(shape, seqlens=[40, 90, 7])
    g, beta = gates_for(inp)
    say("[slots-identity]")
    out_a, fin_a = gpu_prefill(inp, g, beta, algorithm="serial")
    pool = to_dev(inp.initial_state).clone()
    out_b = torch.empty(inp.total_tokens, shape.h_v, shape.d_v, dtype=shape.io_dtype, device="cuda")
    gdn.gdn_prefill_slots(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens), pool,
                          torch.arange(3, dtype=torch.int32, device="cuda"), out=out_b, g=to_dev(g),
                          beta=to_dev(beta), algorithm="serial")
    torch.cuda.synchronize()
    assert torch.equal(out_b.double().cpu(), out_a)
    assert torch.equal(pool.double().cpu(), fin_a)
