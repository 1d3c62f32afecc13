"""GPU parity of the float32 two-pass chunked prefill (d_k 128 or 256,
products on split bfloat16 operands) against the oracle, element by element.

Reduced sizes cover ragged chunk tails (lengths that are not multiples of the
64-token chunk), empty and one-token sequences, several 16-column tiles,
grouped q/k heads, initial states, raw and precomputed gates, state resets
(g = -inf), stretches without decay and tiny beta.  The full-size case runs
the wide-head long prefill exactly as the benchmark launches it and compares
sampled head groups that the oracle computes alone.

Tolerance: |gpu - ref| <= 1e-4 (1 + |ref|) elementwise (float32 I/O).
"""
import dataclasses

import pytest
import torch

from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, gates_for, gpu_prefill, oracle_prefill, say

pytestmark = pytest.mark.gpu

W = synth.BY_NAME
F32 = TOL[torch.float32]

CASES = [
    # (h_qk, h_v, d_k, d_v, seqlens, raw gates, initial state)
    (8, 8, 256, 256, [200], False, False),
    (2, 4, 256, 64, [37, 0, 129, 64, 1, 250, 3], True, True),
    (1, 2, 128, 128, [130, 65], False, True),
    (4, 4, 128, 16, [1, 2, 65, 128], True, False),
    (1, 1, 256, 256, [300], False, True),
    (2, 2, 256, 48, [64, 63, 1], True, True),
]


def _shape(**kw):
    return dataclasses.replace(W["wide_prefill_t32768_d256"], **kw)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"hq{c[0]}_hv{c[1]}_dk{c[2]}_dv{c[3]}_T{sum(c[4])}")
def test_wide_chunked_prefill(case):
    h_qk, h_v, d_k, d_v, lens, raw, init = case
    shape = _shape(h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, init_state=init, gate_mode="raw" if raw else "precomputed")
    say(f"[wide-chunked] {case}")
    inp = synth.generate(shape, seqlens=lens, seed=5)
    g, beta = (None, None) if raw else gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, raw=raw, algorithm="chunked", two_pass=True)
    ro, rf = oracle_prefill(inp, g, beta, raw=raw)
    check(out, ro, F32, "out")
    check(fin, rf, F32, "final state")


def test_wide_chunked_resets_and_weak_decay():
    """Log-decays of -inf (a reset), of 0 (no decay over whole chunks, so the
    state is carried undamped) and tiny beta in one sequence."""
    shape = _shape(h_qk=2, h_v=2, d_k=256, d_v=64, init_state=True)
    inp = synth.generate(shape, seqlens=[300, 70])
    g, beta = gates_for(inp)
    g[5::37] = float("-inf")
    g[100:260] = 0.0
    beta[60:70] = 1e-3
    say("[wide-chunked] resets / no decay / tiny beta")
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, F32, "out")
    check(fin, rf, F32, "final state")


def test_wide_chunked_delta_rule_and_state_only():
    """The delta rule (no decay) through the same kernels, and a call that asks
    for the final state alone."""
    shape = _shape(h_qk=1, h_v=2, d_k=128, d_v=32, init_state=True)
    inp = synth.generate(shape, seqlens=[90, 40], seed=3)
    g, beta = gates_for(inp)
    zero = torch.zeros_like(g)
    say("[wide-chunked] delta rule")
    out, fin = gpu_prefill(inp, zero, beta, algorithm="chunked", two_pass=True)
    ro, rf = oracle_prefill(inp, zero, beta)
    check(out, ro, F32, "out (g = 0)")
    check(fin, rf, F32, "final state (g = 0)")
    _, fin2 = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True, want_out=False)
    _, rf2 = oracle_prefill(inp, g, beta)
    check(fin2, rf2, F32, "final state only")


def test_wide_chunked_auto_with_workspace():
    """GDN_ALGO_AUTO takes the float32 two-pass form at d_k = 256 when handed a workspace."""
    shape = _shape(h_qk=2, h_v=4, d_k=256, d_v=32, init_state=True)
    inp = synth.generate(shape, seqlens=[129, 70], seed=8)
    g, beta = gates_for(inp)
    nbytes = gdn.prefill_workspace_size(2, 4, 256, 32, torch.float32, 2, inp.total_tokens)
    assert nbytes > 0
    say("[wide-chunked] auto with a workspace")
    out, fin = gpu_prefill(inp, g, beta, algorithm="auto", two_pass=True)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, F32, "out")
    check(fin, rf, F32, "final state")


@pytest.mark.parametrize("in_place", [False, True], ids=["out_of_place", "in_place"])
def test_wide_chunked_long_varlen(in_place):
    """Long packed sequences of 313, 3, 0 and 141 chunks, the initial state
    updated in place or written to a separate final state."""
    lens = [20000, 130, 0, 9000]
    shape = _shape(h_qk=1, h_v=2, d_k=128, d_v=16, init_state=True)
    inp = synth.generate(shape, seqlens=lens, seed=13)
    g, beta = gates_for(inp)
    say(f"[wide-chunked long varlen] lens={lens} in_place={in_place}")
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True, in_place=in_place)
    ro, rf = oracle_prefill(inp, g, beta)
    check(out, ro, F32, "out")
    check(fin, rf, F32, "final state")


def test_wide_chunked_needs_workspace():
    shape = _shape(h_qk=1, h_v=1, d_k=256, d_v=16, init_state=False)
    inp = synth.generate(shape, seqlens=[64])
    g, beta = gates_for(inp)
    with pytest.raises(gdn.GdnError, match="workspace"):
        gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=False)


def test_wide_chunked_full_size_sampled():
    """The wide-head long prefill (T = 32768, 8 heads, d = 256, float32) as the
    benchmark launches it; the oracle recomputes head groups 2 and 7."""
    shape = W["wide_prefill_t32768_d256"]
    inp = synth.generate(shape)
    heads = [2, 7]
    say(f"[wide-chunked full] {inp.total_tokens} tokens; oracle on heads {heads}")
    g, beta = gates_for(inp)
    out, fin = gpu_prefill(inp, g, beta, algorithm="chunked", two_pass=True)
    ref = oracle_prefill(inp, g, beta, heads=heads)
    for hq, (ro, rf) in ref.items():
        check(out[:, hq:hq + 1], ro, F32, f"out head {hq}")
        check(fin[:, hq:hq + 1], rf, F32, f"state head {hq}")
    assert torch.isfinite(out).all() and torch.isfinite(fin).all()
