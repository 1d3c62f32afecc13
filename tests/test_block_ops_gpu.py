"""GPU parity of the block's neighbouring operations -- the causal depthwise
conv with carried state and the gated RMSNorm -- through the C ABI, against
the oracle, element by element on seeded inputs.

Outputs: |gpu - ref| <= tol (1 + |ref|) with the recurrence's per-dtype
tolerances (each output is one float32 sum of at most K products, or one
normalisation, narrowed once).  Conv states are copies of inputs, so they are
compared bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, say, to_dev

pytestmark = pytest.mark.gpu

CONV = synth.CONV_BY_NAME


def _conv_shape(base="conv_varlen_8seq", **kw):
    return dataclasses.replace(CONV[base], **kw)


def _oracle_conv(inp, *, silu=True, initial_state="given"):
    s0 = inp.initial_state if initial_state == "given" else None
    return oracle.default().causal_conv(inp.x, inp.weight, inp.cu_seqlens.numpy(), inp.bias, s0,
                                        dilation=inp.shape.dilation, silu=silu)


CONV_CASES = [
    # (channels, K, dilation, dtype, seqlens, initial state, bias, activation)
    (8192, 4, 1, torch.bfloat16, [37, 0, 129, 64, 1, 250, 3], True, True, "silu"),
    (64, 4, 1, torch.float32, [5, 9], False, False, "silu"),
    (24, 3, 1, torch.float16, [17, 2, 40], True, True, "none"),
    (10, 4, 1, torch.bfloat16, [13, 1], True, True, "silu"),
    (32, 4, 2, torch.bfloat16, [20, 3, 0], True, True, "silu"),
    (16, 1, 1, torch.float32, [7], True, True, "none"),
    (48, 2, 1, torch.bfloat16, [100, 8, 1], True, False, "silu"),
    (40, 6, 1, torch.float32, [30, 2], True, True, "silu"),
    (4096, 4, 1, torch.float32, [1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1], True, True, "silu"),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: f"C{c[0]}_K{c[1]}_d{c[2]}_{str(c[3])[6:]}_T{sum(c[4])}")
def test_causal_conv(case):
    C, K, dil, dt, lens, init, bias, act = case
    shape = _conv_shape(channels=C, kernel_size=K, dilation=dil, io_dtype=dt, init_state=init, bias=bias)
    say(f"[conv] {case}")
    inp = synth.generate_conv(shape, seqlens=lens, seed=301)
    y, fin = gdn.causal_conv(to_dev(inp.x), to_dev(inp.weight), to_dev(inp.cu_seqlens), bias=to_dev(inp.bias),
                             initial_state=to_dev(inp.initial_state), dilation=dil, activation=act,
                             cu_seqlens_host=inp.cu_seqlens.tolist())
    torch.cuda.synchronize()
    ry, rf = _oracle_conv(inp, silu=act == "silu")
    check(y.double().cpu(), torch.from_numpy(ry), TOL[dt], "y")
    # the state holds input values: exact
    assert torch.equal(fin.double().cpu(), torch.from_numpy(rf)), "final state differs"


def test_causal_conv_state_in_place():
    """final_state == initial_state: every state row is read before it is replaced."""
    shape = _conv_shape(channels=256, io_dtype=torch.bfloat16)
    inp = synth.generate_conv(shape, seqlens=[2, 0, 1, 9, 3], seed=302)
    say("[conv] in place")
    st = to_dev(inp.initial_state).clone()
    y = torch.empty_like(to_dev(inp.x))
    gdn.gdn_causal_conv(to_dev(inp.x), to_dev(inp.weight), to_dev(inp.cu_seqlens), y=y, bias=to_dev(inp.bias),
                        initial_state=st, final_state=st)
    torch.cuda.synchronize()
    ry, rf = _oracle_conv(inp)
    check(y.double().cpu(), torch.from_numpy(ry), TOL[torch.bfloat16], "y")
    assert torch.equal(st.double().cpu(), torch.from_numpy(rf))


@pytest.mark.parametrize("dil,K,dt", [(1, 4, torch.bfloat16), (2, 3, torch.float32), (1, 1, torch.float16)])
def test_causal_conv_step_chain(dil, K, dt):
    """Three chained one-token steps at the decode batch (B = 64, C = 8192)
    against the oracle's packed form with one token per sequence."""
    shape = _conv_shape("conv_step_b64", kernel_size=K, dilation=dil, io_dtype=dt)
    inp0 = synth.generate_conv(shape)
    say(f"[conv-step] K={K} dil={dil} {dt}")
    st = to_dev(inp0.initial_state).clone()
    ref_state = inp0.initial_state
    for step in range(3):
        inp = synth.generate_conv(shape, seed=4000 + step)
        y = torch.empty_like(to_dev(inp.x))
        gdn.gdn_causal_conv_step(to_dev(inp.x), to_dev(inp0.weight), st, y=y, bias=to_dev(inp0.bias),
                                 dilation=dil)
        torch.cuda.synchronize()
        ry, rf = oracle.default().causal_conv(inp.x, inp0.weight, np.arange(65), inp0.bias, ref_state,
                                              dilation=dil, silu=True)
        check(y.double().cpu(), torch.from_numpy(ry), TOL[dt], f"y step {step}")
        assert torch.equal(st.double().cpu(), torch.from_numpy(rf)), f"state step {step}"
        ref_state = torch.from_numpy(rf).to(dt)


def test_causal_conv_steps_equal_prefill():
    shape = _conv_shape(channels=512, io_dtype=torch.bfloat16)
    inp = synth.generate_conv(shape, seqlens=[7], seed=303)
    say("[conv] steps = prefill")
    y_p, f_p = gdn.causal_conv(to_dev(inp.x), to_dev(inp.weight), to_dev(inp.cu_seqlens), bias=to_dev(inp.bias),
                               initial_state=to_dev(inp.initial_state))
    st = to_dev(inp.initial_state).clone()
    ys = []
    for t in range(7):
        y = torch.empty(1, 512, dtype=torch.bfloat16, device="cuda")
        gdn.gdn_causal_conv_step(to_dev(inp.x[t:t + 1]), to_dev(inp.weight), st, y=y, bias=to_dev(inp.bias))
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys), y_p) and torch.equal(st, f_p)


def test_causal_conv_full_size():
    """The packed conv workload at its full size (33,173 tokens x 8192 channels),
    compared on every token of 64 sampled channels, and every state."""
    shape = CONV["conv_varlen_8seq"]
    inp = synth.generate_conv(shape)
    say(f"[conv] full size T={sum(inp.seqlens)}")
    y, fin = gdn.causal_conv(to_dev(inp.x), to_dev(inp.weight), to_dev(inp.cu_seqlens), bias=to_dev(inp.bias),
                             initial_state=to_dev(inp.initial_state), cu_seqlens_host=inp.cu_seqlens.tolist())
    torch.cuda.synchronize()
    cols = torch.tensor(sorted(np.random.default_rng(5).choice(shape.channels, 64, replace=False).tolist()))
    ry, rf = oracle.default().causal_conv(inp.x[:, cols], inp.weight[cols], inp.cu_seqlens.numpy(), inp.bias[cols],
                                          inp.initial_state[:, :, cols], silu=True)
    check(y[:, cols.cuda()].double().cpu(), torch.from_numpy(ry), TOL[shape.io_dtype], "y (sampled channels)")
    for n in range(len(inp.seqlens)):
        t1 = int(inp.cu_seqlens[n + 1])
        assert torch.equal(fin[n].cpu(), inp.x[t1 - 3:t1]), f"state {n}"


# ------------------------------------------------------------------ gated RMSNorm
NORM_CASES = [
    # (rows, width, group, dtype, activation, eps)
    (1000, 4096, 128, torch.bfloat16, "silu", 1e-5),
    (37, 256, 256, torch.float32, "sigmoid", 1e-6),
    (5, 96, 96, torch.float16, "silu", 1e-5),
    (3, 300, 100, torch.bfloat16, "silu", 1e-5),
    (7, 4096, 4096, torch.bfloat16, "sigmoid", 1e-5),
    (9, 2048, 2048, torch.float32, "silu", 0.0),
    (129, 64, 16, torch.float32, "silu", 1e-5),
    (2, 8, 1, torch.float32, "sigmoid", 1e-5),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: f"r{c[0]}_w{c[1]}_g{c[2]}_{str(c[3])[6:]}_{c[4]}")
def test_gated_rmsnorm(case):
    rows, width, group, dt, act, eps = case
    shape = synth.NormShape("case", dt, rows, width, group)
    inp = synth.generate_norm(shape, seed=501)
    say(f"[norm] {case}")
    y = gdn.gated_rmsnorm(to_dev(inp.x), to_dev(inp.gate), to_dev(inp.scale), eps=eps, activation=act)
    torch.cuda.synchronize()
    ref = oracle.default().gated_rmsnorm(inp.x, inp.gate, inp.scale, eps=eps, activation=act)
    check(y.double().cpu(), torch.from_numpy(ref), TOL[dt], "y")


def test_gated_rmsnorm_in_place_and_full_size():
    """y = x in place, at the full norm workload (33,173 rows x 32 heads of 128),
    compared on 512 sampled rows."""
    shape = synth.NORM_BY_NAME["gated_rmsnorm_t33173"]
    inp = synth.generate_norm(shape)
    say("[norm] full size in place")
    x = to_dev(inp.x).clone()
    gdn.gdn_gated_rmsnorm(x, to_dev(inp.gate), to_dev(inp.scale), y=x)
    torch.cuda.synchronize()
    rows = torch.tensor(sorted(np.random.default_rng(6).choice(shape.rows, 512, replace=False).tolist()))
    ref = oracle.default().gated_rmsnorm(inp.x[rows], inp.gate[rows], inp.scale)
    check(x[rows.cuda()].double().cpu(), torch.from_numpy(ref), TOL[shape.io_dtype], "y (sampled rows)")


# ------------------------------------------------------------------ the conv over a slot-indexed pool
CONV_SLOT_CASES = [
    # (channels, K, dilation, dtype, seqlens, slots, pool rows)
    (8192, 4, 1, torch.bfloat16, [37, 0, 129, 64, 1, 250, 3], [9, 2, -1, 0, 5, 11, 7], 11),  # 11: padding
    (64, 4, 1, torch.float32, [5, 9, 16], [1, 0, 2], 3),
    (32, 3, 2, torch.bfloat16, [20, 3, 0, 8], [3, -5, 1, 6], 7),                              # generic path
    (40, 6, 1, torch.float16, [30, 2], [0, 4], 5),
]


@pytest.mark.parametrize("case", CONV_SLOT_CASES, ids=lambda c: f"C{c[0]}_K{c[1]}_d{c[2]}_{str(c[3])[6:]}")
def test_causal_conv_slots(case):
    """gdn_causal_conv_slots against the oracle's pool form: outputs within
    tolerance, the pool (copies of inputs) bit for bit, rows no sequence
    names untouched."""
    C, K, dil, dt, lens, slots, rows = case
    shape = _conv_shape(channels=C, kernel_size=K, dilation=dil, io_dtype=dt)
    say(f"[conv-slots] {case}")
    inp = synth.generate_conv(shape, seqlens=lens, seed=311)
    carry = (K - 1) * dil
    pool0 = synth.generate_conv(dataclasses.replace(shape, num_seqs=rows), seqlens=[0] * rows, seed=312).initial_state
    pool = to_dev(pool0).clone()
    sl = torch.tensor(slots, dtype=torch.int32)
    y = torch.empty_like(to_dev(inp.x))
    gdn.gdn_causal_conv_slots(to_dev(inp.x), to_dev(inp.weight), to_dev(inp.cu_seqlens), pool, to_dev(sl), y=y,
                              bias=to_dev(inp.bias), dilation=dil, cu_seqlens_host=inp.cu_seqlens.tolist(),
                              slots_host=slots)
    torch.cuda.synchronize()
    assert pool.shape == (rows, carry, C)
    ry, rpool = oracle.default().causal_conv_slots(inp.x, inp.weight, inp.cu_seqlens.numpy(), pool0, slots,
                                                   inp.bias, dilation=dil, silu=True)
    check(y.double().cpu(), torch.from_numpy(ry), TOL[dt], "y")
    assert torch.equal(pool.double().cpu(), torch.from_numpy(rpool)), "pool differs"


def test_causal_conv_step_slots_chain():
    """Three one-token steps of 16 sequences over a pool of 24 rows (two
    padding sequences), against the oracle's pool form step by step."""
    shape = _conv_shape("conv_step_b64", channels=512, num_seqs=16)
    slots = [23, 0, 5, -1, 7, 8, 30, 1, 2, 3, 4, 9, 10, 11, 12, 13]
    pool0 = synth.generate_conv(dataclasses.replace(shape, num_seqs=24), seqlens=[0] * 24, seed=321).initial_state
    pool = to_dev(pool0).clone()
    ref_pool = pool0
    w = synth.generate_conv(shape, seed=322)
    say("[conv-step-slots] 3 steps")
    for step in range(3):
        inp = synth.generate_conv(shape, seed=4100 + step)
        y = torch.empty_like(to_dev(inp.x))
        gdn.gdn_causal_conv_step_slots(to_dev(inp.x), to_dev(w.weight), pool, to_dev(torch.tensor(slots, dtype=torch.int32)),
                                       y=y, bias=to_dev(w.bias), slots_host=slots)
        torch.cuda.synchronize()
        ry, rp = oracle.default().causal_conv_slots(inp.x, w.weight, np.arange(17), ref_pool, slots, w.bias,
                                                    silu=True)
        check(y.double().cpu(), torch.from_numpy(ry), TOL[torch.bfloat16], f"y step {step}")
        assert torch.equal(pool.double().cpu(), torch.from_numpy(rp)), f"pool step {step}"
        ref_pool = torch.from_numpy(rp).to(torch.bfloat16)
