"""GPU parity of the decode step with its conv prologue (gdn_decode_step_conv:
the block's causal depthwise conv [P1] `causal_conv_op` feeding the
recurrence, one token per sequence, in one launch).

Two references on the same seeded inputs:
- the library's unfused pair, gdn_causal_conv_step into a buffer y, then
  gdn_decode_step on y's q, k and v slices.  The fused kernel repeats the
  conv's float32 arithmetic in the same order and narrows each conv output
  once, as the pair stores it, so outputs, recurrent states and carried conv
  inputs agree bit for bit;
- the oracle: its conv (double) over the one-token sequences, rounded to the
  I/O dtype, split into q, k and v, then its decode step (double).  Outputs
  and states to the I/O dtype's tolerance |d| <= tol (1 + |ref|); the carried
  conv inputs are copies of inputs, compared exactly.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, gates_for, say, to_dev

pytestmark = pytest.mark.gpu
W = synth.BY_NAME


def _inputs(h_qk, h_v, d_k, d_v, dt, B, K, bias, seed):
    shape = dataclasses.replace(W["decode_b64"], h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, io_dtype=dt, num_seqs=B)
    rec = synth.generate(shape, seed=seed)
    C = 2 * h_qk * d_k + h_v * d_v
    cshape = dataclasses.replace(synth.CONV_BY_NAME["conv_step_b64"], channels=C, kernel_size=K, io_dtype=dt,
                                 num_seqs=B, bias=bias, init_state=K > 1)
    conv = synth.generate_conv(cshape, seqlens=[1] * B, seed=seed + 1)
    return shape, rec, conv


def _split(y, h_qk, h_v, d_k, d_v):
    B = y.shape[0]
    n = h_qk * d_k
    return (y[:, :n].reshape(B, h_qk, d_k).contiguous(), y[:, n:2 * n].reshape(B, h_qk, d_k).contiguous(),
            y[:, 2 * n:].reshape(B, h_v, d_v).contiguous())


def _gates(rec, raw):
    if raw:
        return (dict(a=to_dev(rec.a), b=to_dev(rec.b), A_log=to_dev(rec.A_log), dt_bias=to_dev(rec.dt_bias)),
                oracle.default().gates(rec.a, rec.b, rec.A_log, rec.dt_bias))
    g, beta = gates_for(rec)
    return dict(g=to_dev(g), beta=to_dev(beta)), (g.double().numpy(), beta.double().numpy())


def _pair(x, w, bias, cs, state, h_qk, d_k, out, gates, **norm):
    """The unfused pair on copies: conv step (state shifted in place), then decode."""
    B, C = x.shape
    y = torch.empty(B, C, dtype=x.dtype, device=x.device)
    cs2 = None if cs is None else cs.clone()
    gdn.gdn_causal_conv_step(x, w, cs2, y=y, bias=bias)
    h_v, d_v = out.shape[1], out.shape[2]
    q, k, v = _split(y, h_qk, h_v, d_k, d_v)
    st2 = state.clone()
    out2 = torch.empty_like(out)
    gdn.gdn_decode_step(q, k, v, st2, out2, **gates, **norm)
    return out2, st2, cs2


GEOMS = [
    # (h_qk, h_v, d_k, d_v, dtype, B, K, bias, raw gates)
    (16, 32, 128, 128, torch.bfloat16, 64, 4, True, False),    # the decode workload, 8192 channels
    (2, 4, 64, 64, torch.float32, 5, 3, True, True),
    (1, 2, 256, 128, torch.float16, 3, 2, False, False),
    (2, 2, 32, 128, torch.bfloat16, 4, 1, True, True),
    (1, 1, 16, 64, torch.bfloat16, 7, 4, True, False),
    (1, 4, 128, 256, torch.float32, 2, 4, True, False),
]


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: f"h{g[0]}x{g[1]}_d{g[2]}x{g[3]}_{str(g[4])[6:]}_B{g[5]}_K{g[6]}")
def test_decode_conv(geom):
    h_qk, h_v, d_k, d_v, dt, B, K, bias, raw = geom
    say(f"[decode-conv] {geom}")
    state = None
    ref_state = None
    cs = None
    ref_cs = None
    orc = oracle.default()
    for step in range(2):
        shape, rec, conv = _inputs(h_qk, h_v, d_k, d_v, dt, B, K, bias, seed=700 + 10 * step)
        if state is None:
            state = to_dev(rec.initial_state).clone()
            ref_state = rec.initial_state.double().numpy().copy()
            cs = to_dev(conv.initial_state)
            ref_cs = conv.initial_state
        x, w, b = to_dev(conv.x), to_dev(conv.weight), to_dev(conv.bias)
        gates, (gr, br) = _gates(rec, raw)
        out = torch.full((B, h_v, d_v), float("nan"), dtype=dt, device="cuda")
        cs_out = None if cs is None else torch.full_like(cs, float("nan"))
        p_out, p_state, p_cs = _pair(x, w, b, cs, state, h_qk, d_k, out, gates)
        gdn.gdn_decode_step_conv(x, w, cs, cs_out, state, out, h_qk=h_qk, d_k=d_k, conv_bias=b, **gates)
        torch.cuda.synchronize()
        assert torch.equal(out, p_out), f"step {step}: out differs from the unfused pair"
        assert torch.equal(state, p_state), f"step {step}: state differs from the unfused pair"
        if cs is not None:
            assert torch.equal(cs_out, p_cs), f"step {step}: carried conv inputs differ from the unfused pair"
        # the oracle: conv (double) -> I/O dtype -> split -> decode step (double)
        ry, rcs = orc.causal_conv(conv.x, conv.weight, np.arange(B + 1), conv.bias, ref_cs, dilation=1, silu=True)
        q, k, v = _split(torch.from_numpy(ry).to(dt), h_qk, h_v, d_k, d_v)
        ro = orc.decode_step(q.double().numpy(), k.double().numpy(), v.double().numpy(), gr, br, ref_state)
        check(out.double().cpu(), torch.from_numpy(ro), TOL[dt], f"out step {step}")
        check(state.double().cpu(), torch.from_numpy(ref_state), TOL[dt], f"state step {step}")
        if cs is not None:
            assert torch.equal(cs_out.double().cpu(), torch.from_numpy(rcs)), f"step {step}: carried conv inputs"
            cs, ref_cs = cs_out, torch.from_numpy(rcs).to(dt)


def test_decode_conv_with_output_norm():
    """The decode workload with the conv prologue and the fused output norm,
    against the unfused pair with the same norm (bit for bit)."""
    h_qk, h_v, d_k, d_v, dt, B = 16, 32, 128, 128, torch.bfloat16, 64
    say("[decode-conv] with the output norm")
    _, rec, conv = _inputs(h_qk, h_v, d_k, d_v, dt, B, 4, True, seed=760)
    gate, scale = synth.output_norm_inputs(B, h_v, d_v, seed=761, io_dtype=dt)
    norm = dict(norm_gate=to_dev(gate), norm_scale=to_dev(scale))
    gates, _ = _gates(rec, False)
    x, w, b, cs = to_dev(conv.x), to_dev(conv.weight), to_dev(conv.bias), to_dev(conv.initial_state)
    state = to_dev(rec.initial_state).clone()
    out = torch.empty(B, h_v, d_v, dtype=dt, device="cuda")
    p_out, p_state, p_cs = _pair(x, w, b, cs, state, h_qk, d_k, out, gates, **norm)
    cs_out = torch.empty_like(cs)
    gdn.gdn_decode_step_conv(x, w, cs, cs_out, state, out, h_qk=h_qk, d_k=d_k, conv_bias=b, **gates, **norm)
    torch.cuda.synchronize()
    assert torch.equal(out, p_out) and torch.equal(state, p_state) and torch.equal(cs_out, p_cs)


def test_decode_conv_unsupported_shapes_refused():
    """Shapes outside the fused kernel's tiles are refused before any launch,
    and leave every buffer untouched."""
    B = 2
    for (h_qk, h_v, d_k, d_v, K, dil) in [(1, 1, 100, 128, 4, 1), (1, 1, 128, 96, 4, 1), (1, 1, 64, 64, 5, 1)]:
        C = 2 * h_qk * d_k + h_v * d_v
        x = torch.zeros(B, C, dtype=torch.bfloat16, device="cuda")
        w = torch.zeros(C, K, dtype=torch.bfloat16, device="cuda")
        cs = torch.zeros(B, K - 1, C, dtype=torch.bfloat16, device="cuda")
        cs_out = torch.full_like(cs, 7.0)
        st = torch.ones(B, h_v, d_k, d_v, device="cuda")
        out = torch.full((B, h_v, d_v), 3.0, dtype=torch.bfloat16, device="cuda")
        g = torch.zeros(B, h_v, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_decode_step_conv(x, w, cs, cs_out, st, out, h_qk=h_qk, d_k=d_k, g=g, beta=g)
        assert e.value.status == gdn.GDN_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert (cs_out == 7.0).all() and (out == 3.0).all() and (st == 1.0).all()
