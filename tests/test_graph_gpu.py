"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: the calls enqueue kernels only (no synchronisation, no memset, no
allocation), so a captured call must give exactly the eager result on every
replay.  Each graph is replayed several times, with eager work and
synchronisations between the replays, and every replay is compared bit for bit
with the eager run of the same call on the same inputs (the kernels have no
atomics, so they are deterministic).
"""
import dataclasses

import pytest
import torch

from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import gates_for, say, to_dev, workspace_for

pytestmark = pytest.mark.gpu

W = synth.BY_NAME
REPLAYS = 3


def _replay_and_compare(run, outputs, reset, what):
    """run(): enqueue the call; outputs(): tensors it writes; reset(): restore its inputs."""
    reset()
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs()]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch asks
        reset()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    for i in range(REPLAYS):
        for t in outputs():
            t.fill_(float("nan"))
        reset()  # after the fill: a state updated in place is input and output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, outputs()):
            assert torch.equal(e, t), f"{what}: replay {i} differs from the eager call"
        _ = torch.ones(1024, device="cuda").sum().item()  # eager work between the replays
    say(f"[graph] {what}: {REPLAYS} replays equal the eager call")


def test_graph_decode_step():
    shape = dataclasses.replace(W["decode_b64"], h_qk=4, h_v=8)
    inp = synth.generate(shape, num_seqs=16, seed=3)
    g, beta = gates_for(inp)
    q, k, v, gg, bb = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(g), to_dev(beta)
    s0 = to_dev(inp.initial_state)
    state = s0.clone()
    out = torch.empty(16, shape.h_v, shape.d_v, dtype=shape.io_dtype, device="cuda")

    def run():
        gdn.gdn_decode_step(q, k, v, state, out=out, g=gg, beta=bb)

    _replay_and_compare(run, lambda: [out, state], lambda: state.copy_(s0), "decode step")


@pytest.mark.parametrize("name,over", [
    ("varlen_prefill_8seq", dict(h_qk=4, h_v=8, init_state=True)),
    ("wide_prefill_t32768_d256", dict(h_qk=2, h_v=2, d_v=64, init_state=True)),
], ids=["bf16_two_pass", "f32_two_pass"])
def test_graph_prefill_two_pass(name, over):
    shape = dataclasses.replace(W[name], **over)
    inp = synth.generate(shape, seqlens=[150, 0, 333, 64], seed=4)
    g, beta = gates_for(inp)
    q, k, v, gg, bb = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(g), to_dev(beta)
    cu = to_dev(inp.cu_seqlens)
    s0 = to_dev(inp.initial_state)
    ws = workspace_for(inp, "chunked")
    assert ws is not None
    n, T = len(inp.seqlens), inp.total_tokens
    out = torch.empty(T, shape.h_v, shape.d_v, dtype=shape.io_dtype, device="cuda")
    fin = torch.empty(n, shape.h_v, shape.d_k, shape.d_v, dtype=torch.float32, device="cuda")

    def run():
        gdn.gdn_prefill(q, k, v, cu, out=out, final_state=fin, initial_state=s0, g=gg, beta=bb,
                        cu_seqlens_host=inp.cu_seqlens.tolist(), algorithm="chunked", workspace=ws)

    _replay_and_compare(run, lambda: [out, fin], lambda: None, f"{name} two-pass prefill")


def test_graph_static_workspace_and_output_norm():
    """gdn_prefill_static_workspace (the entry point for callers that cannot
    allocate, such as code under graph capture) with the output norm as its own
    pass (one sequence), and gdn_prefill with the norm fused into the state pass
    (16 x 32 units, a caller workspace: beyond the static array), captured and
    replayed."""
    for lens, static in (([300], True), ([70] * 16, False)):
        shape = W["varlen_prefill_8seq"]
        inp = synth.generate(shape, seqlens=lens, seed=5)
        g, beta = gates_for(inp)
        T = inp.total_tokens
        gate, scale = synth.output_norm_inputs(T, shape.h_v, shape.d_v, seed=6, io_dtype=shape.io_dtype)
        args = [to_dev(t) for t in (inp.q, inp.k, inp.v, inp.cu_seqlens, g, beta, gate, scale)]
        s0 = to_dev(inp.initial_state)
        fin = torch.empty_like(s0)
        out = torch.empty(T, shape.h_v, shape.d_v, dtype=shape.io_dtype, device="cuda")
        ws = None if static else workspace_for(inp)
        plan = gdn.prefill_query_plan(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, len(lens), T,
                                      workspace_bytes=1 << 40, norm=True)
        assert plan["norm"] == ("separate pass" if static else "fused"), plan

        def run():
            q, k, v, cu, gg, bb, ng, ns = args
            kw = dict(out=out, final_state=fin, initial_state=s0, g=gg, beta=bb, norm_gate=ng, norm_scale=ns,
                      cu_seqlens_host=inp.cu_seqlens.tolist())
            if static:
                gdn.gdn_prefill_static_workspace(q, k, v, cu, **kw)
            else:
                gdn.gdn_prefill(q, k, v, cu, workspace=ws, **kw)
        _replay_and_compare(run, lambda: [out, fin], lambda: None,
                            f"{'static workspace' if static else 'caller workspace'} + output norm ({plan['norm']})")
