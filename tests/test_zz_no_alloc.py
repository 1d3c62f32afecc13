"""gdn_prefill_static_workspace, the entry point for callers that cannot
allocate: its two-pass workspace is the library's own device array.  Held to
gdn_prefill with a caller-allocated workspace (same kernels: bitwise equal) and
to the oracle, on two calls in a row on one device, the second smaller, so
the second finds the first's records in the array."""
import ctypes
import dataclasses

import pytest
import torch

from gated_delta_rule_serial_amd import gdn, synth
from gpu_harness import TOL, check, gates_for, oracle_prefill, say, to_dev, workspace_for

CASES = [
    # (workload, overrides, first call's sequence lengths, second (smaller) call's)
    ("varlen_prefill_8seq", dict(), [700, 300], [200, 0, 99]),
    ("wide_prefill_t32768_d256", dict(h_qk=2, h_v=2, init_state=True), [800], [150, 64]),
]


def _run_both(inp, g, beta):
    sh = inp.shape
    T, n = inp.total_tokens, len(inp.seqlens)
    q, k, v, cu = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.cu_seqlens)
    s0 = to_dev(inp.initial_state)
    res = []
    for static in (True, False):
        out = torch.full((T, sh.h_v, sh.d_v), float("nan"), dtype=sh.io_dtype, device="cuda")
        fin = torch.full((n, sh.h_v, sh.d_k, sh.d_v), float("nan"), dtype=torch.float32, device="cuda")
        kw = dict(out=out, final_state=fin, initial_state=s0, g=to_dev(g), beta=to_dev(beta),
                  cu_seqlens_host=inp.cu_seqlens.tolist())
        if static:
            gdn.gdn_prefill_static_workspace(q, k, v, cu, **kw)
        else:
            gdn.gdn_prefill(q, k, v, cu, workspace=workspace_for(inp), **kw)
        torch.cuda.synchronize()
        res.append((out.double().cpu(), fin.double().cpu()))
    return res


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_static_workspace_matches_caller_workspace(case):
    name, over, first, second = case
    shape = dataclasses.replace(synth.BY_NAME[name], **over)
    for lens in (first, second):
        inp = synth.generate(shape, seqlens=lens, seed=811)
        g, beta = gates_for(inp)
        need = gdn.prefill_workspace_size(shape.h_qk, shape.h_v, shape.d_k, shape.d_v, shape.io_dtype, len(lens),
                                          inp.total_tokens)
        assert 0 < need <= gdn.STATIC_WORKSPACE_BYTES
        say(f"[static workspace] {name} {lens}: {need} bytes")
        (so, sf), (wo, wf) = _run_both(inp, g, beta)
        assert torch.equal(so, wo) and torch.equal(sf, wf), "static and caller workspaces differ"
        ro, rf = oracle_prefill(inp, g, beta)
        check(so, ro, TOL[shape.io_dtype], "out")
        check(sf, rf, TOL[shape.io_dtype], "final state")


def test_static_workspace_refuses_oversized_problem():
    """Host-side: a problem needing more workspace than the array holds is
    refused before anything is enqueued (no device is touched)."""
    lib = gdn.load()
    prob = gdn.make_problem(16, 32, 128, 128, torch.bfloat16, g=torch.empty(0), beta=torch.empty(0))
    prob.g = ctypes.c_void_p(0x100000)
    prob.beta = ctypes.c_void_p(0x200000)
    T = 8192
    vp = ctypes.c_void_p
    st = lib.gdn_prefill_static_workspace(ctypes.byref(prob), 1, vp(0x300000), None, T, vp(0x400000), vp(0x500000),
                                          vp(0x600000), None, vp(0x10000000), vp(0x20000000), None)
    assert st == gdn.GDN_ERR_UNSUPPORTED and "bytes this entry point holds" in gdn.last_error()
    prob.workspace = vp(0x700000)
    prob.workspace_bytes = 1 << 30
    st = lib.gdn_prefill_static_workspace(ctypes.byref(prob), 1, vp(0x300000), None, 64, vp(0x400000), vp(0x500000),
                                          vp(0x600000), None, vp(0x10000000), vp(0x20000000), None)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "takes no workspace" in gdn.last_error()
