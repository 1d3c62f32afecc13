"""Shared plumbing of the GPU parity tests: run the same seeded inputs through
the HIP library (via its C ABI binding) and through the oracle, and compare
element by element.

Gates for workloads with precomputed gates come from the oracle's gate
prologue (double) rounded once to the I/O dtype; both sides then read the same
rounded values.  Workloads with raw gates hand (a, b, A_log, dt_bias) to the
library, and the oracle's gate prologue of the same values to the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gated_delta_rule_serial_amd import gdn, synth

# Tolerances: |gpu - ref| <= tol (1 + |ref|) elementwise.  float32 and
# bfloat16 are the stated bars; float16 takes twice its unit roundoff
# (2^-11): the output is narrowed once, the inputs are the same float16
# values on both sides, and float32 accumulation adds ~1e-6.
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2, torch.float16: 1e-3}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def gates_for(inp: synth.Inputs):
    """(g, beta) in the I/O dtype for precomputed-gate workloads, from the oracle."""
    g, beta = oracle.default().gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    dt = inp.shape.io_dtype
    return torch.from_numpy(g).to(dt), torch.from_numpy(beta).to(dt)


def to_dev(t, dev="cuda"):
    return None if t is None else t.contiguous().to(dev)


def workspace_for(inp: synth.Inputs, algorithm="auto", **variant):
    """The two-pass chunked form's workspace for these inputs (None when it does not apply)."""
    sh = inp.shape
    nbytes = gdn.prefill_workspace_size(sh.h_qk, sh.h_v, sh.d_k, sh.d_v, sh.io_dtype, len(inp.seqlens),
                                        inp.total_tokens, algorithm=algorithm, **variant)
    return torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda") if nbytes else None


def gpu_prefill(inp: synth.Inputs, g=None, beta=None, *, raw=False, scale=0.0, want_out=True,
                want_state=True, in_place=False, use_host_cu=True, algorithm="auto", two_pass=False):
    """Run gdn_prefill on cuda:0; returns (out, final) as CPU float64 tensors (or None).
    two_pass: hand the call a workspace, so the chunked form runs in two passes."""
    dev = "cuda"
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    cu = to_dev(inp.cu_seqlens)
    n = len(inp.seqlens)
    T = inp.total_tokens
    h_v, d_k, d_v = inp.shape.h_v, inp.shape.d_k, inp.shape.d_v
    s0 = to_dev(inp.initial_state)
    out = torch.full((T, h_v, d_v), float("nan"), dtype=inp.shape.io_dtype, device=dev) if want_out else None
    if in_place:
        assert s0 is not None
        fin = s0
    else:
        fin = torch.full((n, h_v, d_k, d_v), float("nan"), dtype=torch.float32, device=dev) if want_state else None
    gates = (dict(a=to_dev(inp.a), b=to_dev(inp.b), A_log=to_dev(inp.A_log), dt_bias=to_dev(inp.dt_bias))
             if raw else dict(g=to_dev(g), beta=to_dev(beta)))
    ws = workspace_for(inp, algorithm) if two_pass else None
    if ws is not None:
        gates["workspace"] = ws
    gdn.gdn_prefill(q, k, v, cu, out=out, final_state=fin, initial_state=s0, scale=scale,
                    cu_seqlens_host=inp.cu_seqlens.tolist() if use_host_cu else None, algorithm=algorithm,
                    **gates)
    torch.cuda.synchronize()
    return (None if out is None else out.double().cpu(), None if fin is None else fin.double().cpu())


def oracle_prefill(inp: synth.Inputs, g=None, beta=None, *, raw=False, scale=0.0, heads=None):
    """Oracle on all heads, or on the q/k head groups listed in ``heads``
    (each group = one q/k head and its consecutive value heads)."""
    orc = oracle.default()
    if raw:
        g, beta = orc.gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    else:
        g, beta = g.double().numpy(), beta.double().numpy()
    q, k, v = inp.q.double().numpy(), inp.k.double().numpy(), inp.v.double().numpy()
    s0 = None if inp.initial_state is None else inp.initial_state.double().numpy()
    cu = inp.cu_seqlens.numpy()
    if heads is None:
        o, f = orc.prefill(q, k, v, g, beta, cu, s0, scale=scale)
        return torch.from_numpy(o), torch.from_numpy(f)
    ratio = inp.shape.h_v // inp.shape.h_qk
    res = {}
    for hq in heads:
        hv = slice(hq * ratio, (hq + 1) * ratio)
        o, f = orc.prefill(q[:, hq:hq + 1], k[:, hq:hq + 1], v[:, hv], g[:, hv], beta[:, hv], cu,
                           None if s0 is None else s0[:, hv], scale=scale)
        res[hq] = (torch.from_numpy(o), torch.from_numpy(f))
    return res


def max_err(gpu: torch.Tensor, ref: torch.Tensor) -> float:
    gpu = gpu.double()
    ref = ref.double()
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.numel() == 0:
        return 0.0
    assert torch.isfinite(gpu).all(), "non-finite values in the GPU result (an element was not written?)"
    return float(((gpu - ref).abs() / (1.0 + ref.abs())).max())


def rel_errors(gpu: torch.Tensor, ref: torch.Tensor):
    """(||d||_F / ||ref||_F, max |d|/|ref| over |ref| >= 1e-3) with d = gpu - ref.
    The normwise figure falls back to ||d||_F when ref is all zero."""
    d = gpu.double() - ref.double()
    r = ref.double()
    if r.numel() == 0:
        return 0.0, 0.0
    nref = float(r.norm())
    fro = float(d.norm()) / nref if nref > 0 else float(d.norm())
    big = r.abs() >= 1e-3
    mrel = float((d.abs()[big] / r.abs()[big]).max()) if bool(big.any()) else 0.0
    return fro, mrel


# Half-precision I/O ("<= 1e-2 relative" for bfloat16) is held to a normwise
# relative bound as well as the elementwise one: at these workloads the
# outputs have an RMS near 5e-3, so tol (1 + |ref|) alone would admit errors
# of the outputs' own size.  float32 I/O keeps the stated elementwise bound.


def check(gpu, ref, tol, what, normwise=None):
    """Assert |gpu - ref| <= tol (1 + |ref|) elementwise and, for half-precision
    tolerances (tol >= 1e-3, i.e. bf16 and f16 I/O) or when ``normwise`` is
    True, ||gpu - ref||_F <= tol ||ref||_F.  Prints both, and the largest
    elementwise relative error over |ref| >= 1e-3."""
    e = max_err(gpu, ref)
    fro, mrel = rel_errors(gpu, ref)
    if normwise is None:
        normwise = tol >= 1e-3
    say(f"    {what}: max |d|/(1+|ref|) = {e:.3e}  (tol {tol:.0e}), ||d||/||ref|| = {fro:.3e}"
        f"{' (asserted)' if normwise else ''}, max |d|/|ref| over |ref|>=1e-3 = {mrel:.3e}")
    assert e <= tol, f"{what}: {e:.3e} > {tol:.0e}"
    if normwise:
        assert fro <= tol, f"{what}: normwise relative error {fro:.3e} > {tol:.0e}"
    return e
