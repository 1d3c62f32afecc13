"""ctypes binding of libgdn (include/gdn.h).

Argument marshalling only: tensors are turned into device pointers, shapes
into the ``gdn_problem`` struct, and the C entry points of the same names are
called on the current HIP stream.  Every step of the recurrence runs in the
library's HIP kernels; there is no other code path.  If ``libgdn.so`` is not
built, or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "gdn.h")

GDN_OK, GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, 1, 2, 3
GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
GDN_GATES_PRECOMPUTED, GDN_GATES_RAW = 0, 1
GDN_ALGO_AUTO, GDN_ALGO_SERIAL, GDN_ALGO_CHUNKED = 0, 1, 2
ALGORITHMS = {"auto": GDN_ALGO_AUTO, "serial": GDN_ALGO_SERIAL, "chunked": GDN_ALGO_CHUNKED}
RULES = {"gated_delta": 0, "delta": 1, "gated": 2, "linear": 3}
GDN_ACT_NONE, GDN_ACT_SILU, GDN_ACT_SIGMOID = 0, 1, 2
ACTIVATIONS = {"none": GDN_ACT_NONE, "silu": GDN_ACT_SILU, "swish": GDN_ACT_SILU, "sigmoid": GDN_ACT_SIGMOID}

_DTYPES = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}


class gdn_problem(ctypes.Structure):
    _fields_ = [
        ("h_qk", ctypes.c_int32), ("h_v", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("gate_mode", ctypes.c_int32),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("algorithm", ctypes.c_int32),
        ("rule", ctypes.c_int32),
        ("decay_per_key", ctypes.c_int32),
        ("beta_shared", ctypes.c_int32),
        ("state_window", ctypes.c_int32),
        ("state_history", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
        ("norm_gate", ctypes.c_void_p), ("norm_scale", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float), ("norm_activation", ctypes.c_int32),
    ]


class gdn_prefill_plan(ctypes.Structure):
    _fields_ = [
        ("form", ctypes.c_int32), ("columns_per_block", ctypes.c_int32),
        ("state_workgroups", ctypes.c_int32), ("norm", ctypes.c_int32), ("kernels", ctypes.c_char * 184),
    ]


FORMS = {0: "none", 1: "serial", 2: "chunked_one_pass", 3: "chunked_two_pass", 4: "chunked_f32"}


class gdn_conv_problem(ctypes.Structure):
    _fields_ = [
        ("channels", ctypes.c_int32), ("kernel_size", ctypes.c_int32),
        ("dilation", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_serial_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    pp = ctypes.POINTER(gdn_problem)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.gdn_prefill.argtypes = [pp, i32, vp, ip, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [pp, i32, vp, vp, vp, vp, vp, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_prefill_slots.argtypes = [pp, i32, vp, ip, i32, vp, vp, vp, vp, i32, vp, ip, vp, vp]
    lib.gdn_prefill_slots.restype = ctypes.c_int
    lib.gdn_decode_step_slots.argtypes = [pp, i32, vp, vp, vp, vp, i32, vp, ip, vp, vp]
    lib.gdn_decode_step_slots.restype = ctypes.c_int
    lib.gdn_gate_prologue.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_gate_prologue.restype = ctypes.c_int
    cp = ctypes.POINTER(gdn_conv_problem)
    lib.gdn_causal_conv.argtypes = [cp, i32, vp, ip, i32, vp, vp, vp, vp, vp]
    lib.gdn_causal_conv.restype = ctypes.c_int
    lib.gdn_causal_conv_step.argtypes = [cp, i32, vp, vp, vp, vp]
    lib.gdn_causal_conv_step.restype = ctypes.c_int
    lib.gdn_causal_conv_slots.argtypes = [cp, i32, vp, ip, i32, vp, vp, i32, vp, ip, vp, vp]
    lib.gdn_causal_conv_slots.restype = ctypes.c_int
    lib.gdn_causal_conv_step_slots.argtypes = [cp, i32, vp, vp, i32, vp, ip, vp, vp]
    lib.gdn_causal_conv_step_slots.restype = ctypes.c_int
    lib.gdn_decode_step_conv.argtypes = [pp, cp, i32, vp, vp, vp, vp, vp, vp]
    lib.gdn_decode_step_conv.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [ctypes.c_int64, i32, i32, i32, vp, vp, vp, ctypes.c_float, i32, vp, vp]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size.argtypes = [pp, i32, i32, ctypes.POINTER(ctypes.c_uint64)]
    lib.gdn_prefill_workspace_size.restype = ctypes.c_int
    lib.gdn_prefill_static_workspace.argtypes = [pp, i32, vp, ip, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_prefill_static_workspace.restype = ctypes.c_int
    lib.gdn_prefill_query_plan.argtypes = [pp, i32, i32, ctypes.POINTER(gdn_prefill_plan)]
    lib.gdn_prefill_query_plan.restype = ctypes.c_int
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def header_symbols(path: str = HEADER) -> list:
    """Names of the functions include/gdn.h declares."""
    with open(path) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(gdn_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def status_string(status: int) -> str:
    return load().gdn_status_string(status).decode()


def last_error() -> str:
    return load().gdn_last_error().decode()


def abi_version() -> int:
    return int(load().gdn_abi_version())


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libgdn takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr()) if t.data_ptr() else None


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def make_problem(h_qk: int, h_v: int, d_k: int, d_v: int, io_dtype: torch.dtype, *, scale: float = 0.0,
                 g=None, beta=None, a=None, b=None, A_log=None, dt_bias=None,
                 algorithm: str = "auto", rule: str = "gated_delta", decay_per_key: bool = False,
                 beta_shared: bool = False, state_history: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, norm_gate: Optional[torch.Tensor] = None,
                 norm_scale: Optional[torch.Tensor] = None, norm_eps: float = 1e-5,
                 norm_activation: str = "silu") -> gdn_problem:
    """Fill the ``gdn_problem`` struct.  Raw gates are used when ``a`` (or, for
    rules without decay, ``b``) is given.  ``state_history`` [N, W, h_v, d_k, d_v]
    sets the state window W; ``workspace`` (a device tensor of at least
    prefill_workspace_size bytes) enables the two-pass chunked prefill;
    ``norm_gate`` [tokens, h_v, d_v] and ``norm_scale`` [d_v] ask for the gated
    RMSNorm of the output (per value head)."""
    if io_dtype not in _DTYPES:
        raise ValueError(f"io dtype {io_dtype} is not supported")
    raw = a is not None or (g is None and b is not None)
    window = 0 if state_history is None else int(state_history.shape[1])
    return gdn_problem(h_qk, h_v, d_k, d_v, _DTYPES[io_dtype], float(scale),
                       GDN_GATES_RAW if raw else GDN_GATES_PRECOMPUTED,
                       _ptr(g), _ptr(beta), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                       ALGORITHMS[algorithm], RULES[rule], int(decay_per_key), int(beta_shared),
                       window, _ptr(state_history), _ptr(workspace),
                       0 if workspace is None else workspace.numel() * workspace.element_size(),
                       _ptr(norm_gate), _ptr(norm_scale), float(norm_eps), ACTIVATIONS[norm_activation])


def gdn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                out: Optional[torch.Tensor], final_state: Optional[torch.Tensor],
                initial_state: Optional[torch.Tensor] = None, g=None, beta=None, a=None, b=None,
                A_log=None, dt_bias=None, scale: float = 0.0,
                cu_seqlens_host: Optional[Sequence[int]] = None, algorithm: str = "auto",
                stream=None, **variant) -> None:
    """gdn_prefill of include/gdn.h: q, k [T, h_qk, d_k]; v, out [T, h_v, d_v];
    cu_seqlens int32 [N+1] on the device; states float32 [N, h_v, d_k, d_v];
    algorithm "auto", "serial" or "chunked"; ``variant``: rule, decay_per_key,
    beta_shared, state_history, workspace (see make_problem)."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    prob = make_problem(h_qk, h_v, d_k, d_v, q.dtype, scale=scale, g=g, beta=beta, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, algorithm=algorithm, **variant)
    n = cu_seqlens.numel() - 1
    host = None
    if cu_seqlens_host is not None:
        vals = [int(x) for x in cu_seqlens_host]
        host = (ctypes.c_int32 * len(vals))(*vals)
    _check(load().gdn_prefill(ctypes.byref(prob), n, _ptr(cu_seqlens), host, T, _ptr(q), _ptr(k), _ptr(v),
                              _ptr(initial_state), _ptr(out), _ptr(final_state), _stream(stream, q.device)))


STATIC_WORKSPACE_BYTES = 64 << 20


def gdn_prefill_static_workspace(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                                 out: Optional[torch.Tensor], final_state: Optional[torch.Tensor],
                                 initial_state: Optional[torch.Tensor] = None, g=None, beta=None, a=None, b=None,
                                 A_log=None, dt_bias=None, scale: float = 0.0,
                                 cu_seqlens_host: Optional[Sequence[int]] = None, algorithm: str = "auto",
                                 stream=None, **variant) -> None:
    """gdn_prefill_static_workspace of include/gdn.h: gdn_prefill with the
    two-pass form's workspace taken from the library's own device array (no
    ``workspace`` argument)."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    prob = make_problem(h_qk, h_v, d_k, d_v, q.dtype, scale=scale, g=g, beta=beta, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, algorithm=algorithm, **variant)
    n = cu_seqlens.numel() - 1
    _check(load().gdn_prefill_static_workspace(ctypes.byref(prob), n, _ptr(cu_seqlens), _host_i32(cu_seqlens_host),
                                               T, _ptr(q), _ptr(k), _ptr(v), _ptr(initial_state), _ptr(out),
                                               _ptr(final_state), _stream(stream, q.device)))


def gdn_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: torch.Tensor,
                    out: torch.Tensor, *, g=None, beta=None, a=None, b=None, A_log=None, dt_bias=None,
                    scale: float = 0.0, stream=None, **variant) -> None:
    """gdn_decode_step of include/gdn.h: q, k [B, h_qk, d_k]; v, out [B, h_v, d_v];
    state float32 [B, h_v, d_k, d_v], updated in place; ``variant``: rule,
    decay_per_key, beta_shared."""
    B, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    prob = make_problem(h_qk, h_v, d_k, d_v, q.dtype, scale=scale, g=g, beta=beta, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, **variant)
    _check(load().gdn_decode_step(ctypes.byref(prob), B, _ptr(q), _ptr(k), _ptr(v), _ptr(state), _ptr(out),
                                  _stream(stream, q.device)))


def prefill_workspace_size(h_qk: int, h_v: int, d_k: int, d_v: int, io_dtype: torch.dtype, num_seqs: int,
                           total_tokens: int, *, algorithm: str = "auto", **variant) -> int:
    """gdn_prefill_workspace_size of include/gdn.h (0 when the two-pass form does not apply)."""
    prob = make_problem(h_qk, h_v, d_k, d_v, io_dtype, algorithm=algorithm, **variant)
    out = ctypes.c_uint64(0)
    _check(load().gdn_prefill_workspace_size(ctypes.byref(prob), num_seqs, total_tokens, ctypes.byref(out)))
    return int(out.value)


def prefill_query_plan(h_qk: int, h_v: int, d_k: int, d_v: int, io_dtype: torch.dtype, num_seqs: int,
                       total_tokens: int, *, algorithm: str = "auto", raw_gates: bool = False,
                       workspace_bytes: int = 0, norm: bool = False, **variant) -> dict:
    """gdn_prefill_query_plan of include/gdn.h: what gdn_prefill would launch.
    ``workspace_bytes`` stands for a workspace of that size (no memory is
    touched).  Returns {"form", "columns_per_block", "state_workgroups", "kernels"}."""
    prob = make_problem(h_qk, h_v, d_k, d_v, io_dtype, algorithm=algorithm, **variant)
    if raw_gates:
        prob.gate_mode = GDN_GATES_RAW
    if norm:
        prob.norm_gate = prob.norm_scale = ctypes.c_void_p(512)  # stand-ins: the query reads no memory
    if workspace_bytes:
        prob.workspace = ctypes.c_void_p(256)  # a non-null, aligned stand-in: the query reads no memory
        prob.workspace_bytes = int(workspace_bytes)
    plan = gdn_prefill_plan()
    _check(load().gdn_prefill_query_plan(ctypes.byref(prob), num_seqs, total_tokens, ctypes.byref(plan)))
    return {"form": FORMS.get(plan.form, str(plan.form)), "columns_per_block": plan.columns_per_block,
            "state_workgroups": plan.state_workgroups, "norm": {0: "none", 1: "fused", 2: "separate pass"}[plan.norm],
            "kernels": plan.kernels.decode()}


def _host_i32(vals):
    if vals is None:
        return None
    vals = [int(x) for x in vals]
    return (ctypes.c_int32 * len(vals))(*vals)


def gdn_prefill_slots(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                      state_pool: torch.Tensor, slots: torch.Tensor, *, out: Optional[torch.Tensor], g=None,
                      beta=None, a=None, b=None, A_log=None, dt_bias=None, scale: float = 0.0,
                      cu_seqlens_host: Optional[Sequence[int]] = None, slots_host: Optional[Sequence[int]] = None,
                      algorithm: str = "auto", workspace: Optional[torch.Tensor] = None, stream=None,
                      **variant) -> None:
    """gdn_prefill_slots of include/gdn.h: sequence i runs from and writes back
    state_pool[slots[i]] (float32 [num_slots, h_v, d_k, d_v]); ``variant`` as
    for gdn_prefill."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    prob = make_problem(h_qk, h_v, d_k, d_v, q.dtype, scale=scale, g=g, beta=beta, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, algorithm=algorithm, workspace=workspace, **variant)
    n = cu_seqlens.numel() - 1
    _check(load().gdn_prefill_slots(ctypes.byref(prob), n, _ptr(cu_seqlens), _host_i32(cu_seqlens_host), T,
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(state_pool), state_pool.shape[0], _ptr(slots),
                                    _host_i32(slots_host), _ptr(out), _stream(stream, q.device)))


def gdn_decode_step_slots(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state_pool: torch.Tensor,
                          slots: torch.Tensor, out: torch.Tensor, *, g=None, beta=None, a=None, b=None,
                          A_log=None, dt_bias=None, scale: float = 0.0,
                          slots_host: Optional[Sequence[int]] = None, stream=None, **variant) -> None:
    """gdn_decode_step_slots of include/gdn.h: sequence i updates state_pool[slots[i]] in place;
    ``variant``: rule, decay_per_key, beta_shared, norm_* (see make_problem)."""
    B, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    prob = make_problem(h_qk, h_v, d_k, d_v, q.dtype, scale=scale, g=g, beta=beta, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, **variant)
    _check(load().gdn_decode_step_slots(ctypes.byref(prob), B, _ptr(q), _ptr(k), _ptr(v), _ptr(state_pool),
                                        state_pool.shape[0], _ptr(slots), _host_i32(slots_host), _ptr(out),
                                        _stream(stream, q.device)))


def gdn_gate_prologue(a: torch.Tensor, b: Optional[torch.Tensor], A_log: torch.Tensor, dt_bias: torch.Tensor,
                      *, g: Optional[torch.Tensor], beta: Optional[torch.Tensor], stream=None) -> None:
    """gdn_gate_prologue of include/gdn.h: a, b, g, beta [tokens, h_v]; A_log, dt_bias float32 [h_v]."""
    tokens, h_v = a.shape
    _check(load().gdn_gate_prologue(tokens, h_v, _DTYPES[a.dtype], _ptr(a), _ptr(b), _ptr(A_log),
                                    _ptr(dt_bias), _ptr(g), _ptr(beta), _stream(stream, a.device)))


def make_conv_problem(weight: torch.Tensor, bias: Optional[torch.Tensor] = None, *, dilation: int = 1,
                      activation: str = "silu") -> gdn_conv_problem:
    """Fill the ``gdn_conv_problem`` struct from weight [C, K] (and bias [C])."""
    if weight.dtype not in _DTYPES:
        raise ValueError(f"io dtype {weight.dtype} is not supported")
    C, K = weight.shape
    return gdn_conv_problem(C, K, int(dilation), _DTYPES[weight.dtype], ACTIVATIONS[activation],
                            _ptr(weight), _ptr(bias))


def gdn_causal_conv(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor, *, y: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None, dilation: int = 1, activation: str = "silu",
                    cu_seqlens_host: Optional[Sequence[int]] = None, stream=None) -> None:
    """gdn_causal_conv of include/gdn.h: x, y [T, C]; weight [C, K]; states
    [N, (K - 1) dilation, C], all in the I/O dtype; cu_seqlens int32 [N+1]."""
    prob = make_conv_problem(weight, bias, dilation=dilation, activation=activation)
    n = cu_seqlens.numel() - 1
    _check(load().gdn_causal_conv(ctypes.byref(prob), n, _ptr(cu_seqlens), _host_i32(cu_seqlens_host), x.shape[0],
                                  _ptr(x), _ptr(initial_state), _ptr(y), _ptr(final_state),
                                  _stream(stream, x.device)))


def gdn_causal_conv_step(x: torch.Tensor, weight: torch.Tensor, state: torch.Tensor, *, y: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, dilation: int = 1, activation: str = "silu",
                         stream=None) -> None:
    """gdn_causal_conv_step of include/gdn.h: x, y [B, C]; state [B, carry, C], shifted in place."""
    prob = make_conv_problem(weight, bias, dilation=dilation, activation=activation)
    _check(load().gdn_causal_conv_step(ctypes.byref(prob), x.shape[0], _ptr(x), _ptr(state), _ptr(y),
                                       _stream(stream, x.device)))


def gdn_decode_step_conv(x: torch.Tensor, conv_weight: torch.Tensor, conv_state: Optional[torch.Tensor],
                         conv_state_out: Optional[torch.Tensor], state: torch.Tensor, out: torch.Tensor, *,
                         h_qk: int, d_k: int, conv_bias: Optional[torch.Tensor] = None, conv_activation: str = "silu",
                         g=None, beta=None, a=None, b=None, A_log=None, dt_bias=None, scale: float = 0.0,
                         stream=None, **variant) -> None:
    """gdn_decode_step_conv of include/gdn.h: x [B, C] with C = 2 h_qk d_k + h_v d_v
    (q | k | v); conv_state, conv_state_out [B, K - 1, C] (distinct buffers, or
    None when K = 1); state float32 [B, h_v, d_k, d_v], updated in place; out
    [B, h_v, d_v].  ``variant`` as in gdn_decode_step (rule, norm_gate, ...)."""
    B = x.shape[0]
    h_v, d_v = out.shape[1], out.shape[2]
    prob = make_problem(h_qk, h_v, d_k, d_v, x.dtype, scale=scale, g=g, beta=beta, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, **variant)
    cprob = make_conv_problem(conv_weight, conv_bias, dilation=1, activation=conv_activation)
    _check(load().gdn_decode_step_conv(ctypes.byref(prob), ctypes.byref(cprob), B, _ptr(x), _ptr(conv_state),
                                       _ptr(conv_state_out), _ptr(state), _ptr(out), _stream(stream, x.device)))


def gdn_causal_conv_slots(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor, state_pool: torch.Tensor,
                          slots: torch.Tensor, *, y: torch.Tensor, bias: Optional[torch.Tensor] = None,
                          dilation: int = 1, activation: str = "silu", cu_seqlens_host: Optional[Sequence[int]] = None,
                          slots_host: Optional[Sequence[int]] = None, stream=None) -> None:
    """gdn_causal_conv_slots of include/gdn.h: sequence i runs from and writes
    back state_pool[slots[i]] ([num_slots, carry, C], the I/O dtype)."""
    prob = make_conv_problem(weight, bias, dilation=dilation, activation=activation)
    n = cu_seqlens.numel() - 1
    _check(load().gdn_causal_conv_slots(ctypes.byref(prob), n, _ptr(cu_seqlens), _host_i32(cu_seqlens_host),
                                        x.shape[0], _ptr(x), _ptr(state_pool), state_pool.shape[0], _ptr(slots),
                                        _host_i32(slots_host), _ptr(y), _stream(stream, x.device)))


def gdn_causal_conv_step_slots(x: torch.Tensor, weight: torch.Tensor, state_pool: torch.Tensor, slots: torch.Tensor,
                               *, y: torch.Tensor, bias: Optional[torch.Tensor] = None, dilation: int = 1,
                               activation: str = "silu", slots_host: Optional[Sequence[int]] = None,
                               stream=None) -> None:
    """gdn_causal_conv_step_slots of include/gdn.h: one token per sequence, the
    state of sequence i at state_pool[slots[i]] shifted in place."""
    prob = make_conv_problem(weight, bias, dilation=dilation, activation=activation)
    _check(load().gdn_causal_conv_step_slots(ctypes.byref(prob), x.shape[0], _ptr(x), _ptr(state_pool),
                                             state_pool.shape[0], _ptr(slots), _host_i32(slots_host), _ptr(y),
                                             _stream(stream, x.device)))


def gdn_gated_rmsnorm(x: torch.Tensor, gate: torch.Tensor, scale: torch.Tensor, *, y: torch.Tensor,
                      eps: float = 1e-5, activation: str = "silu", stream=None) -> None:
    """gdn_gated_rmsnorm of include/gdn.h over groups of len(scale) elements of
    x's last axis; x, gate, y share a shape, all in the I/O dtype."""
    width = x.shape[-1]
    rows = x.numel() // width if width else 0
    _check(load().gdn_gated_rmsnorm(rows, width, scale.numel(), _DTYPES[x.dtype], _ptr(x), _ptr(gate), _ptr(scale),
                                    float(eps), ACTIVATIONS[activation], _ptr(y), _stream(stream, x.device)))


# ----------------------------------------------------------------- helpers
def prefill(q, k, v, cu_seqlens, *, initial_state=None, want_state=True, scale=0.0,
            cu_seqlens_host=None, algorithm="auto", two_pass=True, stream=None, **kw):
    """Allocate ``out`` (and the final state, and the chunked form's workspace
    unless two_pass is False) with torch and call gdn_prefill."""
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n = cu_seqlens.numel() - 1
    out = torch.empty(T, h_v, d_v, dtype=q.dtype, device=q.device)
    fin = torch.empty(n, h_v, d_k, d_v, dtype=torch.float32, device=q.device) if want_state else None
    ws = None
    if two_pass and "workspace" not in kw:
        variant = {key: kw[key] for key in ("rule", "decay_per_key", "beta_shared", "state_history") if key in kw}
        nbytes = prefill_workspace_size(h_qk, h_v, d_k, d_v, q.dtype, n, T, algorithm=algorithm, **variant)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    gdn_prefill(q, k, v, cu_seqlens, out=out, final_state=fin, initial_state=initial_state, scale=scale,
                cu_seqlens_host=cu_seqlens_host, algorithm=algorithm, stream=stream,
                **({"workspace": ws} if ws is not None else {}), **kw)
    return out, fin


def decode_step(q, k, v, state, *, scale=0.0, stream=None, **kw):
    """Allocate ``out`` with torch and call gdn_decode_step (state updated in place)."""
    out = torch.empty(q.shape[0], v.shape[1], v.shape[2], dtype=q.dtype, device=q.device)
    gdn_decode_step(q, k, v, state, out, scale=scale, stream=stream, **kw)
    return out


def causal_conv(x, weight, cu_seqlens, *, bias=None, initial_state=None, want_state=True, dilation=1,
                activation="silu", cu_seqlens_host=None, stream=None):
    """Allocate y (and the final state) with torch and call gdn_causal_conv."""
    C, K = weight.shape
    n = cu_seqlens.numel() - 1
    y = torch.empty_like(x)
    fin = torch.empty(n, (K - 1) * dilation, C, dtype=x.dtype, device=x.device) if want_state else None
    gdn_causal_conv(x, weight, cu_seqlens, y=y, bias=bias, initial_state=initial_state, final_state=fin,
                    dilation=dilation, activation=activation, cu_seqlens_host=cu_seqlens_host, stream=stream)
    return y, fin


def gated_rmsnorm(x, gate, scale, *, eps=1e-5, activation="silu", stream=None):
    """Allocate y with torch and call gdn_gated_rmsnorm."""
    y = torch.empty_like(x)
    gdn_gated_rmsnorm(x, gate, scale, y=y, eps=eps, activation=activation, stream=stream)
    return y


def gate_prologue(a, b, A_log, dt_bias, *, stream=None):
    """Allocate g and beta with torch and call gdn_gate_prologue."""
    g = torch.empty_like(a)
    beta = torch.empty_like(b)
    gdn_gate_prologue(a, b, A_log, dt_bias, g=g, beta=beta, stream=stream)
    return g, beta
