"""The C ABI on the CPU: the library loads, exports what include/gdn.h
declares, and rejects malformed calls on the host with the documented status
before anything reaches a GPU.  Every call here fails validation, so no
device work is ever attempted."""
import ctypes
import os
import subprocess

import pytest
import torch

from gated_delta_rule_serial_amd import gdn

pytestmark = pytest.mark.skipif(not os.path.exists(gdn.LIB_PATH), reason="libgdn.so not built")

FAKE = 0x100000  # 16-byte aligned non-null address; never dereferenced by validation


@pytest.fixture(scope="module")
def lib():
    return gdn.load()


def test_exports_every_declared_symbol(lib):
    declared = gdn.header_symbols()
    assert set(declared) >= {"gdn_prefill", "gdn_decode_step", "gdn_gate_prologue", "gdn_last_error",
                             "gdn_status_string", "gdn_abi_version"}
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/gdn.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(declared), f"exported functions {sorted(exported)} != declared {declared}"


def test_version_and_status_strings(lib):
    assert gdn.abi_version() == 10
    assert gdn.status_string(0) == "GDN_OK"
    assert gdn.status_string(1) == "GDN_ERR_INVALID_ARGUMENT"
    assert gdn.status_string(2) == "GDN_ERR_UNSUPPORTED"
    assert gdn.status_string(3) == "GDN_ERR_HIP"
    assert gdn.status_string(99) == "GDN_STATUS_UNKNOWN"


def _prob(**kw):
    base = dict(h_qk=2, h_v=4, d_k=16, d_v=16, io_dtype=gdn.GDN_F32, scale=0.0,
                gate_mode=gdn.GDN_GATES_PRECOMPUTED, g=FAKE, beta=FAKE + 0x1000, a=None, b=None,
                A_log=None, dt_bias=None, algorithm=gdn.GDN_ALGO_AUTO, rule=0, decay_per_key=0, beta_shared=0,
                state_window=0, state_history=None, workspace=None, workspace_bytes=0)
    base.update(kw)
    return gdn.gdn_problem(**base)


def _prefill(lib, prob, *, n=1, cu=FAKE + 0x2000, cu_host=None, T=8, q=FAKE + 0x10000, k=FAKE + 0x20000,
             v=FAKE + 0x30000, s0=None, out=FAKE + 0x40000, sN=FAKE + 0x50000):
    host = None
    if cu_host is not None:
        host = (ctypes.c_int32 * len(cu_host))(*cu_host)
    vp = ctypes.c_void_p
    return lib.gdn_prefill(ctypes.byref(prob) if prob is not None else None, n, vp(cu) if cu else None, host, T,
                           vp(q) if q else None, vp(k) if k else None, vp(v) if v else None,
                           vp(s0) if s0 else None, vp(out) if out else None, vp(sN) if sN else None, None)


INVALID, UNSUPPORTED = gdn.GDN_ERR_INVALID_ARGUMENT, gdn.GDN_ERR_UNSUPPORTED


@pytest.mark.parametrize("label,prob_kw,call_kw,status,needle", [
    ("null problem", None, {}, INVALID, "problem is NULL"),
    ("zero heads", dict(h_qk=0), {}, INVALID, "head counts"),
    ("head ratio", dict(h_qk=3, h_v=4), {}, INVALID, "not a multiple"),
    ("zero d_k", dict(d_k=0), {}, INVALID, "head sizes must be positive"),
    ("d_k too large", dict(d_k=257), {}, UNSUPPORTED, "above 256"),
    ("d_v too large", dict(d_v=512), {}, UNSUPPORTED, "above 256"),
    ("dtype", dict(io_dtype=7), {}, UNSUPPORTED, "io_dtype"),
    ("nan scale", dict(scale=float("nan")), {}, INVALID, "scale"),
    ("missing g", dict(g=None), {}, INVALID, "precomputed gates"),
    ("missing raw", dict(gate_mode=gdn.GDN_GATES_RAW, a=FAKE), {}, INVALID, "raw gates"),
    ("bad gate mode", dict(gate_mode=5), {}, INVALID, "gate_mode"),
    ("bad algorithm", dict(algorithm=7), {}, INVALID, "algorithm"),
    ("chunked on f32", dict(algorithm=gdn.GDN_ALGO_CHUNKED), {}, UNSUPPORTED, "chunked algorithm needs"),
    ("chunked on f16", dict(algorithm=gdn.GDN_ALGO_CHUNKED, io_dtype=gdn.GDN_F16, d_k=64, d_v=64), {}, UNSUPPORTED,
     "got f16"),
    ("chunked on d_k 48", dict(algorithm=gdn.GDN_ALGO_CHUNKED, io_dtype=gdn.GDN_BF16, d_k=48), {}, UNSUPPORTED,
     "chunked algorithm needs"),
    ("misaligned g", dict(g=FAKE + 2), {}, INVALID, "aligned"),
    ("bad rule", dict(rule=4), {}, INVALID, "unknown rule"),
    ("bad flag", dict(beta_shared=2), {}, INVALID, "must be 0 or 1"),
    ("per-key g misaligned", dict(decay_per_key=1, g=FAKE + 8), {}, INVALID, "16-byte"),
    ("delta rule needs beta", dict(rule=1, beta=None), {}, INVALID, "need g and beta"),
    ("window without history", dict(state_window=3), {}, INVALID, "needs state_history"),
    ("negative window", dict(state_window=-1), {}, INVALID, "negative"),
    ("chunked per-key", dict(algorithm=gdn.GDN_ALGO_CHUNKED, io_dtype=gdn.GDN_BF16, d_k=64, d_v=64,
                             decay_per_key=1), {}, UNSUPPORTED, "chunked algorithm needs"),
    ("chunked gated rule", dict(algorithm=gdn.GDN_ALGO_CHUNKED, io_dtype=gdn.GDN_BF16, d_k=64, d_v=12, rule=2),
     {}, UNSUPPORTED, "chunked algorithm needs"),
    ("negative seqs", {}, dict(n=-1), INVALID, "negative"),
    ("negative tokens", {}, dict(T=-1), INVALID, "negative"),
    ("tokens without seqs", {}, dict(n=0, T=4), INVALID, "no sequences"),
    ("null cu", {}, dict(cu=0), INVALID, "cu_seqlens is NULL"),
    ("null q", {}, dict(q=0), INVALID, "required"),
    ("misaligned q", {}, dict(q=FAKE + 0x10004), INVALID, "16-byte"),
    ("misaligned state", {}, dict(s0=FAKE + 0x60008), INVALID, "16-byte"),
    ("cu not from 0", {}, dict(cu_host=[1, 8]), INVALID, "expected 0"),
    ("cu decreasing", {}, dict(n=2, cu_host=[0, 5, 4]), INVALID, "decreases"),
    ("cu total", {}, dict(cu_host=[0, 7]), INVALID, "total_tokens"),
    ("state partial overlap", {}, dict(s0=FAKE + 0x50000, sN=FAKE + 0x50010), INVALID, "partially overlaps"),
    ("out overlaps q", {}, dict(out=FAKE + 0x10000), INVALID, "out overlaps"),
])
def test_prefill_validation(lib, label, prob_kw, call_kw, status, needle):
    prob = None if prob_kw is None else _prob(**prob_kw)
    st = _prefill(lib, prob, **call_kw)
    assert st == status, f"{label}: status {st}, message {gdn.last_error()!r}"
    assert needle in gdn.last_error(), f"{label}: message {gdn.last_error()!r}"


def test_prefill_nothing_to_do_is_ok(lib):
    # no sequences at all: OK without any launch
    assert _prefill(lib, _prob(), n=0, T=0, cu=0, q=0, k=0, v=0, out=0, sN=0) == gdn.GDN_OK
    assert gdn.last_error() == ""


@pytest.mark.parametrize("label,prob_kw,args,status,needle", [
    ("negative batch", {}, dict(B=-1), INVALID, "negative"),
    ("null state", {}, dict(state=0), INVALID, "required"),
    ("misaligned out", {}, dict(out=FAKE + 0x40002), INVALID, "16-byte"),
    ("out overlaps state", {}, dict(out=FAKE + 0x50000), INVALID, "overlaps"),
    ("state overlaps q", {}, dict(state=FAKE + 0x10000), INVALID, "overlaps"),
    ("ratio", dict(h_qk=3), {}, INVALID, "not a multiple"),
])
def test_decode_validation(lib, label, prob_kw, args, status, needle):
    a = dict(B=4, q=FAKE + 0x10000, k=FAKE + 0x20000, v=FAKE + 0x30000, state=FAKE + 0x50000,
             out=FAKE + 0x40000)
    a.update(args)
    vp = ctypes.c_void_p
    st = lib.gdn_decode_step(ctypes.byref(_prob(**prob_kw)), a["B"], vp(a["q"]), vp(a["k"]), vp(a["v"]),
                             vp(a["state"]) if a["state"] else None, vp(a["out"]), None)
    assert st == status, f"{label}: status {st}, message {gdn.last_error()!r}"
    assert needle in gdn.last_error()


def test_decode_empty_batch_is_ok(lib):
    assert lib.gdn_decode_step(ctypes.byref(_prob()), 0, None, None, None, None, None, None) == gdn.GDN_OK


@pytest.mark.parametrize("args,status,needle", [
    (dict(tokens=-1), INVALID, "tokens"),
    (dict(h_v=0), INVALID, "h_v"),
    (dict(dtype=3), UNSUPPORTED, "io_dtype"),
    (dict(dtype=-1), UNSUPPORTED, "io_dtype"),
    (dict(a=0), INVALID, "g needs"),
    (dict(b=0), INVALID, "beta needs"),
    (dict(g=FAKE + 0x40001), INVALID, "aligned"),
])
def test_gate_prologue_validation(lib, args, status, needle):
    a = dict(tokens=8, h_v=4, dtype=gdn.GDN_BF16, a=FAKE, b=FAKE + 0x1000, A_log=FAKE + 0x2000,
             dt_bias=FAKE + 0x3000, g=FAKE + 0x4000, beta=FAKE + 0x5000)
    a.update(args)
    vp = ctypes.c_void_p
    st = lib.gdn_gate_prologue(a["tokens"], a["h_v"], a["dtype"], *(vp(a[x]) if a[x] else None for x in
                                                                      ("a", "b", "A_log", "dt_bias", "g", "beta")),
                               None)
    assert st == status, gdn.last_error()
    assert needle in gdn.last_error()


def test_slot_validation(lib):
    vp = ctypes.c_void_p
    prob = _prob()
    host = (ctypes.c_int32 * 3)(2, 5, 2)
    cu_host = (ctypes.c_int32 * 4)(0, 2, 4, 8)
    st = lib.gdn_prefill_slots(ctypes.byref(prob), 3, vp(FAKE + 0x2000), cu_host, 8, vp(FAKE + 0x10000),
                               vp(FAKE + 0x20000), vp(FAKE + 0x30000), vp(FAKE + 0x80000), 6, vp(FAKE + 0x3000),
                               host, vp(FAKE + 0x40000), None)
    assert st == INVALID and "slot 2 is used by sequences 0 and 2" in gdn.last_error()
    st = lib.gdn_prefill_slots(ctypes.byref(prob), 3, vp(FAKE + 0x2000), cu_host, 8, vp(FAKE + 0x10000),
                               vp(FAKE + 0x20000), vp(FAKE + 0x30000), None, 6, vp(FAKE + 0x3000), None,
                               vp(FAKE + 0x40000), None)
    assert st == INVALID and "state_pool is NULL" in gdn.last_error()
    st = lib.gdn_decode_step_slots(ctypes.byref(prob), 4, vp(FAKE + 0x10000), vp(FAKE + 0x20000),
                                   vp(FAKE + 0x30000), vp(FAKE + 0x80000), 6, None, None, vp(FAKE + 0x40000), None)
    assert st == INVALID and "slots is NULL" in gdn.last_error()
    st = lib.gdn_decode_step_slots(ctypes.byref(prob), 4, vp(FAKE + 0x10000), vp(FAKE + 0x20000),
                                   vp(FAKE + 0x30000), vp(FAKE + 0x80000), -1, vp(FAKE + 0x3000), None,
                                   vp(FAKE + 0x40000), None)
    assert st == INVALID and "num_slots" in gdn.last_error()


# ------------------------------------------------------------------ conv and norm
def _conv_prob(**kw):
    base = dict(channels=64, kernel_size=4, dilation=1, io_dtype=gdn.GDN_BF16, activation=gdn.GDN_ACT_SILU,
                weight=FAKE + 0x6000, bias=None)
    base.update(kw)
    return gdn.gdn_conv_problem(**base)


def _conv(lib, prob, *, n=2, cu=FAKE + 0x2000, cu_host=(0, 3, 8), T=8, x=FAKE + 0x10000, s0=None,
          y=FAKE + 0x40000, sN=None):
    vp = ctypes.c_void_p
    host = None if cu_host is None else (ctypes.c_int32 * len(cu_host))(*cu_host)
    return lib.gdn_causal_conv(ctypes.byref(prob) if prob is not None else None, n, vp(cu) if cu else None, host,
                               T, vp(x) if x else None, vp(s0) if s0 else None, vp(y) if y else None,
                               vp(sN) if sN else None, None)


@pytest.mark.parametrize("label,prob_kw,call_kw,status,needle", [
    ("null problem", None, {}, INVALID, "problem is NULL"),
    ("channels", dict(channels=0), {}, INVALID, "channels"),
    ("kernel size", dict(kernel_size=0), {}, INVALID, "kernel_size"),
    ("dilation", dict(dilation=0), {}, INVALID, "dilation"),
    ("kernel too large", dict(kernel_size=65), {}, UNSUPPORTED, "above 64"),
    ("receptive field", dict(kernel_size=64, dilation=100), {}, UNSUPPORTED, "4096"),
    ("dtype", dict(io_dtype=5), {}, UNSUPPORTED, "io_dtype"),
    ("activation", dict(activation=gdn.GDN_ACT_SIGMOID), {}, INVALID, "activation"),
    ("weight misaligned", dict(weight=FAKE + 0x6002), {}, INVALID, "16-byte"),
    ("negative tokens", {}, dict(T=-1), INVALID, "must be >= 0"),
    ("tokens without sequences", {}, dict(n=0, cu_host=None), INVALID, "no sequences"),
    ("no cu", {}, dict(cu=None), INVALID, "cu_seqlens is NULL"),
    ("no x", {}, dict(x=None), INVALID, "required"),
    ("no weight", dict(weight=None), {}, INVALID, "required"),
    ("x misaligned", {}, dict(x=FAKE + 0x10008), INVALID, "16-byte"),
    ("cu start", {}, dict(cu_host=(1, 3, 8)), INVALID, "expected 0"),
    ("cu decreasing", {}, dict(cu_host=(0, 5, 3)), INVALID, "decreases"),
    ("cu total", {}, dict(cu_host=(0, 3, 7)), INVALID, "total_tokens"),
    ("y overlaps x", {}, dict(y=FAKE + 0x10000 + 0x100), INVALID, "y overlaps x"),
    ("state overlaps y", {}, dict(sN=FAKE + 0x40000 + 0x40), INVALID, "overlaps"),
    ("states partly overlap", {}, dict(s0=FAKE + 0x80000, sN=FAKE + 0x80000 + 0x40), INVALID, "partially"),
])
def test_conv_validation(lib, label, prob_kw, call_kw, status, needle):
    prob = None if prob_kw is None else _conv_prob(**prob_kw)
    st = _conv(lib, prob, **call_kw)
    assert st == status, (label, gdn.last_error())
    assert needle in gdn.last_error(), (label, gdn.last_error())


def test_conv_nothing_to_do_is_ok(lib):
    vp = ctypes.c_void_p
    assert _conv(lib, _conv_prob(), n=0, cu=None, cu_host=None, T=0, x=None, y=None) == gdn.GDN_OK
    assert lib.gdn_causal_conv_step(ctypes.byref(_conv_prob()), 0, None, None, None, None) == gdn.GDN_OK
    st = lib.gdn_causal_conv_step(ctypes.byref(_conv_prob()), 2, vp(FAKE), None, vp(FAKE + 0x1000), None)
    assert st == INVALID and "required" in gdn.last_error()
    st = lib.gdn_causal_conv_step(ctypes.byref(_conv_prob()), 2, vp(FAKE), vp(FAKE + 0x40), vp(FAKE + 0x1000), None)
    assert st == INVALID and "overlap" in gdn.last_error()


@pytest.mark.parametrize("args,status,needle", [
    (dict(rows=-1), INVALID, "rows"),
    (dict(width=0), INVALID, "width"),
    (dict(width=100, group=64), INVALID, "multiple"),
    (dict(dtype=9), UNSUPPORTED, "io_dtype"),
    (dict(act=gdn.GDN_ACT_NONE), INVALID, "activation"),
    (dict(eps=-1.0), INVALID, "eps"),
    (dict(eps=float("inf")), INVALID, "eps"),
    (dict(group=8192, width=8192), UNSUPPORTED, "larger"),
    (dict(group=513, width=513), UNSUPPORTED, "larger"),
    (dict(x=0), INVALID, "required"),
    (dict(gate=FAKE + 0x20004), INVALID, "16-byte"),
    (dict(y=FAKE + 0x20000), INVALID, "overlaps"),
    (dict(y=FAKE + 0x10010), INVALID, "overlaps"),
])
def test_gated_rmsnorm_validation(lib, args, status, needle):
    a = dict(rows=4, width=256, group=128, dtype=gdn.GDN_BF16, x=FAKE + 0x10000, gate=FAKE + 0x20000,
             scale=FAKE + 0x30000, eps=1e-5, act=gdn.GDN_ACT_SILU, y=FAKE + 0x40000)
    a.update(args)
    vp = ctypes.c_void_p
    st = lib.gdn_gated_rmsnorm(a["rows"], a["width"], a["group"], a["dtype"], vp(a["x"]) if a["x"] else None,
                               vp(a["gate"]), vp(a["scale"]), a["eps"], a["act"], vp(a["y"]), None)
    assert st == status, gdn.last_error()
    assert needle in gdn.last_error()


def test_gated_rmsnorm_no_rows_is_ok(lib):
    assert lib.gdn_gated_rmsnorm(0, 128, 128, gdn.GDN_F32, None, None, None, 1e-5, gdn.GDN_ACT_SILU, None,
                                 None) == gdn.GDN_OK


def test_prefill_workspace_size(lib):
    size = ctypes.c_uint64(123)
    chunky = dict(io_dtype=gdn.GDN_BF16, d_k=128, d_v=128, h_qk=16, h_v=32)
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**chunky)), 8, 33173, ctypes.byref(size)) == gdn.GDN_OK
    # the chunk table, then one record per (chunk, head) for ceil(T / 64) + N chunks.
    # 256 (sequence, head) units take the column-block state pass: the six lower
    # blocks of T diag(beta gam), T diag(beta) and M (1 KiB each), then gam and
    # exp(G_last - G) in a 1 KiB tail
    per_rec = 18 * 1024 + 1024
    bound = 33173 // 64 + 1 + 8
    assert size.value == 256 + (bound * 8 + 255) // 256 * 256 + bound * 32 * per_rec
    # one sequence of 32 heads (32 x 8 16-column tiles fill the 256 compute units
    # assumed without a device) takes the row-split pass and the full record:
    # operand fragments (W, diag(gam) Q: 16 each; Kt^T: 16; M: 6; T'': 6) of 1 KiB, gam_last
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**chunky)), 1, 4096, ctypes.byref(size)) == gdn.GDN_OK
    per_rec = (16 + 16 + 16 + 6 + 6) * 1024 + 256
    bound = 4096 // 64 + 1
    assert size.value == 256 + (bound * 8 + 255) // 256 * 256 + bound * 32 * per_rec
    # the gated and linear rules (no delta correction) always take the small record
    for rule in (2, 3):
        assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**chunky, rule=rule, beta=None)), 1, 4096,
                                              ctypes.byref(size)) == gdn.GDN_OK
        assert size.value == 256 + (bound * 8 + 255) // 256 * 256 + bound * 32 * (18 * 1024 + 1024), rule
    for kw in (dict(algorithm=gdn.GDN_ALGO_SERIAL), dict(io_dtype=gdn.GDN_F16), dict(d_k=96), dict(d_v=36),
               dict(decay_per_key=1), dict(state_window=2)):
        st = lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**{**chunky, **kw})), 8, 33173, ctypes.byref(size))
        assert st == gdn.GDN_OK and size.value == 0, kw
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**chunky)), 0, 0, ctypes.byref(size)) == gdn.GDN_OK
    assert size.value == 0
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**chunky)), -1, 0, ctypes.byref(size)) == INVALID
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**chunky)), 1, 1, None) == INVALID


def test_prefill_workspace_size_f32(lib):
    """The float32 chunked form (two passes only): a record of split W, scale diag(gam) Q and
    Kt^T fragments, M's six lower blocks (hi and lo, 1 KiB each), U in f32 and gam_last."""
    size = ctypes.c_uint64(123)

    def rec_bytes(d_k, d_v):
        b = (d_k // 32) * 8 * 1024 * 2 + (d_k // 16) * 4 * 1024 + 12 * 1024 + (d_v // 16) * 4 * 1024 + 256
        return (b + 255) // 256 * 256

    wide = dict(io_dtype=gdn.GDN_F32, d_k=256, d_v=256, h_qk=8, h_v=8)
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**wide)), 1, 32768, ctypes.byref(size)) == gdn.GDN_OK
    bound = (32768 + 63) // 64 + 1
    assert rec_bytes(256, 256) == 268 * 1024 + 256
    assert size.value == 256 + (bound * 8 + 255) // 256 * 256 + bound * 8 * rec_bytes(256, 256)
    # d_k = 128: AUTO and CHUNKED alike
    d128 = dict(wide, d_k=128, d_v=48)
    bound = (1000 + 63) // 64 + 3
    for algo in (gdn.GDN_ALGO_AUTO, gdn.GDN_ALGO_CHUNKED):
        assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**d128, algorithm=algo)), 3, 1000,
                                              ctypes.byref(size)) == gdn.GDN_OK
        assert size.value == 256 + (bound * 8 + 255) // 256 * 256 + bound * 8 * rec_bytes(128, 48)
    # every rule takes the same record (the gated and linear rules write W = 0 and U = V)
    assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**wide)), 1, 32768, ctypes.byref(size)) == gdn.GDN_OK
    full = size.value
    for rule in (1, 2, 3):
        assert lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**wide, rule=rule)), 1, 32768,
                                              ctypes.byref(size)) == gdn.GDN_OK
        assert size.value == full, rule
    # geometries the float32 form does not serve
    for kw in (dict(d_k=64), dict(d_v=24), dict(decay_per_key=1), dict(state_window=1),
               dict(algorithm=gdn.GDN_ALGO_SERIAL)):
        st = lib.gdn_prefill_workspace_size(ctypes.byref(_prob(**{**wide, **kw})), 1, 32768, ctypes.byref(size))
        assert st == gdn.GDN_OK and size.value == 0, kw


def test_prefill_chunked_f32_without_workspace(lib):
    prob = _prob(io_dtype=gdn.GDN_F32, d_k=256, d_v=32, h_qk=1, h_v=1, algorithm=gdn.GDN_ALGO_CHUNKED)
    st = _prefill(lib, prob, n=1, cu_host=[0, 8], T=8)
    assert st == gdn.GDN_ERR_UNSUPPORTED and "workspace" in gdn.last_error()
    prob = _prob(io_dtype=gdn.GDN_F32, d_k=256, d_v=32, h_qk=1, h_v=1, algorithm=gdn.GDN_ALGO_CHUNKED,
                 workspace=FAKE + 0x900000, workspace_bytes=1024)
    st = _prefill(lib, prob, n=1, cu_host=[0, 8], T=8)
    assert st == gdn.GDN_ERR_UNSUPPORTED and "too small a workspace" in gdn.last_error()


def test_prefill_workspace_misaligned(lib):
    st = _prefill(lib, _prob(workspace=FAKE + 0x90008, workspace_bytes=1 << 20))
    assert st == INVALID and "workspace" in gdn.last_error()


def test_prefill_query_plan(lib):
    """The host-only plan query: the form AUTO resolves to at each workload's
    geometry (on a 256-compute-unit device, which is also the answer when no
    device can be asked), and the refusal of an unserved explicit request."""
    ws = 1 << 40
    q = gdn.prefill_query_plan
    bf16, f32 = torch.bfloat16, torch.float32
    p = q(2, 2, 16, 16, f32, 1, 64)
    assert p["form"] == "serial" and p["kernels"] == "scan_kernel"
    p = q(16, 32, 128, 128, bf16, 1, 4096, raw_gates=True, workspace_bytes=ws)
    assert p["form"] == "chunked_two_pass" and p["kernels"].endswith("chunk_rows_kernel")
    assert p["state_workgroups"] == 32 * 8
    p = q(16, 32, 128, 128, bf16, 8, 33173, workspace_bytes=ws)
    assert p["form"] == "chunked_two_pass" and p["kernels"].endswith("chunk_state_kernel")
    assert "chunk_trec_kernel" in p["kernels"]  # the small record's preparation pass
    assert p["columns_per_block"] == 64
    p = q(16, 32, 128, 128, bf16, 8, 33173)
    assert p["form"] == "chunked_one_pass" and p["kernels"] == "chunk_kernel"
    p = q(8, 8, 256, 256, f32, 1, 32768, workspace_bytes=ws)
    assert p["form"] == "chunked_f32" and p["kernels"].split(" + ")[-1] == "wide_state_kernel"
    p = q(8, 8, 256, 256, f32, 1, 32768)
    assert p["form"] == "serial" and p["kernels"] == "scan_plain_kernel"
    # sequences averaging under 64 tokens stay serial under AUTO
    assert q(16, 32, 128, 128, bf16, 8, 8 * 63)["form"] == "serial"
    assert q(16, 32, 128, 128, bf16, 8, 8 * 63, algorithm="chunked")["form"] == "chunked_one_pass"
    assert q(16, 32, 128, 128, bf16, 8, 33173, algorithm="serial")["form"] == "serial"
    assert q(16, 32, 128, 128, bf16, 0, 0)["form"] == "none"
    with pytest.raises(gdn.GdnError, match="chunked algorithm needs"):
        q(2, 2, 16, 16, f32, 1, 64, algorithm="chunked")
    assert lib.gdn_prefill_query_plan(None, 1, 8, None) == INVALID


def test_conv_slots_validation(lib):
    """The pool forms of the convolution check their slots like the recurrence's."""
    prob = gdn.gdn_conv_problem(64, 4, 1, gdn.GDN_BF16, gdn.GDN_ACT_SILU, ctypes.c_void_p(FAKE), None)
    vp = ctypes.c_void_p
    host = (ctypes.c_int32 * 2)(3, 3)
    cu = (ctypes.c_int32 * 3)(0, 4, 8)
    st = lib.gdn_causal_conv_slots(ctypes.byref(prob), 2, vp(FAKE + 0x1000), cu, 8, vp(FAKE + 0x10000),
                                   vp(FAKE + 0x20000), 5, vp(FAKE + 0x3000), host, vp(FAKE + 0x40000), None)
    assert st == INVALID and "slot 3" in gdn.last_error()
    st = lib.gdn_causal_conv_step_slots(ctypes.byref(prob), 2, vp(FAKE + 0x10000), vp(FAKE + 0x20000), 5,
                                        vp(FAKE + 0x3000), host, vp(FAKE + 0x40000), None)
    assert st == INVALID and "slot 3" in gdn.last_error()
    st = lib.gdn_causal_conv_step_slots(ctypes.byref(prob), 2, vp(FAKE + 0x10000), vp(FAKE + 0x20000), -1,
                                        vp(FAKE + 0x3000), None, vp(FAKE + 0x40000), None)
    assert st == INVALID and "num_slots" in gdn.last_error()
    st = lib.gdn_causal_conv_step_slots(ctypes.byref(prob), 2, vp(FAKE + 0x10000), vp(FAKE + 0x20000), 5,
                                        None, None, vp(FAKE + 0x40000), None)
    assert st == INVALID and "slots is NULL" in gdn.last_error()


def test_output_norm_validation(lib):
    """The gated RMSNorm epilogue's arguments are checked before anything runs."""
    base = dict(io_dtype=gdn.GDN_BF16, d_k=128, d_v=128, h_qk=1, h_v=2, norm_gate=FAKE + 0x80000,
                norm_scale=FAKE + 0x90000, norm_eps=1e-5, norm_activation=gdn.GDN_ACT_SILU)
    for kw, needle in ((dict(norm_scale=None), "norm_scale"), (dict(norm_gate=FAKE + 0x80008), "16-byte"),
                       (dict(norm_eps=-1.0), "norm_eps"), (dict(norm_activation=gdn.GDN_ACT_NONE), "norm_activation"),
                       (dict(norm_eps=float("inf")), "norm_eps")):
        st = _prefill(lib, _prob(**{**base, **kw}), n=1, cu_host=[0, 8], T=8)
        assert st == INVALID and needle in gdn.last_error(), (kw, gdn.last_error())
    # the gate may not overlap out (out at FAKE + 0x40000, 8 x 2 x 128 bf16)
    st = _prefill(lib, _prob(**{**base, "norm_gate": FAKE + 0x40000}), n=1, cu_host=[0, 8], T=8)
    assert st == INVALID and "norm_gate" in gdn.last_error()
    p = gdn.prefill_query_plan(16, 32, 128, 256, torch.bfloat16, 8, 33173, workspace_bytes=1 << 40, norm=True)
    assert p["norm"] == "separate pass" and p["kernels"].endswith("rmsnorm_kernel")
    p = gdn.prefill_query_plan(16, 32, 128, 128, torch.bfloat16, 8, 33173, workspace_bytes=1 << 40, norm=True)
    assert p["norm"] == "separate pass" and p["columns_per_block"] == 64
    # from 512 (sequence, head) units the state pass runs 128-column blocks anyway, and fuses the norm
    p = gdn.prefill_query_plan(16, 32, 128, 128, torch.bfloat16, 16, 32768, workspace_bytes=1 << 40, norm=True)
    assert p["norm"] == "fused" and p["columns_per_block"] == 128


def test_decode_conv_validation(lib):
    """The decode step with its conv prologue checks the conv's geometry
    against the problem's, and its buffers, before anything runs."""
    vp = ctypes.c_void_p
    base = dict(io_dtype=gdn.GDN_BF16, h_qk=1, h_v=2, d_k=128, d_v=128)
    C = 2 * 128 + 2 * 128

    def call(prob_kw=None, C=C, K=4, dil=1, dtype=gdn.GDN_BF16, B=2, x=FAKE + 0x100000, cs=FAKE + 0x200000,
             cs_out=FAKE + 0x300000, state=FAKE + 0x400000, out=FAKE + 0x500000):
        conv = gdn.gdn_conv_problem(C, K, dil, dtype, gdn.GDN_ACT_SILU, vp(FAKE + 0x600000), None)
        prob = _prob(**{**base, **(prob_kw or {})})
        return lib.gdn_decode_step_conv(ctypes.byref(prob), ctypes.byref(conv), B, vp(x) if x else None,
                                        vp(cs) if cs else None, vp(cs_out) if cs_out else None,
                                        vp(state) if state else None, vp(out) if out else None, None)

    for kw, status, needle in (
            (dict(C=C + 1), INVALID, "channels"),
            (dict(dtype=gdn.GDN_F32), INVALID, "io_dtype"),
            (dict(cs_out=FAKE + 0x200000), INVALID, "in place"),
            (dict(cs_out=None), INVALID, "required"),
            (dict(x=FAKE + 0x100002), INVALID, "16-byte"),
            (dict(out=FAKE + 0x100000), INVALID, "overlap"),
            (dict(state=None), INVALID, "required"),
            (dict(B=-1), INVALID, "negative"),
            (dict(dil=2), UNSUPPORTED, "dilation"),
            (dict(K=5), UNSUPPORTED, "kernel_size"),
            (dict(prob_kw=dict(d_k=100), C=2 * 100 + 2 * 128), UNSUPPORTED, "d_k"),
            (dict(prob_kw=dict(d_v=96), C=2 * 128 + 2 * 96), UNSUPPORTED, "multiple"),
            (dict(prob_kw=dict(decay_per_key=1)), UNSUPPORTED, "per-key")):
        st = call(**kw)
        assert st == status and needle in gdn.last_error(), (kw, st, gdn.last_error())
    # nothing to do: OK without a launch; K = 1 carries nothing, so no conv states are needed
    assert call(B=0, x=None, cs=None, cs_out=None, state=None, out=None) == gdn.GDN_OK
    assert gdn.last_error() == ""
