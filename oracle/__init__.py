"""Reference (test-infrastructure) implementation of the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  The arithmetic lives in ``gdn_oracle.c`` (plain C,
IEEE double); this module builds it with gcc and marshals numpy arrays into it
with ctypes.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  It imports nothing from the HIP library and
the HIP library imports nothing from it.

Sources are cited in ``gdn_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(HERE, "libgdn_oracle.so")

RULES = {"linear": 0, "gated": 1, "delta": 2, "gated_delta": 3}

# -ffp-contract=off keeps every multiply and add a separately rounded IEEE
# double operation, exactly as written in the C source.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source file into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-I", HERE, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``gdn_oracle.c`` into ``oracle/libgdn_oracle.so`` (and the
    float32 baseline build for this host, see ``build_f32``)."""
    if not force and os.path.exists(LIB_PATH) and os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC):
        return LIB_PATH
    out = compile_source(SRC, LIB_PATH)
    build_f32(force=force)
    return out


# The timed CPU baseline: the same source with a float32 working state,
# optimised for the host it runs on.  -march=native makes the library specific
# to the CPU that built it, so its file name carries a digest of that CPU's
# model and feature flags and it is rebuilt on any other host.
CFLAGS_F32 = ["-O3", "-march=native", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-DGDNREF_ACC=float",
              "-Wall", "-Wextra"]


def host_cpu() -> dict:
    """Model name and logical CPU count of this host (from /proc/cpuinfo)."""
    model, flags, n = "unknown", "", 0
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("processor"):
                    n += 1
                elif line.startswith("model name") and model == "unknown":
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("flags") and not flags:
                    flags = line.split(":", 1)[1].strip()
    except OSError:
        pass
    return {"model": model, "flags": flags, "logical_cpus": n or os.cpu_count() or 1}


def f32_lib_path() -> str:
    import hashlib
    cpu = host_cpu()
    tag = hashlib.sha256((cpu["model"] + "|" + cpu["flags"]).encode()).hexdigest()[:10]
    return os.path.join(HERE, f"libgdn_oracle_f32_{tag}.so")


def build_f32(force: bool = False) -> str:
    """Compile the float32 baseline build of ``gdn_oracle.c`` for this host."""
    path = f32_lib_path()
    if not force and os.path.exists(path) and os.path.getmtime(path) >= os.path.getmtime(SRC):
        return path
    tmp = path + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS_F32, "-I", HERE, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, path)
    return path


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """numpy front end over one compiled copy of the oracle."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.gdnref_sigmoid.argtypes = [f64]
        lib.gdnref_sigmoid.restype = f64
        lib.gdnref_softplus.argtypes = [f64]
        lib.gdnref_softplus.restype = f64
        lib.gdnref_gates.argtypes = [i64, i32, dp, dp, dp, dp, dp, dp]
        lib.gdnref_gates.restype = None
        lib.gdnref_prefill.argtypes = [i32, i32, i32, i32, i32, f64, i32, ip,
                                       dp, dp, dp, dp, dp, dp, dp, dp]
        lib.gdnref_prefill.restype = ctypes.c_int
        lib.gdnref_prefill_ex.argtypes = [i32, i32, i32, i32, i32, f64, i32, ip,
                                          dp, dp, dp, dp, dp, i32, i32, dp, dp, dp, i32, dp]
        lib.gdnref_prefill_ex.restype = ctypes.c_int
        lib.gdnref_decode_step.argtypes = [i32, i32, i32, i32, i32, f64, i32,
                                           dp, dp, dp, dp, dp, dp, dp]
        lib.gdnref_decode_step.restype = ctypes.c_int
        lib.gdnref_causal_conv.argtypes = [i32, i32, i32, i32, i32, ip, dp, dp, dp, dp, dp, dp]
        lib.gdnref_causal_conv.restype = ctypes.c_int
        lib.gdnref_causal_conv_slots.argtypes = [i32, i32, i32, i32, i32, ip, dp, dp, dp, dp, i32, ip, dp]
        lib.gdnref_causal_conv_slots.restype = ctypes.c_int
        lib.gdnref_gated_rmsnorm.argtypes = [i64, i32, i32, dp, dp, dp, f64, i32, dp]
        lib.gdnref_gated_rmsnorm.restype = ctypes.c_int
        lib.gdnref_max_threads.argtypes = []
        lib.gdnref_max_threads.restype = ctypes.c_int
        lib.gdnref_set_threads.argtypes = [i32]
        lib.gdnref_set_threads.restype = None
        lib.gdnref_acc_bytes.argtypes = []
        lib.gdnref_acc_bytes.restype = i32
        self.lib = lib
        self.path = lib_path

    def sigmoid(self, x: float) -> float:
        return self.lib.gdnref_sigmoid(float(x))

    def softplus(self, x: float) -> float:
        return self.lib.gdnref_softplus(float(x))

    def max_threads(self) -> int:
        return int(self.lib.gdnref_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.gdnref_set_threads(int(n))

    def acc_bytes(self) -> int:
        """8 for the reference (double) build, 4 for the float32 baseline build."""
        return int(self.lib.gdnref_acc_bytes())

    def gates(self, a, b, A_log, dt_bias):
        """(g, beta) = (-exp(A_log) softplus(a + dt_bias), sigmoid(b)), shaped like ``a``."""
        a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
        h_v = A_log.shape[-1]
        rows = a.size // h_v
        g = np.empty(a.shape, np.float64)
        beta = np.empty(b.shape, np.float64)
        self.lib.gdnref_gates(rows, h_v, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                              _ptr(g), _ptr(beta))
        return g, beta

    def prefill(self, q, k, v, g, beta, cu_seqlens, initial_state=None, *,
                rule="gated_delta", scale=0.0, want_out=True, decay_per_key=False,
                beta_shared=False, window=0):
        """Serial scan over packed sequences.

        q, k: [T, h_qk, d_k]; v: [T, h_v, d_v]; g: [T, h_v] ([T, h_v, d_k] with
        decay_per_key); beta: [T, h_v] ([T] with beta_shared) -- None when the
        rule does not use them; cu_seqlens: ints [N+1]; initial_state:
        [N, h_v, d_k, d_v] or None.  Returns (out [T, h_v, d_v], final
        [N, h_v, d_k, d_v]) as float64 arrays, plus the state history
        [N, window, h_v, d_k, d_v] when window > 0.
        """
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        s0 = _f64(initial_state)
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        T, h_qk, d_k = q.shape
        h_v, d_v = v.shape[1], v.shape[2]
        n = cu.size - 1
        out = np.empty((T, h_v, d_v), np.float64) if want_out else None
        fin = np.empty((n, h_v, d_k, d_v), np.float64)
        hist = np.empty((n, window, h_v, d_k, d_v), np.float64) if window > 0 else None
        rc = self.lib.gdnref_prefill_ex(RULES[rule], h_qk, h_v, d_k, d_v, float(scale), n,
                                        _ptr(cu, ctypes.c_int32), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(g), _ptr(beta), int(decay_per_key), int(beta_shared),
                                        _ptr(s0), _ptr(out), _ptr(fin), int(window), _ptr(hist))
        if rc != 0:
            raise ValueError("gdnref_prefill_ex rejected its arguments")
        return (out, fin, hist) if window > 0 else (out, fin)

    def decode_step(self, q, k, v, g, beta, state, *, rule="gated_delta", scale=0.0):
        """One token per sequence; ``state`` (float64 [B, h_v, d_k, d_v]) is updated in place."""
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous):
            raise TypeError("state must be a C-contiguous float64 numpy array")
        B, h_qk, d_k = q.shape
        h_v, d_v = v.shape[1], v.shape[2]
        out = np.empty((B, h_v, d_v), np.float64)
        rc = self.lib.gdnref_decode_step(RULES[rule], h_qk, h_v, d_k, d_v, float(scale), B,
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(state), _ptr(out))
        if rc != 0:
            raise ValueError("gdnref_decode_step rejected its arguments")
        return out


    def causal_conv(self, x, weight, cu_seqlens, bias=None, initial_state=None, *, dilation=1, silu=False):
        """Causal depthwise conv with carried state.  x: [T, C]; weight: [C, K];
        bias: [C] or None; cu_seqlens: ints [N+1]; initial_state: [N, carry, C]
        or None (zeros).  Returns (y [T, C], final_state [N, carry, C]) float64."""
        x, w, b, s0 = _f64(x), _f64(weight), _f64(bias), _f64(initial_state)
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        T, C = x.shape
        K = w.shape[1]
        carry = (K - 1) * dilation
        n = cu.size - 1
        y = np.empty((T, C), np.float64)
        fin = np.empty((n, carry, C), np.float64)
        rc = self.lib.gdnref_causal_conv(C, K, int(dilation), int(bool(silu)), n, _ptr(cu, ctypes.c_int32),
                                         _ptr(x), _ptr(w), _ptr(b), _ptr(s0), _ptr(y), _ptr(fin))
        if rc != 0:
            raise ValueError("gdnref_causal_conv rejected its arguments")
        return y, fin

    def causal_conv_slots(self, x, weight, cu_seqlens, pool, slots, bias=None, *, dilation=1, silu=False):
        """The convolution over a state pool.  pool: [num_slots, carry, C] (not
        modified); slots: ints [N].  Returns (y [T, C], the updated pool) float64."""
        x, w, b = _f64(x), _f64(weight), _f64(bias)
        pool = _f64(pool).copy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
        T, C = x.shape
        n = cu.size - 1
        y = np.empty((T, C), np.float64)
        rc = self.lib.gdnref_causal_conv_slots(C, w.shape[1], int(dilation), int(bool(silu)), n,
                                               _ptr(cu, ctypes.c_int32), _ptr(x), _ptr(w), _ptr(b), _ptr(pool),
                                               pool.shape[0], _ptr(sl, ctypes.c_int32), _ptr(y))
        if rc != 0:
            raise ValueError("gdnref_causal_conv_slots rejected its arguments")
        return y, pool

    def gated_rmsnorm(self, x, gate, scale, *, eps=1e-5, activation="silu"):
        """Gated RMSNorm over groups of len(scale) elements of the last axis of x."""
        x, g, s = _f64(x), _f64(gate), _f64(scale)
        width = x.shape[-1]
        rows = x.size // width if width else 0
        y = np.empty(x.shape, np.float64)
        act = {"silu": 1, "swish": 1, "sigmoid": 2}[activation]
        rc = self.lib.gdnref_gated_rmsnorm(rows, width, s.size, _ptr(x), _ptr(g), _ptr(s), float(eps), act, _ptr(y))
        if rc != 0:
            raise ValueError("gdnref_gated_rmsnorm rejected its arguments")
        return y


_default = None
_f32 = None


def default() -> Oracle:
    """The oracle built from ``gdn_oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def float32_baseline() -> Oracle:
    """The float32 baseline build for this host (compiled on first use)."""
    global _f32
    if _f32 is None:
        _f32 = Oracle(build_f32())
    return _f32
