"""The oracle's float32 build (the timed CPU baseline) held to the double build
and to the invariants the delta rule fixes, on the CPU.

Same source, -DGDNREF_ACC=float, -O3 -march=native: only the working
precision of the state and the accumulations differs, so it must agree with
the reference build to float32 rounding (about 1e-6 relative per step here),
and reproduce exactly what involves no rounding at all.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_serial_amd import synth


@pytest.fixture(scope="module")
def f32():
    return oracle.float32_baseline()


@pytest.fixture(scope="module")
def f64():
    return oracle.default()


def test_working_precision(f32, f64):
    assert f32.acc_bytes() == 4 and f64.acc_bytes() == 8


def _case(shape_name, seqlens, seed, **over):
    import dataclasses
    shape = dataclasses.replace(synth.BY_NAME[shape_name], **over)
    inp = synth.generate(shape, seqlens=seqlens, seed=seed)
    return inp


@pytest.mark.parametrize("over,lens", [
    (dict(h_qk=2, h_v=4, d_k=64, d_v=48, io_dtype=torch.float32, init_state=True), [200, 0, 37]),
    (dict(h_qk=1, h_v=1, d_k=256, d_v=256, io_dtype=torch.float32), [120]),
    (dict(h_qk=16, h_v=32, d_k=128, d_v=128, io_dtype=torch.bfloat16, init_state=True), [64, 9]),
], ids=["d64_packed", "d256", "d128_bf16_inputs"])
def test_matches_double_build(f32, f64, over, lens):
    inp = _case("varlen_prefill_8seq", lens, 31, **over)
    g, beta = f64.gates(inp.a, inp.b, inp.A_log, inp.dt_bias)
    args = (inp.q, inp.k, inp.v, g, beta, inp.cu_seqlens.numpy(),
            None if inp.initial_state is None else inp.initial_state)
    o32, s32 = f32.prefill(*args)
    o64, s64 = f64.prefill(*args)
    eo = np.max(np.abs(o32 - o64) / (1 + np.abs(o64)))
    es = np.max(np.abs(s32 - s64) / (1 + np.abs(s64)))
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)
    # and it is float32 arithmetic: the results are float32 values, not doubles
    assert np.array_equal(o32, o32.astype(np.float32).astype(np.float64))
    assert np.array_equal(s32, s32.astype(np.float32).astype(np.float64))


def test_frozen_state_is_exact(f32):
    """beta = 0 and g = 0: the state never changes, and o = scale S0^T q."""
    rng = np.random.default_rng(5)
    T, h, dk, dv = 20, 2, 32, 16
    q = rng.standard_normal((T, h, dk)).astype(np.float32)
    k = rng.standard_normal((T, h, dk)).astype(np.float32)
    v = rng.standard_normal((T, h, dv)).astype(np.float32)
    s0 = rng.standard_normal((1, h, dk, dv)).astype(np.float32)
    z = np.zeros((T, h))
    o, s = f32.prefill(q, k, v, z, z, [0, T], s0)
    assert np.array_equal(s, s0.astype(np.float64))
    ref = np.einsum("hij,thi->thj", s0[0].astype(np.float64), q.astype(np.float64)) / np.sqrt(dk)
    assert np.max(np.abs(o - ref)) <= 1e-5


def test_memorisation(f32):
    """beta = 1 with a unit key: S^T k = v after the update (to float32 rounding)."""
    rng = np.random.default_rng(6)
    T, dk, dv = 12, 64, 32
    k = rng.standard_normal((T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, dv))
    g = np.full((T, 1), -0.3)
    beta = np.ones((T, 1))
    for t in range(1, T + 1):
        _, s = f32.prefill(k[:t], k[:t], v[:t], g[:t], beta[:t], [0, t])
        r = s[0, 0].T @ k[t - 1, 0]
        assert np.max(np.abs(r - v[t - 1, 0])) <= 1e-5


def test_reset(f32):
    """g = -inf forgets everything before: S = beta k v^T."""
    rng = np.random.default_rng(7)
    T, dk, dv = 6, 16, 8
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((T, 1, dv)).astype(np.float32).astype(np.float64)
    g = np.full((T, 1), -0.5)
    g[-1] = -np.inf
    beta = np.full((T, 1), 0.75)
    s0 = rng.standard_normal((1, 1, dk, dv))
    _, s = f32.prefill(q, k, v, g, beta, [0, T], s0)
    ref = 0.75 * np.outer(k[-1, 0], v[-1, 0])
    assert np.max(np.abs(s[0, 0] - ref)) <= 1e-6
