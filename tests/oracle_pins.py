"""Pins of the oracle to facts other than itself.

Every function here takes an ``oracle.Oracle`` instance and raises
``AssertionError`` when the oracle disagrees with:
  * a brute-force unrolled matrix form in long double (shares no code with the
    scan: it multiplies the per-token transition matrices out explicitly),
  * invariants the delta rule fixes, closed forms and special cases,
  * library routines (numpy / scipy / torch) for the gate functions, the
    depthwise convolution and the RMS normalisation,
  * the values printed in the pages' one worked example (tests/golden/).

``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires each copy to fail at least one.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LD = np.longdouble


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, *, T_list=(5, 0, 7), h_qk=2, h_v=4, d_k=5, d_v=3, init=True,
                g_scale=1.0, unit_keys=True):
    """Small random packed problem (float64)."""
    rng = np.random.default_rng(seed)
    T = sum(T_list)
    cu = np.concatenate([[0], np.cumsum(T_list)]).astype(np.int32)
    q = rng.standard_normal((T, h_qk, d_k))
    k = rng.standard_normal((T, h_qk, d_k))
    if unit_keys:
        q, k = _unit_rows(q), _unit_rows(k)
    v = rng.standard_normal((T, h_v, d_v))
    g = -np.abs(rng.standard_normal((T, h_v))) * g_scale
    beta = rng.uniform(0.05, 0.95, (T, h_v))
    s0 = rng.standard_normal((len(T_list), h_v, d_k, d_v)) * 0.3 if init else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu=cu, s0=s0)


def brute_force(q, k, v, g, beta, cu, s0, *, rule="gated_delta", scale=0.0, decay_per_key=False,
                beta_shared=False):
    """Unrolled matrix form, long double.

    Token t of a sequence maps the state by S -> A_t S + B_t with
      A_t = (I - beta_t k_t k_t^T) D_t,  B_t = beta_t k_t v_t^T   (delta rules)
      A_t = D_t,                         B_t = k_t v_t^T          (plain rules)
    with the decay D_t = exp(g_t) I (diag(exp(g_t)) for per-key-dim decay) for
    gated rules and D_t = I otherwise.  The state after
    token t is formed from scratch as
      S_t = (A_t ... A_1) S_0 + sum_s (A_t ... A_{s+1}) B_s
    and read out as out_t = scale S_t^T q_t.  Query/key heads are widened to
    the value heads by repeating each one over consecutive value heads.
    """
    decays = rule in ("gated", "gated_delta")
    deltas = rule in ("delta", "gated_delta")
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    ratio = h_v // h_qk
    qr = np.repeat(np.asarray(q, LD), ratio, axis=1)
    kr = np.repeat(np.asarray(k, LD), ratio, axis=1)
    vv = np.asarray(v, LD)
    sc = LD(1) / np.sqrt(LD(d_k)) if scale == 0 else LD(scale)
    n = len(cu) - 1
    out = np.zeros((T, h_v, d_v), LD)
    fin = np.zeros((n, h_v, d_k, d_v), LD)
    eye = np.eye(d_k, dtype=LD)
    for s in range(n):
        toks = list(range(int(cu[s]), int(cu[s + 1])))
        for h in range(h_v):
            S0 = np.zeros((d_k, d_v), LD) if s0 is None else np.asarray(s0[s, h], LD)
            A, B = [], []
            for t in toks:
                kt = kr[t, h][:, None]
                if not decays:
                    Dg = eye
                elif decay_per_key:
                    Dg = np.diag(np.exp(np.asarray(g[t, h], LD)))   # row i scaled by exp(g_i)
                else:
                    Dg = np.exp(LD(g[t, h])) * eye
                if deltas:
                    bt = LD(beta[t] if beta_shared else beta[t, h])
                    A.append((eye - bt * (kt @ kt.T)) @ Dg)
                    B.append(bt * (kt @ vv[t, h][None, :]))
                else:
                    A.append(Dg)
                    B.append(kt @ vv[t, h][None, :])
            St = S0
            for idx, t in enumerate(toks):
                M = eye.copy()
                acc = np.zeros((d_k, d_v), LD)
                for j in range(idx, -1, -1):
                    acc = acc + M @ B[j]
                    M = M @ A[j]
                St = M @ S0 + acc
                out[t, h] = sc * (St.T @ qr[t, h])
            fin[s, h] = St
    return out, fin


def _close(a, b, tol, what):
    a = np.asarray(a, LD)
    b = np.asarray(b, LD)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if a.size == 0:
        return
    err = float(np.max(np.abs(a - b) / (1 + np.abs(b))))
    assert err <= tol, f"{what}: max |a-b|/(1+|b|) = {err:.3e} > {tol:.1e}"


def _bitwise(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.array_equal(a, b), f"{what}: not bitwise equal (max diff {np.max(np.abs(a - b)) if a.size else 0})"


# ---------------------------------------------------------------- brute force
def pin_brute_force(orc):
    cases = [
        dict(seed=1, rule="gated_delta", scale=0.0),
        dict(seed=2, rule="gated_delta", scale=0.75, d_k=3, d_v=6, h_qk=1, h_v=3),
        dict(seed=3, rule="delta", scale=0.0, T_list=(12,), h_qk=2, h_v=2),
        dict(seed=4, rule="gated", scale=1.5, init=False),
        dict(seed=5, rule="linear", scale=0.0, T_list=(4, 6)),
        dict(seed=6, rule="gated_delta", scale=0.0, unit_keys=False, g_scale=3.0, T_list=(9, 1)),
        dict(seed=7, rule="gated_delta", scale=0.0, d_k=6, d_v=6, h_qk=1, h_v=4, T_list=(3, 2, 4)),
    ]
    for c in cases:
        c = dict(c)
        rule, scale = c.pop("rule"), c.pop("scale")
        x = random_case(**c)
        uses_g = rule in ("gated", "gated_delta")
        uses_b = rule in ("delta", "gated_delta")
        o, f = orc.prefill(x["q"], x["k"], x["v"], x["g"] if uses_g else None,
                           x["beta"] if uses_b else None, x["cu"], x["s0"], rule=rule, scale=scale)
        bo, bf = brute_force(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"],
                             rule=rule, scale=scale)
        _close(o, bo, 1e-12, f"brute force out (seed {c['seed']}, {rule})")
        _close(f, bf, 1e-12, f"brute force state (seed {c['seed']}, {rule})")


# ---------------------------------------------------------------- invariants
def pin_delta_rule_memorises(orc):
    """beta = 1 and a unit key: the updated state retrieves v exactly, S^T k = v.
    With q = k and scale 1 the readout is that retrieval."""
    x = random_case(11, T_list=(8,), h_qk=2, h_v=2, d_k=6, d_v=4)
    beta = np.ones_like(x["beta"])
    o, _ = orc.prefill(x["k"], x["k"], x["v"], x["g"], beta, x["cu"], x["s0"], scale=1.0)
    _close(o, x["v"], 1e-12, "S^T k = v after a beta = 1 update")


def pin_frozen_state(orc):
    """beta = 0 and g = 0 leave the state untouched; the readout is scale S0^T q."""
    x = random_case(12, T_list=(6, 3), h_qk=1, h_v=2, d_k=4, d_v=5)
    z = np.zeros_like(x["g"])
    o, f = orc.prefill(x["q"], x["k"], x["v"], z, z, x["cu"], x["s0"], scale=0.5)
    _bitwise(f, x["s0"], "frozen final state")
    for s in range(2):
        for t in range(int(x["cu"][s]), int(x["cu"][s + 1])):
            for h in range(2):
                _close(o[t, h], 0.5 * (x["s0"][s, h].T @ x["q"][t, 0]), 1e-14, "frozen readout")


def pin_reset(orc):
    """g = -inf zeroes the carried state: after token t the state is exactly
    beta_t k_t v_t^T, whatever the initial state was."""
    x = random_case(13, T_list=(4,), h_qk=1, h_v=1, d_k=4, d_v=3)
    g = np.full_like(x["g"], -np.inf)
    _, f1 = orc.prefill(x["q"], x["k"], x["v"], g, x["beta"], x["cu"], x["s0"])
    _, f2 = orc.prefill(x["q"], x["k"], x["v"], g, x["beta"], x["cu"], None)
    _bitwise(f1, f2, "reset independent of the initial state")
    t = 3
    expect = x["k"][t, 0][:, None] * (x["beta"][t, 0] * x["v"][t, 0])[None, :]
    _bitwise(f1[0, 0], expect, "reset state = beta k v^T")


def pin_power_of_two_scaling(orc):
    """The map is linear in (v, S0): scaling both by 2^m scales (out, S) by 2^m exactly."""
    x = random_case(14)
    o1, f1 = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"])
    o2, f2 = orc.prefill(x["q"], x["k"], x["v"] * 8.0, x["g"], x["beta"], x["cu"], x["s0"] * 8.0)
    _bitwise(o2, o1 * 8.0, "out scaling")
    _bitwise(f2, f1 * 8.0, "state scaling")


def pin_packing_invariance(orc):
    """Packed sequences give exactly what each sequence gives run alone."""
    x = random_case(15, T_list=(5, 0, 7, 2))
    o, f = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"])
    cu = x["cu"]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        oo, ff = orc.prefill(x["q"][a:b], x["k"][a:b], x["v"][a:b], x["g"][a:b], x["beta"][a:b],
                             [0, b - a], x["s0"][s:s + 1])
        _bitwise(o[a:b], oo, f"packed out seq {s}")
        _bitwise(f[s:s + 1], ff, f"packed state seq {s}")


def pin_continuation(orc):
    """prefill(T1) then prefill(T2) from its final state = prefill(T1 + T2);
    T decode steps = prefill(T)."""
    x = random_case(16, T_list=(9,), h_qk=2, h_v=4, d_k=5, d_v=3)
    q, k, v, g, b = x["q"], x["k"], x["v"], x["g"], x["beta"]
    o, f = orc.prefill(q, k, v, g, b, [0, 9], x["s0"])
    o1, f1 = orc.prefill(q[:4], k[:4], v[:4], g[:4], b[:4], [0, 4], x["s0"])
    o2, f2 = orc.prefill(q[4:], k[4:], v[4:], g[4:], b[4:], [0, 5], f1)
    _bitwise(np.concatenate([o1, o2]), o, "continued out")
    _bitwise(f2, f, "continued state")
    st = np.array(x["s0"], np.float64)
    outs = []
    for t in range(9):
        outs.append(orc.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], st))
    _bitwise(np.concatenate(outs), o, "decode steps out")
    _bitwise(st, f, "decode steps state")


def pin_gqa_repeat(orc):
    """h_qk < h_v equals the run with each q/k head repeated over its
    consecutive value heads."""
    x = random_case(17, T_list=(6, 4), h_qk=2, h_v=6, d_k=4, d_v=3)
    o, f = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"])
    qr = np.repeat(x["q"], 3, axis=1)
    kr = np.repeat(x["k"], 3, axis=1)
    o2, f2 = orc.prefill(qr, kr, x["v"], x["g"], x["beta"], x["cu"], x["s0"])
    _bitwise(o, o2, "GQA out")
    _bitwise(f, f2, "GQA state")


def pin_empty(orc):
    """No tokens: the final state is the initial state (zeros without one)."""
    x = random_case(18, T_list=(0, 0), h_qk=1, h_v=2, d_k=3, d_v=2)
    o, f = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"])
    assert o.shape == (0, 2, 2)
    _bitwise(f, x["s0"], "empty sequences keep their state")
    _, f0 = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], None)
    _bitwise(f0, np.zeros_like(f0), "empty sequences without a state")


# ---------------------------------------------------------------- closed forms
def pin_scalar_closed_form(orc):
    """d_k = d_v = 1: s_t = alpha_t (1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t,
    out_t = scale q_t s_t."""
    rng = np.random.default_rng(19)
    T = 20
    q = rng.standard_normal((T, 1, 1))
    k = rng.standard_normal((T, 1, 1))
    v = rng.standard_normal((T, 1, 1))
    g = -rng.uniform(0, 2, (T, 1))
    b = rng.uniform(0, 1, (T, 1))
    s0 = np.array([[[[0.7]]]])
    o, f = orc.prefill(q, k, v, g, b, [0, T], s0, scale=1.3)
    s = 0.7
    for t in range(T):
        kk = k[t, 0, 0]
        s = math.exp(g[t, 0]) * (1 - b[t, 0] * kk * kk) * s + b[t, 0] * kk * v[t, 0, 0]
        assert abs(o[t, 0, 0] - 1.3 * q[t, 0, 0] * s) <= 1e-13 * (1 + abs(s)), f"scalar out t={t}"
    assert abs(f[0, 0, 0, 0] - s) <= 1e-13 * (1 + abs(s)), "scalar final state"


def pin_orthonormal_keys(orc):
    """With beta = 1, g = 0 and keys e_1..e_d the state becomes sum_i e_i v_i^T;
    a later token with key 0 and query e_i reads scale v_i back exactly."""
    d, dv = 4, 3
    rng = np.random.default_rng(20)
    T = 2 * d
    q = np.zeros((T, 1, d))
    k = np.zeros((T, 1, d))
    v = rng.standard_normal((T, 1, dv))
    for i in range(d):
        k[i, 0, i] = 1.0
        q[d + i, 0, i] = 1.0
    o, f = orc.prefill(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), [0, T], None, scale=0.5)
    for i in range(d):
        _bitwise(o[d + i, 0], 0.5 * v[i, 0], f"orthonormal read {i}")
        _bitwise(f[0, 0, i], v[i, 0], f"orthonormal row {i}")


def pin_gates_library(orc):
    """Gate prologue against library routines and spot values."""
    rng = np.random.default_rng(21)
    a = np.concatenate([rng.standard_normal((64, 4)) * 3, [[40.0, -40.0, 700.0, -700.0]]])
    b = np.concatenate([rng.standard_normal((64, 4)) * 3, [[800.0, -800.0, 0.0, 30.0]]])
    A_log = rng.uniform(0, 1, 4)
    dt = rng.uniform(-1, 1, 4)
    g, beta = orc.gates(a, b, A_log, dt)
    g_lib = -np.exp(A_log) * np.logaddexp(0.0, a + dt)
    b_lib = scipy.special.expit(b)
    _close(g, g_lib, 1e-14, "g vs -exp(A_log) logaddexp(0, a + dt_bias)")
    assert np.all(np.abs(beta - b_lib) <= 1e-15 * np.maximum(b_lib, 1e-300) + 1e-300), "beta vs expit"
    # spot values
    g0, b0 = orc.gates(np.array([[0.25]]), np.array([[0.0]]), np.array([0.0]), np.array([-0.25]))
    assert abs(g0[0, 0] + math.log(2.0)) <= 1e-16, "A_log = 0, a + dt_bias = 0 gives g = -ln 2"
    assert abs(math.exp(g0[0, 0]) - 0.5) <= 1e-16, "... so alpha = 1/2"
    assert b0[0, 0] == 0.5, "b = 0 gives beta = 1/2"
    # asymptotes: softplus(x) -> x for large x, -> e^x for very negative x
    assert abs(orc.softplus(40.0) - 40.0) <= 1e-14
    assert abs(orc.softplus(-40.0) / math.exp(-40.0) - 1.0) <= 1e-14
    assert orc.softplus(800.0) == 800.0
    assert orc.sigmoid(-800.0) == 0.0 and orc.sigmoid(800.0) == 1.0


def pin_default_scale(orc):
    """scale == 0 means 1/sqrt(d_k), with d_k != d_v."""
    x = random_case(22, T_list=(5,), h_qk=1, h_v=1, d_k=9, d_v=2)
    o0, _ = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"], scale=0.0)
    o1, _ = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"], scale=1.0)
    _close(o0, o1 / 3.0, 1e-15, "default scale 1/sqrt(9)")


# ---------------------------------------------------------------- printed values
def pin_page_worked_example(orc):
    """The pages' one worked example (tests/golden/p1_wide_bf16_linear_state.json):
    rule `linear`, q = k = e0, v = 1/256, S0[0,0] = 1, scale 1.  The f32 output
    after token t is 1 + (t+1)/256 and the bf16 state after 1, 2, 3 tokens is
    1.0, 1.0078125, 1.015625 (round to nearest even of a state carried exactly)."""
    with open(os.path.join(GOLDEN, "p1_wide_bf16_linear_state.json")) as fh:
        fx = json.load(fh)
    for d_k in fx["d_k_cases"]:
        for T in (1, 2, 3):
            q = np.zeros((T, 1, d_k))
            q[:, 0, 0] = 1.0
            v = np.full((T, 1, 1), fx["value"])
            s0 = np.zeros((1, 1, d_k, 1))
            s0[0, 0, 0, 0] = fx["initial_state_row0"]
            o, f = orc.prefill(q, q, v, None, None, [0, T], s0, rule="linear", scale=fx["scale"])
            out32 = torch.from_numpy(o[:, 0, 0]).to(torch.float32).double().numpy()
            _bitwise(out32, np.array(fx["expected_output_T3"][:T]), f"page example out d_k={d_k} T={T}")
            st = torch.from_numpy(f[0, 0, :, 0]).to(torch.bfloat16).double().numpy()
            assert st[0] == fx["expected_state_bf16_after_T_steps"][T - 1], f"page example state T={T}"
            assert np.all(st[1:] == fx["expected_state_other_rows"])


def pin_rounding_tie(orc):
    """Delta-rule form of the same rounding question: q = k = e0, g = 0,
    beta = 1/2, S0 = 1, v = 1.0078125 (a bf16 value), scale 1.  Exactly,
    out_1 = 1 + 2^-8 (a bf16 tie, to even: 1.0) and out_2 = 1.005859375
    (to bf16: 1.0078125)."""
    v = Fraction(1) + Fraction(1, 128)
    s = Fraction(1)
    exact = []
    for _ in range(2):
        s = s + Fraction(1, 2) * (v - s)
        exact.append(s)
    q = np.zeros((2, 1, 4))
    q[:, 0, 0] = 1.0
    o, _ = orc.prefill(q, q, np.full((2, 1, 1), float(v)), np.zeros((2, 1)),
                       np.full((2, 1), 0.5), [0, 2], np.eye(4, 1).reshape(1, 1, 4, 1), scale=1.0)
    assert [Fraction(x) for x in o[:, 0, 0]] == exact, "tie-case outputs exact"
    assert torch.tensor(o[:, 0, 0]).to(torch.bfloat16).tolist() == [1.0, 1.0078125]


# ---------------------------------------------------------------- variants
def pin_variants_brute_force(orc):
    """Per-key-dim decay, shared beta and every rule against the unrolled form."""
    rng = np.random.default_rng(31)
    for seed, rule, per_key, shared in [(32, "gated_delta", True, False), (33, "gated_delta", False, True),
                                        (34, "gated", True, False), (35, "delta", False, True),
                                        (36, "gated_delta", True, True)]:
        x = random_case(seed, T_list=(6, 0, 5), h_qk=1, h_v=3, d_k=4, d_v=3)
        T = x["q"].shape[0]
        g = -np.abs(rng.standard_normal((T, 3, 4))) if per_key else x["g"]
        beta = rng.uniform(0.05, 0.95, T) if shared else x["beta"]
        uses_g = rule in ("gated", "gated_delta")
        uses_b = rule in ("delta", "gated_delta")
        o, f = orc.prefill(x["q"], x["k"], x["v"], g if uses_g else None, beta if uses_b else None, x["cu"],
                           x["s0"], rule=rule, decay_per_key=per_key, beta_shared=shared)
        bo, bf = brute_force(x["q"], x["k"], x["v"], g, beta, x["cu"], x["s0"], rule=rule,
                             decay_per_key=per_key, beta_shared=shared)
        _close(o, bo, 1e-12, f"variant out ({rule}, per_key={per_key}, shared={shared})")
        _close(f, bf, 1e-12, f"variant state ({rule}, per_key={per_key}, shared={shared})")


def pin_variant_reductions(orc):
    """Per-key-dim decay with equal rows is the per-head decay; a shared beta is a
    per-head beta broadcast over the heads (both bitwise)."""
    x = random_case(37, T_list=(7, 3), h_qk=2, h_v=4, d_k=5, d_v=3)
    g_rows = np.repeat(x["g"][:, :, None], 5, axis=2)
    o1, f1 = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"])
    o2, f2 = orc.prefill(x["q"], x["k"], x["v"], g_rows, x["beta"], x["cu"], x["s0"], decay_per_key=True)
    _bitwise(o1, o2, "per-key decay with equal rows")
    _bitwise(f1, f2, "per-key decay with equal rows (state)")
    b1 = x["beta"][:, 0].copy()
    o3, f3 = orc.prefill(x["q"], x["k"], x["v"], x["g"], b1, x["cu"], x["s0"], beta_shared=True)
    o4, f4 = orc.prefill(x["q"], x["k"], x["v"], x["g"], np.repeat(b1[:, None], 4, axis=1), x["cu"], x["s0"])
    _bitwise(o3, o4, "shared beta")
    _bitwise(f3, f4, "shared beta (state)")


def pin_state_history(orc):
    """History slot w holds the state after token L - W + w (the final state of
    the prefix that ends there); slots before the first token are zero."""
    x = random_case(38, T_list=(5, 2, 0), h_qk=1, h_v=2, d_k=3, d_v=4)
    W = 4
    _, fin, hist = orc.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"], x["s0"], window=W)
    cu = x["cu"]
    nonempty = [s for s in range(3) if cu[s + 1] > cu[s]]
    _bitwise(hist[nonempty, W - 1], fin[nonempty], "last history slot = final state")
    for s in range(3):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for w in range(W):
            end = L - W + w + 1  # tokens in the prefix
            if end <= 0:
                assert np.all(hist[s, w] == 0.0), f"seq {s} slot {w} should be zero"
                continue
            _, fp = orc.prefill(x["q"][a:a + end], x["k"][a:a + end], x["v"][a:a + end], x["g"][a:a + end],
                                x["beta"][a:a + end], [0, end], x["s0"][s:s + 1])
            _bitwise(hist[s, w], fp[0], f"seq {s} slot {w}")


def pin_page_worked_example_window(orc):
    """The worked example with a state window of 4: slots before the first
    step are zero, then the bf16 states 1.0, 1.0078125, 1.015625 in order
    (tests/golden/p1_wide_bf16_linear_state.json)."""
    with open(os.path.join(GOLDEN, "p1_wide_bf16_linear_state.json")) as fh:
        fx = json.load(fh)
    W = fx["window"]
    for d_k in fx["d_k_cases"]:
        for T in fx["T_cases"]:
            q = np.zeros((T, 1, d_k))
            q[:, 0, 0] = 1.0
            s0 = np.zeros((1, 1, d_k, 1))
            s0[0, 0, 0, 0] = fx["initial_state_row0"]
            _, _, hist = orc.prefill(q, q, np.full((T, 1, 1), fx["value"]), None, None, [0, T], s0,
                                     rule="linear", scale=fx["scale"], window=W)
            st = torch.from_numpy(hist[0, :, 0, :, 0]).to(torch.bfloat16).double().numpy()
            expect = [0.0] * (W - T) + fx["expected_state_bf16_after_T_steps"][:T]
            assert st[:, 0].tolist() == expect, f"window slots d_k={d_k} T={T}: {st[:, 0].tolist()} != {expect}"
            assert np.all(st[:, 1:] == 0.0)


# ---------------------------------------------------------------- causal conv with state
def _conv_case(seed, lens, C=5, K=4, init=True):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    b = rng.standard_normal(C)
    return rng, cu, x, w, b


def pin_conv_library(orc):
    """Each sequence against torch's depthwise conv1d (groups = channels, a
    cross-correlation) over [initial state ; x], plus torch's silu."""
    import torch.nn.functional as F
    for dil, silu, bias_on in [(1, False, True), (1, True, True), (2, True, False), (3, False, True)]:
        rng, cu, x, w, b = _conv_case(11 + dil, [9, 0, 3, 1])
        K, C = w.shape[1], w.shape[0]
        carry = (K - 1) * dil
        s0 = rng.standard_normal((len(cu) - 1, carry, C))
        y, fin = orc.causal_conv(x, w, cu, b if bias_on else None, s0, dilation=dil, silu=silu)
        for n in range(len(cu) - 1):
            xp = np.concatenate([s0[n], x[cu[n]:cu[n + 1]]], 0)           # [carry + L, C]
            assert np.array_equal(fin[n], xp[xp.shape[0] - carry:]), (dil, n)
            if cu[n + 1] == cu[n]:
                continue
            ref = F.conv1d(torch.from_numpy(xp.T[None].copy()), torch.from_numpy(w[:, None, :].copy()),
                           torch.from_numpy(b) if bias_on else None, dilation=dil, groups=C)[0].T
            if silu:
                ref = F.silu(ref)
            assert np.allclose(y[cu[n]:cu[n + 1]], ref.numpy(), rtol=1e-13, atol=1e-13), (dil, silu, n)


def pin_conv_continuation(orc):
    """conv(x1) then conv(x2) from its final state = conv(x1 x2), bitwise, for
    pieces shorter and longer than the carried window; token-by-token steps
    equal the whole sequence."""
    for dil in (1, 2):
        rng, _, x, w, b = _conv_case(21 + dil, [13])
        K, C = w.shape[1], w.shape[0]
        s0 = rng.standard_normal((1, (K - 1) * dil, C))
        y_all, f_all = orc.causal_conv(x, w, [0, 13], b, s0, dilation=dil, silu=True)
        for cut in (1, 2, 5, 12):
            y1, f1 = orc.causal_conv(x[:cut], w, [0, cut], b, s0, dilation=dil, silu=True)
            y2, f2 = orc.causal_conv(x[cut:], w, [0, 13 - cut], b, f1, dilation=dil, silu=True)
            assert np.array_equal(np.concatenate([y1, y2]), y_all) and np.array_equal(f2, f_all), (dil, cut)
        st, ys = s0, []
        for t in range(13):
            yt, st = orc.causal_conv(x[t:t + 1], w, [0, 1], b, st, dilation=dil, silu=True)
            ys.append(yt)
        assert np.array_equal(np.concatenate(ys), y_all) and np.array_equal(st, f_all), dil


def pin_conv_special_kernels(orc):
    """A kernel with only its last tap set passes x through; only its first
    tap delays x by the carried window; an empty sequence keeps its state;
    packed = each sequence alone."""
    rng, cu, x, w, b = _conv_case(31, [6, 0, 4])
    C, K = w.shape
    s0 = rng.standard_normal((3, K - 1, C))
    last = np.zeros((C, K)); last[:, K - 1] = 1.0
    y, fin = orc.causal_conv(x, last, cu, None, s0)
    assert np.array_equal(y, x)
    assert np.array_equal(fin[1], s0[1])                      # empty sequence
    first = np.zeros((C, K)); first[:, 0] = 1.0
    y, _ = orc.causal_conv(x, first, cu, None, s0)
    for n in range(3):
        xp = np.concatenate([s0[n], x[cu[n]:cu[n + 1]]], 0)
        assert np.array_equal(y[cu[n]:cu[n + 1]], xp[:cu[n + 1] - cu[n]])
    y_all, f_all = orc.causal_conv(x, w, cu, b, s0, silu=True)
    for n in range(3):
        yn, fn = orc.causal_conv(x[cu[n]:cu[n + 1]], w, [0, cu[n + 1] - cu[n]], b, s0[n:n + 1], silu=True)
        assert np.array_equal(yn, y_all[cu[n]:cu[n + 1]]) and np.array_equal(fn[0], f_all[n])
    y0, f0 = orc.causal_conv(x, w, cu, b, None)              # no initial state = zeros
    yz, fz = orc.causal_conv(x, w, cu, b, np.zeros_like(s0))
    assert np.array_equal(y0, yz) and np.array_equal(f0, fz)


def pin_conv_slots(orc):
    """The pool form: gathering the states at the slots (numpy indexing), the
    plain convolution (pinned above against torch), and scattering the new
    states back is exactly what the slot-pool conv gives, bitwise; rows no
    sequence names stay as they were; a padding slot (outside the pool) runs
    from zeros and writes nothing; identity slots equal the plain call."""
    rng, cu, x, w, b = _conv_case(51, [6, 0, 4, 3, 5])
    C, K = w.shape
    for dil in (1, 2):
        carry = (K - 1) * dil
        pool = rng.standard_normal((7, carry, C))
        for slots in ([4, 1, -1, 6, 0], [0, 1, 2, 3, 4], [6, 5, 7, 2, -3]):
            states = np.zeros((len(slots), carry, C))
            for n, sl in enumerate(slots):
                if 0 <= sl < 7:
                    states[n] = pool[sl]
            y_ref, f_ref = orc.causal_conv(x, w, cu, b, states, dilation=dil, silu=True)
            pool_ref = pool.copy()
            for n, sl in enumerate(slots):
                if 0 <= sl < 7:
                    pool_ref[sl] = f_ref[n]
            y, new_pool = orc.causal_conv_slots(x, w, cu, pool, slots, b, dilation=dil, silu=True)
            assert np.array_equal(y, y_ref) and np.array_equal(new_pool, pool_ref), (dil, slots)
        y_id, pool_id = orc.causal_conv_slots(x, w, cu, pool[:5], [0, 1, 2, 3, 4], b, dilation=dil, silu=True)
        y_pl, f_pl = orc.causal_conv(x, w, cu, b, pool[:5], dilation=dil, silu=True)
        assert np.array_equal(y_id, y_pl) and np.array_equal(pool_id, f_pl), dil


# ---------------------------------------------------------------- gated RMSNorm
def pin_rmsnorm_library(orc):
    """Against torch's rms_norm (with the scale as its weight) times torch's
    silu / sigmoid of the gate; a saturated sigmoid gate leaves rms_norm alone."""
    import torch.nn.functional as F
    rng = np.random.default_rng(41)
    C = 12
    x = rng.standard_normal((7, 3 * C))
    gate = rng.standard_normal((7, 3 * C)) * 3
    scale = rng.standard_normal(C)
    eps = 1e-5
    xt = torch.from_numpy(x.reshape(-1, C))
    norm = F.rms_norm(xt, (C,), weight=torch.from_numpy(scale), eps=eps)
    gt = torch.from_numpy(gate.reshape(-1, C))
    for act, f in (("silu", F.silu), ("sigmoid", torch.sigmoid)):
        y = orc.gated_rmsnorm(x, gate, scale, eps=eps, activation=act)
        ref = (norm * f(gt)).reshape(x.shape).numpy()
        assert np.allclose(y, ref, rtol=1e-13, atol=1e-15), act
    y = orc.gated_rmsnorm(x, np.full_like(x, 50.0), scale, eps=eps, activation="sigmoid")
    assert np.allclose(y, norm.reshape(x.shape).numpy(), rtol=1e-14, atol=1e-15)


def pin_rmsnorm_invariants(orc):
    """eps = 0: scaling x by a power of two changes nothing (bitwise); the
    normalised rows have unit mean square; a constant row normalises to its
    sign; a zero gate gives 0 (silu) or half the normalised row (sigmoid);
    groups are independent rows."""
    rng = np.random.default_rng(43)
    C = 8
    x = rng.standard_normal((5, 2 * C))
    gate = rng.standard_normal((5, 2 * C))
    scale = rng.standard_normal(C)
    y = orc.gated_rmsnorm(x, gate, scale, eps=0.0)
    assert np.array_equal(orc.gated_rmsnorm(x * 2.0 ** 7, gate, scale, eps=0.0), y)
    sat = np.full_like(x, 60.0)
    u = orc.gated_rmsnorm(x, sat, np.ones(C), eps=0.0, activation="sigmoid")
    assert np.allclose((u.reshape(-1, C) ** 2).mean(1), 1.0, rtol=0, atol=1e-14)
    const = np.full((2, C), -3.25)
    assert np.array_equal(orc.gated_rmsnorm(const, np.full((2, C), 60.0), scale, eps=0.0, activation="sigmoid"),
                          np.broadcast_to(-scale, (2, C)))
    z = np.zeros_like(x)
    assert np.array_equal(orc.gated_rmsnorm(x, z, scale, eps=0.0, activation="silu"), z)
    half = orc.gated_rmsnorm(x, z, scale, eps=0.0, activation="sigmoid")
    assert np.allclose(half, 0.5 * orc.gated_rmsnorm(x, sat, scale, eps=0.0, activation="sigmoid"), rtol=1e-15)
    rows = orc.gated_rmsnorm(x.reshape(-1, C), gate.reshape(-1, C), scale)
    assert np.array_equal(rows.reshape(x.shape), orc.gated_rmsnorm(x, gate, scale))
    assert np.array_equal(orc.gated_rmsnorm(np.zeros((1, C)), gate[:1, :C], scale), np.zeros((1, C)))


ALL_PINS = [
    pin_brute_force, pin_delta_rule_memorises, pin_frozen_state, pin_reset,
    pin_power_of_two_scaling, pin_packing_invariance, pin_continuation, pin_gqa_repeat,
    pin_empty, pin_scalar_closed_form, pin_orthonormal_keys, pin_gates_library,
    pin_default_scale, pin_page_worked_example, pin_rounding_tie, pin_variants_brute_force,
    pin_variant_reductions, pin_state_history, pin_page_worked_example_window,
    pin_conv_library, pin_conv_continuation, pin_conv_special_kernels, pin_conv_slots,
    pin_rmsnorm_library, pin_rmsnorm_invariants,
]
