"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
the pin suite to catch every one of them: a dropped term, a flipped sign, a
wrong operand or index, a wrong default."""
import os

import pytest

import oracle
import oracle_pins

# (label, text in gdn_oracle.c, replacement)
MUTANTS = [
    ("dropped decay", "S[i * d_v + j] *= alpha;", ";"),
    ("decay applied as g, not exp(g)", "const acc_t alpha = (acc_t)exp(g[t * h_v + h]);",
     "const acc_t alpha = (acc_t)g[t * h_v + h];"),
    ("delta sign flipped", "d[j] = bt * ((acc_t)vt[j] - r[j]);", "d[j] = bt * (r[j] - (acc_t)vt[j]);"),
    ("beta ignored", "d[j] = bt * ((acc_t)vt[j] - r[j]);", "d[j] = ((acc_t)vt[j] - r[j]);"),
    ("retrieval against the query", "acc += S[i * d_v + j] * (acc_t)kt[i];\n        r[j] = acc;",
     "acc += S[i * d_v + j] * (acc_t)qt[i];\n        r[j] = acc;"),
    ("update with the query", "S[i * d_v + j] += (acc_t)kt[i] * d[j];", "S[i * d_v + j] += (acc_t)qt[i] * d[j];"),
    ("scale dropped", "ot[j] = (double)((acc_t)scale * acc);", "ot[j] = (double)acc;"),
    ("interleaved head map", "const int32_t hq = h / (h_v / h_qk);", "const int32_t hq = h % h_qk;"),
    ("initial state ignored",
     "S[e] = initial_state ? (acc_t)initial_state[u * state_elems + e] : (acc_t)0;",
     "S[e] = (acc_t)0;"),
    ("default scale from d_v", "scale = 1.0 / sqrt((double)d_k);", "scale = 1.0 / sqrt((double)d_v);"),
    ("softplus tail sign", "log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    ("sigmoid negative branch", "return e / (1.0 + e);", "return 1.0 / (1.0 + e);"),
    ("decay sign", "g[idx] = -exp(A_log[h])", "g[idx] = exp(A_log[h])"),
    ("dt_bias dropped", "gdnref_softplus(a[idx] + dt_bias[h])", "gdnref_softplus(a[idx])"),
    ("per-key decay row ignored", "const acc_t alpha_i = (acc_t)exp(gt[i]);",
     "const acc_t alpha_i = (acc_t)exp(gt[0]);"),
    ("shared beta not per token", "beta_shared ? beta[t] :", "beta_shared ? beta[0] :"),
    ("history slot off by one", "const int64_t w = (t - t0) - ((t1 - t0) - window);",
     "const int64_t w = (t - t0) - ((t1 - t0) - window) - 1;"),
    ("conv taps reversed", "z += weight[(int64_t)c * ksize + j]", "z += weight[(int64_t)c * ksize + (ksize - 1 - j)]"),
    ("conv dilation ignored", "XP(t - carry + (int64_t)j * dilation)", "XP(t - carry + (int64_t)j)"),
    ("conv silu dropped", "y[(t0 + t) * channels + c] = silu ? z * gdnref_sigmoid(z) : z;",
     "y[(t0 + t) * channels + c] = z;"),
    ("conv bias dropped", "double z = bias ? bias[c] : 0.0;", "double z = 0.0;"),
    ("conv state off by one", "fs[i * channels + c] = XP(L - carry + i);", "fs[i * channels + c] = XP(L - carry + i - 1);"),
    ("conv initial state ignored", "(s0 ? s0[(carry + (p)) * channels + c] : 0.0)", "0.0"),
    ("conv slot ignored", "states[n * per + e] = pool[(int64_t)s * per + e];",
     "states[n * per + e] = pool[(int64_t)n * per + e];"),
    ("conv new state not written back", "pool[(int64_t)s * per + e] = fresh[n * per + e];", ";"),
    ("rmsnorm mean over the row", "sqrt(ss / group + eps)", "sqrt(ss / width + eps)"),
    ("rmsnorm eps outside the root", "sqrt(ss / group + eps)", "(sqrt(ss / group) + eps)"),
    ("rmsnorm activations swapped", "activation == 1 ? gr[i] * s : s", "activation == 2 ? gr[i] * s : s"),
    ("rmsnorm scale not per element", "scale[i] * act", "scale[0] * act"),
]


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, label, old, new):
    with open(oracle.SRC) as fh:
        src = fh.read()
    assert src.count(old) == 1, f"mutation anchor for '{label}' not unique in gdn_oracle.c"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as fh:
        fh.write(src.replace(old, new))
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmutant.so"))
    m = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{label}'"
