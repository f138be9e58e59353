"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pins catch every one of them (CPU only; nothing here touches a GPU)."""
import os

import pytest

import oracle
from tests import oracle_pins

# (name, text in kda_oracle.c, replacement)
MUTANTS = [
    ("delta sign", "u[j] = b * (bf16_to_f64(v[v_off + j]) - u[j]);", "u[j] = b * (bf16_to_f64(v[v_off + j]) + u[j]);"),
    ("missing beta in write", "u[j] = b * (bf16_to_f64(v[v_off + j]) - u[j]);", "u[j] = (bf16_to_f64(v[v_off + j]) - u[j]);"),
    ("decay applied twice", "S[d * V + j] *= dec[d];", "S[d * V + j] *= dec[d] * dec[d];"),
    ("no decay", "S[d * V + j] *= dec[d];", "S[d * V + j] *= 1.0;"),
    ("clamp with min", "return a > lower_bound ? a : lower_bound;", "return a < lower_bound ? a : lower_bound;"),
    ("softplus sign", "log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    ("rate without exp", "double a = -exp(A_log) * kda_softplus(g + dt_bias);", "double a = -A_log * kda_softplus(g + dt_bias);"),
    ("q normalised by |k|", "qh[d] *= rq; kh[d] *= rk;", "qh[d] *= rk; kh[d] *= rk;"),
    ("state read transposed", "u[j] += S[d * V + j] * qh[d];", "u[j] += S[j * K + d] * qh[d];"),
    ("sigmoid sign", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("dt_bias ignores head", "(double)dt_bias[h * K + d]", "(double)dt_bias[d]"),
    ("initial state dropped", "S[i] = initial_state ? initial_state[sidx + (size_t)i] : 0.0;", "S[i] = 0.0;"),
    ("scale dropped", "out[v_off + j] = scale * u[j];", "out[v_off + j] = u[j];"),
    ("norm epsilon 1e-3", "#define KDA_ORACLE_EPS 1e-6", "#define KDA_ORACLE_EPS 1e-3"),
    ("write uses unnormalised k", "S[d * V + j] += kh[d] * u[j];", "S[d * V + j] += kh[d] * u[j] / rk * rk * (1.0 + 1e-3);"),
]

# cheap pins first: a mutant is caught at its first failing pin
ORDER = ["pin_gate_values", "pin_single_token", "pin_two_tokens", "pin_decay_only", "pin_hadamard_recall",
         "pin_overwrite", "pin_golden", "pin_chunked_form", "pin_brute_force", "pin_linearity",
         "pin_varlen_separate", "pin_split_run", "pin_contraction", "pin_head_permutation"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source()
    assert old in src, "mutation site not found: " + name
    path = oracle.compile_variant(src.replace(old, new, 1), str(tmp_path / "mutant.so"))
    orc = oracle.Oracle(path)
    pins = {p.__name__: p for p in oracle_pins.ALL_PINS}
    caught = None
    for pname in ORDER:
        try:
            pins[pname](orc)
        except AssertionError:
            caught = pname
            break
    assert caught is not None, "no pin caught the mutant: " + name
