"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The mistakes are planted by text substitution into a temporary copy of ``oracle/oracle.c`` that
is compiled with the oracle's own build step; the real oracle is never modified.  Every
substitution must match the source exactly once, so a change to the oracle that makes a mutant
stale fails loudly instead of silently testing nothing.  CPU only.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement, which occurrence (0-based))
MUTANTS = [
    ("rope_sign", "out[i] = x1 * c - x2 * s;", "out[i] = x1 * c + x2 * s;", 0),
    ("rope_interleaved_pairs", "double x1 = x[i], x2 = x[i + half];",
     "double x1 = x[2 * i], x2 = x[2 * i + 1];", 0),
    ("rope_freq_exponent", "pow(base, -2.0 * i / n)", "pow(base, -1.0 * i / n)", 0),
    ("rope_position_off_by_one", "(double)(a->pos0 + t), a->rope_base, kt)",
     "(double)(a->pos0 + t + 1), a->rope_base, kt)", 0),
    ("no_key_scale", "kt[i] *= ks;", "kt[i] *= 1.0;", 0),
    ("rmsnorm_sum_not_mean", "sqrt(ss / n + eps)", "sqrt(ss + eps)", 0),
    ("rmsnorm_eps_outside", "1.0 / sqrt(ss / n + eps)", "1.0 / sqrt(ss / n) + eps", 0),
    ("rmsnorm_no_weight", "(w ? w[i] : 1.0)", "1.0", 0),
    ("key_norm_uses_query_weight", "oracle_rmsnorm(tmp, wk, d, a->eps, tmp);",
     "oracle_rmsnorm(tmp, wq, d, a->eps, tmp);", 0),
    ("sigmoid_sign", "1.0 / (1.0 + exp(-x))", "1.0 / (1.0 + exp(x))", 0),
    ("no_gate", "y[i] *= oracle_sigmoid(g[i]);", "y[i] *= 1.0;", 0),
    ("gate_reads_wrong_input", "for (int i = 0; i < d; ++i) gt[i] = load_elem(a->g",
     "for (int i = 0; i < d; ++i) gt[i] = load_elem(a->q", 0),
    ("token_decayed_at_insert",
     "S[(size_t)r * d + c] = lam * S[(size_t)r * d + c] + kt[r] * vt[c];",
     "S[(size_t)r * d + c] = lam * (S[(size_t)r * d + c] + kt[r] * vt[c]);", 0),
    ("state_transposed_in_query", "acc += qt[r] * S[(size_t)r * d + c];",
     "acc += qt[r] * S[(size_t)c * d + r];", 0),
    ("outer_product_transposed", "+ kt[r] * vt[c];", "+ kt[c] * vt[r];", 0),
    ("initial_state_ignored", "for (size_t i = 0; i < (size_t)d * d; ++i) S[i] = s0[i];",
     "for (size_t i = 0; i < (size_t)d * d; ++i) S[i] = 0.0 * s0[i];", 0),
    ("chunk_carry_off_by_one", "double carry = pow(lam, i + 1);", "double carry = pow(lam, i);", 0),
    ("chunk_intra_decay_sign", "score *= pow(lam, i - j);", "score *= pow(lam, j - i + 0.0 * i);", 0),
    ("chunk_state_weight", "double w = pow(lam, n - 1 - j);", "double w = pow(lam, n - j);", 0),
    ("chunk_state_decay", "double decay_all = pow(lam, n);", "double decay_all = pow(lam, n - 1);", 0),
    ("decode_no_decay", "= lam * (double)a->state_in[sb", "= 1.0 * (double)a->state_in[sb", 0),
    ("bf16_widen_wrong_shift", "<< 16;", "<< 15;", 0),
]


def _mutate(text, old, new, which):
    count = text.count(old)
    assert count >= which + 1, f"mutation anchor not found: {old!r}"
    start = -1
    for _ in range(which + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, which, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"{name}: anchor missing from oracle.c"
    mutated = _mutate(src, old, new, which)
    assert mutated != src
    path = tmp_path / "oracle_mutant.c"
    path.write_text(mutated)
    lib_path = str(tmp_path / "liboracle_mutant.so")
    oracle_build.build(str(path), lib_path, extra_flags=("-w",))
    lib = oracle.load(lib_path)
    failed = []
    for pin in ALL_PINS:
        try:
            err, tol = pin(lib)
        except Exception as exc:  # a mutant may also break an invariant outright
            failed.append(f"{pin.__name__} raised {type(exc).__name__}")
            continue
        if not err <= tol:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
