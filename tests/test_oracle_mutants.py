"""The oracle's pins are strong enough to catch plausible mistakes.

Each case below plants one mistake in a *copy* of ``oracle/kda_oracle.c`` (text
substitution or swapping two steps of the token loop), compiles the copy into
a temporary directory with gcc, points the oracle's front end at it, and runs
the pins of ``test_oracle_pins``.  A mutant passes this test only if at least
one pin fails for it.  Everything runs on the CPU; the real oracle is untouched.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")).read()

# Step markers inside the token loop (each opens one step of the update).
STEP_DECAY = "/* S' = Diag(alpha_t) S_{t-1}"
STEP_PREDICT = "/* vhat = S'^T k_t */"
STEP_WRITE = "/* S_t = S' + beta_t k_t e_t^T"
STEP_READ = "/* o_t = S_t^T q_t */"
LOOP_END = "\n        }\n\n        if (state_out)"


def _steps(src):
    """Split the token loop body into (head, [decay, predict, write, read], tail)."""
    idx = [src.index(m) for m in (STEP_DECAY, STEP_PREDICT, STEP_WRITE, STEP_READ)]
    end = src.index(LOOP_END)
    # back up to the start of each marker's line
    starts = [src.rindex("\n", 0, i) + 1 for i in idx]
    parts = [src[a:b] for a, b in zip(starts, starts[1:] + [end + 1])]
    return src[:starts[0]], parts, src[end + 1:]


def _swap(src, a, b):
    head, parts, tail = _steps(src)
    parts[a], parts[b] = parts[b], parts[a]
    return head + "".join(parts) + tail


def _sub(old, new):
    def f(src):
        assert old in src, f"mutation anchor not found: {old}"
        return src.replace(old, new)
    return f


MUTANTS = {
    "beta_dropped_from_write": _sub("+= bt * kt[i] * (vt[j] - vhat[j])",
                                    "+= kt[i] * (vt[j] - vhat[j])"),
    "gate_sign_flipped": _sub("exp(gt[i])", "exp(-gt[i])"),
    "read_with_key_not_query": _sub("acc += S[i * d_v + j] * qt[i];",
                                    "acc += S[i * d_v + j] * kt[i];"),
    "error_sign_flipped": _sub("(vt[j] - vhat[j])", "(vhat[j] - vt[j])"),
    "plain_write_no_error": _sub("(vt[j] - vhat[j])", "vt[j]"),
    "state_stored_untransposed": _sub("M1[j * d_k + i] = S[i * d_v + j];",
                                      "M1[i * d_v + j] = S[i * d_v + j];"),
    "state_loaded_untransposed": _sub("M0[j * d_k + i]", "M0[i * d_v + j]"),
    "decay_along_values": _sub("S[i * d_v + j] *= alpha_i;",
                               "S[i * d_v + j] *= exp(gt[j % d_k]);"),
    "next_tokens_gate": _sub(
        "const double *gt = log_alpha + (t * n_heads + h) * d_k;",
        "const double *gt = log_alpha + (((t + 1 < seq_start[n + 1]) ? t + 1 : t)"
        " * n_heads + h) * d_k;"),
    "read_before_write": lambda s: _swap(s, 2, 3),
    "predict_before_decay": lambda s: _swap(s, 0, 1),
}

PIN_CALLS = [
    (pins.test_brute_force_exact_transition_products, (0, 8, 3, 4)),
    (pins.test_brute_force_exact_transition_products, (1, 8, 4, 3)),
    (pins.test_projection_form_agrees, (0, 50, 5, 7)),
    (pins.test_beta_zero_is_pure_per_channel_decay, ()),
    (pins.test_beta_zero_alpha_one_freezes_state, ()),
    (pins.test_unit_key_beta_one_retrieves_value_exactly, ()),
    (pins.test_orthonormal_keys_reduce_to_linear_attention, ()),
    (pins.test_one_hot_keys_decayed_sum, (False,)),
    (pins.test_scalar_gate_equals_gated_deltanet, ()),
    (pins.test_already_correct_memory_writes_nothing, ()),
]


def _failing_pins(lib):
    saved = oracle._lib
    oracle._lib = lib
    failed = []
    try:
        for fn, args in PIN_CALLS:
            try:
                fn(*args)
            except AssertionError:
                failed.append(fn.__name__)
    finally:
        oracle._lib = saved
    return failed


def _compile(src, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    "-o", str(so), str(c), "-lm"], check=True)
    return oracle.open_library(str(so))


def test_unmodified_copy_passes_every_pin(tmp_path):
    assert _failing_pins(_compile(SRC, tmp_path, "same")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    mutant = MUTANTS[name](SRC)
    assert mutant != SRC
    failed = _failing_pins(_compile(mutant, tmp_path, name))
    assert failed, f"no pin caught mutant {name}"
