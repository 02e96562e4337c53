"""Mutation tests: plant plausible mistakes in a copy of the oracle's C source,
build it, and require that at least one pin fails for every mistake.  Runs on
the CPU only; the oracle itself is never modified."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, exact source text, replacement).  Each replacement keeps every memory
# access in bounds, so a mutant can only compute wrong numbers.
MUTANTS = [
    ("decay_sign", "double alpha = exp(g[i]);", "double alpha = exp(-g[i]);"),
    ("decay_dropped", "S[i * dv + j] *= alpha;", "S[i * dv + j] *= 1.0;"),
    ("decay_wrong_channel", "double alpha = exp(g[i]);", "double alpha = exp(g[dk - 1 - i]);"),
    ("erase_sign", "- beta * k[i] * e[j] + beta", "+ beta * k[i] * e[j] + beta"),
    ("erase_dropped", "- beta * k[i] * e[j] + beta", "- 0.0 * k[i] * e[j] + beta"),
    ("erase_without_beta", "- beta * k[i] * e[j] + beta", "- k[i] * e[j] + beta"),
    ("write_dropped", "+ beta * k[i] * v[j];", "+ 0.0 * k[i] * v[j];"),
    ("retrieve_with_query", "e[j] += k[i] * S[i * dv + j];", "e[j] += q[i] * S[i * dv + j];"),
    ("read_with_key", "o[j] += S[i * dv + j] * q[i];", "o[j] += S[i * dv + j] * k[i];"),
    ("read_before_decay_only", "o[j] += S[i * dv + j] * q[i];",
     "o[j] += (S[i * dv + j] + beta * k[i] * (e[j] - v[j])) * q[i];"),
    ("token_layout", "size_t row = ((size_t)b * T + t) * H + h;",
     "size_t row = ((size_t)h * T + t) * B + b;"),
    ("initial_state_ignored", "memcpy(S, S0 + (size_t)bh * sd, sd * sizeof(double));",
     "memset(S, 0, sd * sizeof(double));"),
    ("checkpoint_off_by_one", "(t + 1) % ckpt_every == 0 || t == T - 1",
     "(t + 2) % ckpt_every == 0 || t == T - 1"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site for %s not found exactly once" % name
    mutant_src = tmp_path / ("kda_oracle_%s.c" % name)
    mutant_src.write_text(src.replace(old, new))
    so = str(tmp_path / ("libkda_oracle_%s.so" % name))
    flags = [f for f in oracle.CFLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, "-o", so, str(mutant_src), "-lm"], check=True)
    lib = oracle.load_library(so)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(lib=lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
