"""CPU tests: the f64 oracle against facts it does not compute itself, and proof that
plausible mistakes planted in copies of the oracle are caught by those facts."""
from __future__ import annotations

import subprocess
from pathlib import Path

import pytest

from oracle import oracle as orc
from tests import oracle_pins

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# Each mutant changes one thing a careless oracle could get wrong.  The replacement
# must match exactly one place in the source so the mutant is the intended one.
MUTANTS = {
    "no_max_subtraction": ("w[j] = exp(w[j] - m);", "w[j] = exp(w[j]);"),
    "causal_excludes_diagonal": ("p->causal ? i + 1 : key_hi", "p->causal ? i : key_hi"),
    "negated_scale": ("w[j] = p->scale * dot;", "w[j] = -p->scale * dot;"),
    "head_dropped_from_key_index": ("int64_t kj = ((key_lo + j) * H + h) * (int64_t)d;",
                                    "int64_t kj = ((key_lo + j) * H) * (int64_t)d;"),
    "no_normalisation": ("for (int64_t j = 0; j < nk; ++j) w[j] /= z;", ""),
    "segment_start_ignored_for_keys": ("int64_t kj = ((key_lo + j) * H + h)", "int64_t kj = ((j) * H + h)"),
    "value_row_from_query": ("int64_t vj = ((key_lo + j) * H + h)", "int64_t vj = ((i) * H + h)"),
    "transposed_qk_channel": ("elem(p->k, p->dtype, kj + c)", "elem(p->k, p->dtype, kj + (d - 1 - c))"),
    "last_key_dropped": ("int64_t nk = last - key_lo;", "int64_t nk = last - key_lo - (last - key_lo > 1);"),
    "bf16_widened_wrongly": ("(uint32_t)((const uint16_t*)base)[idx] << 16", "(uint32_t)((const uint16_t*)base)[idx] << 15"),
    "value_weight_squared": ("o[c] += w[j] * elem(p->v", "o[c] += w[j] * w[j] * elem(p->v"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path: Path):
    old, new = MUTANTS[name]
    src = orc.SRC.read_text()
    assert src.count(old) == 1, f"mutation target for {name} not unique"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(lib_path),
                    str(mutated), "-lm"], check=True)
    lib = orc.load(lib_path)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with_np_errors_quiet(pin, lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def with_np_errors_quiet(fn, lib):
    import numpy as np

    with np.errstate(all="ignore"):
        fn(lib)
