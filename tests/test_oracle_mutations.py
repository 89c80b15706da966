"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a temporary copy of oracle/gdn_oracle.c (a
flipped sign, a dropped factor, a wrong index or operand), compiles it with
gcc on the CPU, points the oracle wrapper at it and requires that at least
one pin of test_oracle_pins.py fails.  The committed oracle is never touched.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

MUTATIONS = {
    "error_sign": ("r[j] = b * (vt[j] - alpha * r[j]);", "r[j] = b * (vt[j] + alpha * r[j]);"),
    "drop_beta": ("r[j] = b * (vt[j] - alpha * r[j]);", "r[j] = (vt[j] - alpha * r[j]);"),
    "error_undecayed": ("r[j] = b * (vt[j] - alpha * r[j]);", "r[j] = b * (vt[j] - r[j]);"),
    "decay_sign": ("const double alpha = exp(J->g[(size_t)t * hv + h]);",
                   "const double alpha = exp(-J->g[(size_t)t * hv + h]);"),
    "drop_decay": ("S[(size_t)i * dv + j] = alpha * S[(size_t)i * dv + j] + kt[i] * r[j];",
                   "S[(size_t)i * dv + j] = S[(size_t)i * dv + j] + kt[i] * r[j];"),
    "gqa_modulo": ("const int32_t hq = (int32_t)(((int64_t)h * hqk) / hv);",
                   "const int32_t hq = (int32_t)(h % hqk);"),
    "read_with_q": ("r[j] += kt[i] * S[(size_t)i * dv + j];", "r[j] += qt[i] * S[(size_t)i * dv + j];"),
    "write_with_q": ("alpha * S[(size_t)i * dv + j] + kt[i] * r[j];", "alpha * S[(size_t)i * dv + j] + qt[i] * r[j];"),
    "output_with_k": ("ot[j] += qt[i] * S[(size_t)i * dv + j];", "ot[j] += kt[i] * S[(size_t)i * dv + j];"),
    "drop_scale": ("ot[j] *= J->scale;", "ot[j] *= 1.0;"),
    "g_head_index": ("exp(J->g[(size_t)t * hv + h])", "exp(J->g[(size_t)t * hv])"),
    "beta_head_index": ("J->beta[(size_t)t * hv + h]", "J->beta[(size_t)t * hv + (hv - 1 - h)]"),
    "state_offset": ("const size_t state_off = ((size_t)n * hv + h) * state_elems;",
                     "const size_t state_off = ((size_t)n * hv) * state_elems;"),
}

PINS = [
    lambda: pins.test_against_closed_form_factor_products(True),
    lambda: pins.test_against_closed_form_factor_products(False),
    pins.test_pure_decay_when_beta_is_zero,
    pins.test_exact_recall_alpha_one_beta_one_unit_keys,
    pins.test_one_hot_keys_overwrite_rows,
    lambda: pins.test_chunkwise_parallel_form(16, "forward"),
    pins.test_output_is_linear_in_scale,
    pins.test_grouped_heads_read_their_block_of_query_key_heads,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, "mutation site vanished from the oracle source"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(so),
                    str(mutated), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    lib.gdn_oracle_forward.argtypes = oracle._load().gdn_oracle_forward.argtypes
    lib.gdn_oracle_forward.restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, "no pin caught the planted mistake %r" % name
