"""The oracle's pins have teeth: each plausible mistake planted in a copy of
the oracle's C source (a wrong index, a dropped term, a flipped sign, a
swapped operand) is caught by at least one pin.

Mistakes are planted only in a temporary copy of the oracle, compiled with
gcc on the CPU; the real oracle is untouched.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_attention as pins
import test_oracle_varlen as vpins

MUTATIONS = {
    "interleaved head map": ("int h = kv * G + g;", "int h = g * j->hkv + kv;"),
    "offset used as logical block": ("int64_t phys = row[t / j->B];",
                                     "int64_t phys = row[t % j->B];"),
    "pool axes swapped": ("((phys * j->hkv + kv) * j->B + t % j->B)",
                          "((kv * j->num_blocks + phys) * j->B + t % j->B)"),
    "softmax sign": ("double w = exp(z[t - lo] - m);", "double w = exp(m - z[t - lo]);"),
    "no normalisation": ("for (int d = 0; d < D; ++d) o[d] /= l;", ";"),
    "scale dropped": ("z[t - lo] = scale * dot;", "z[t - lo] = dot;"),
    "f16 exponent bias": ("e - 25);", "e - 24);"),
    "bf16 shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "K used as V": ("o[d] += w * V[(int64_t)t * D + d];", "o[d] += w * K[(int64_t)t * D + d];"),
    "partition end": ("(p + 1) * P < visible ? (p + 1) * P : visible;",
                      "(p + 1) * P < visible ? (p + 1) * P + 1 : visible;"),
    "merge drops l": ("double w = l[base + p] * exp(m[base + p] - M);",
                      "double w = exp(m[base + p] - M);"),
    "merge sign": ("double w = l[base + p] * exp(m[base + p] - M);",
                   "double w = l[base + p] * exp(M - m[base + p]);"),
    "q indexed by head first": ("((int64_t)(q0 + i) * j->hq + h) * D + d",
                                "((int64_t)h * j->hq + (q0 + i)) * D + d"),
    "causal limit off by one": ("int visible = ctx - qn + i + 1;",
                                "int visible = ctx - qn + i;"),
    "causal mask aligned to the start": ("int visible = ctx - qn + i + 1;",
                                         "int visible = i + 1 < ctx ? i + 1 : ctx;"),
    "output rows reversed in a chunk": ("j->out + ((int64_t)(orow + i) * j->hq + h) * D;",
                                        "j->out + ((int64_t)(orow + qn - 1 - i) * j->hq + h) * D;"),
    "max misses first score": ("if (z[t - lo] > m) m = z[t - lo];",
                               "if (t > lo && z[t - lo] > m) m = z[t - lo];"),
}


def _golden_loader():
    from conftest import load_golden
    return load_golden


def _run_pins():
    """Run the attention pins; return how many failed."""
    failed = 0
    checks = [
        lambda: pins.test_widen_f16_all_patterns(),
        lambda: pins.test_widen_bf16_all_patterns(),
        lambda: [pins.test_attention_matches_brute_force(s) for s in range(6)],
        lambda: pins.test_page_example_paged_equals_contiguous(_golden_loader()),
        lambda: pins.test_query_head_group_map(),
        lambda: pins.test_two_positions_give_logistic(3.0),
        lambda: pins.test_single_position_returns_its_value(),
        lambda: [pins.test_partials_merge_equals_whole(p) for p in (4, 12)],
        lambda: pins.test_one_token_partitions(),
        lambda: pins.test_lse_combine_closed_forms(),
        lambda: [vpins.test_varlen_matches_sdpa_lower_right(s) for s in range(4)],
        lambda: vpins.test_first_prefill_token_sees_one_position(),
    ]
    for c in checks:
        try:
            c()
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed += 1
    return failed


def _mutant_lib(tmp_path, old, new):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-o", str(so),
                    str(path), "-lm"], check=True)
    return str(so)


def test_clean_oracle_passes_all_pins():
    assert _run_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    so = _mutant_lib(tmp_path, old, new)
    real = oracle._load()
    lib = ctypes.CDLL(so)
    for f in ("orc_widen", "orc_gather", "orc_attention", "orc_attention_partials",
              "orc_lse_combine", "orc_attention_varlen"):
        getattr(lib, f).argtypes = getattr(real, f).argtypes
        getattr(lib, f).restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    with np.errstate(all="ignore"):
        assert _run_pins() >= 1, f"no pin caught: {name}"
