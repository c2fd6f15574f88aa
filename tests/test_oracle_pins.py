"""The CPU oracle against its pins, and the pins against planted mistakes.

CPU only.  ``test_pin`` runs every pin against the oracle as built.
``test_mutant_is_caught`` copies the oracle's C source, plants one plausible
mistake in the copy (a swapped sign, a wrong bit order, a dropped term, a
wrong index, a wrong exponent bias ...), builds it, and checks that at least
one pin fails on it.  The oracle's own source is never modified.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.fixture(scope="module")
def real_oracle():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(real_oracle, pin):
    pin(real_oracle)


# (name, text in tern_oracle.c, replacement).  Every replacement keeps all
# memory accesses in bounds, so a mutant can only give wrong numbers.
MUTANTS = [
    ("signs_swapped", "case 1: return 1;\n    case 2: return -1;",
     "case 1: return -1;\n    case 2: return 1;"),
    ("reserved_as_minus_one", "case 3: return 0;", "case 3: return -1;"),
    ("reserved_as_plus_one", "case 3: return 0;", "case 3: return 1;"),
    ("unpack_msb_first", "(byte >> (2 * (k % 4)))", "(byte >> (2 * (3 - k % 4)))"),
    ("pack_msb_first", "<< (2 * i);", "<< (2 * (3 - i));"),
    ("pack_minus_one_code", "if (t == -1) return 2;", "if (t == -1) return 1;"),
    ("row_stride_wrong", "packed[n * (K / 4) + k / 4]", "packed[n * (K / 8) + k / 4]"),
    ("subtract_dropped", "else if (t == -1) block -= x;", "else if (t == -1) block += x;"),
    ("minus_one_skipped", "else if (t == -1) block -= x;", "else if (t == -1) block -= 0.0;"),
    ("scale_dropped", "y += s * block;                        /* scale applied", "y += block;                        /* scale applied"),
    ("scale_group_zero", "double s = oracle_f16_to_f64(S[n * groups + g]);",
     "double s = oracle_f16_to_f64(S[n * groups]);"),
    ("scale_groups_reversed", "double s = oracle_f16_to_f64(S[n * groups + g]);",
     "double s = oracle_f16_to_f64(S[n * groups + (groups - 1 - g)]);"),
    ("block_last_weight_dropped", "for (int64_t k = k0; k < k1; ++k) {", "for (int64_t k = k0; k < k1 - 1; ++k) {"),
    ("x_reversed_along_k", "uint16_t bits = X[m * K + k];", "uint16_t bits = X[m * K + (K - 1 - k)];"),
    ("x_row_ignored", "uint16_t bits = X[m * K + k];", "uint16_t bits = X[k];"),
    ("f16_bias_off", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("f16_subnormal_off", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("f16_hidden_bit_missing", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(f), e - 25)"),
    ("bf16_bias_off", "ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)"),
    ("bf16_read_as_f16", "return x_kind == 1 ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);",
     "return oracle_f16_to_f64(bits);"),
    ("bound_signed", "        ax += fabs(x);", "        ax += x;"),
    ("bound_unscaled", "        b += fabs(s) * ax;\n    }\n    *y_out = y;", "        b += ax;\n    }\n    *y_out = y;"),
    ("round_truncates", "nearbyint(a / q) * q", "floor(a / q) * q"),
    ("ulp_too_small", "return ldexp(1.0, e - p + 1);", "return ldexp(1.0, e - p);"),
    ("unpack_row_zero", "T[n * K + k] = (int8_t)oracle_weight(packed, K, n, k);",
     "T[n * K + k] = (int8_t)oracle_weight(packed, K, 0, k);"),
    ("cols_last_dropped", "for (int64_t n = n0; n < n1; ++n)\n            one_output",
     "for (int64_t n = n0; n < n1 - 1; ++n)\n            one_output"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"lib{name}.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", so, str(path), "-lm"],
                   check=True)
    return so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    mutant = oracle.Oracle(_build_mutant(tmp_path, name, old, new))
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError) as e:  # a pin failed: the mistake is visible
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"


def test_negative_control_page1_map_fails_anchors():
    """The illustrative map of the m.xxqk.cn page is not the method's map."""
    wrong = {int(a): int(b) for a, b in oracle_pins.read_table("wrong_code_map_page1.txt")}
    bad = 0
    for byte, weights in oracle_pins.anchor_bytes():
        got = [wrong[(byte >> (2 * i)) & 3] for i in range(4)]
        bad += got != weights
    assert bad > 0
