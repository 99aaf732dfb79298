"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

# (name, text in qknorm_oracle.c, replacement)
MUTANTS = [
    ("eps_outside_sqrt", "sqrt(S / (double)H_total + eps)", "(sqrt(S / (double)H_total) + eps)"),
    ("mean_over_slice_width", "S / (double)H_total", "S / (double)W"),
    ("sum_not_mean", "S / (double)H_total", "S"),
    ("dropped_last_term", "j < (s + 1) * w;", "j < (s + 1) * w - 1;"),
    ("slices_reversed", "P[(int64_t)s * T + t] = acc;", "P[(int64_t)(K - 1 - s) * T + t] = acc;"),
    ("row_stride_ignored", "const float *row = x + t * ldx;\n        for (int s", "const float *row = x + t;\n        for (int s"),
    ("gamma_reversed", "* (double)gamma[j]; /* Eq. 1 order */", "* (double)gamma[W - 1 - j];"),
    ("multiply_by_rms", "(double)row[j] / rms", "(double)row[j] * rms"),
    ("output_sign", "out[j] = (double)row[j]", "out[j] = -(double)row[j]"),
    ("abs_not_square", "acc += v * v;", "acc += v < 0 ? -v : v;"),
    ("first_slice_only", "for (int s = 0; s < K; ++s) /* Eq. 5", "for (int s = 0; s < 1; ++s) /* Eq. 5"),
    # inverse RMS alone
    ("rinv_over_slice", "r[t] = 1.0 / sqrt(S / (double)H + eps);", "r[t] = 1.0 / sqrt(S / (double)(H / K) + eps);"),
    ("rinv_rms_not_inverse", "r[t] = 1.0 / sqrt(S / (double)H + eps);", "r[t] = sqrt(S / (double)H + eps);"),
    ("rinv_first_slice", "for (int s = 0; s < K; ++s)\n            S += P", "for (int s = 0; s < 1; ++s)\n            S += P"),
    # headwise
    ("head_mean_over_row", "sqrt(S / (double)D + eps)", "sqrt(S / (double)H + eps)"),
    ("head_eps_outside_sqrt", "sqrt(S / (double)D + eps)", "(sqrt(S / (double)D) + eps)"),
    ("head_stat_of_first_head", "const double v = (double)row[h0 + j];", "const double v = (double)row[j];"),
    ("head_dropped_last_term", "for (int64_t j = 0; j < D; ++j) {", "for (int64_t j = 0; j < D - 1; ++j) {"),
    ("head_weights_shifted", "/ rms * (double)gamma[j];\n        }", "/ rms * (double)gamma[(j + 1) % D];\n        }"),
    ("head_weights_by_column", "/ rms * (double)gamma[j];\n        }", "/ rms * (double)gamma[(j + (h0 > 0)) % D];\n        }"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, "mutation site vanished from the oracle: " + name
    mutated = src.replace(old, new)
    msrc = os.path.join(tmp_path, "mutant.c")
    with open(msrc, "w") as f:
        f.write(mutated)
    lib = obuild.build(src=msrc, out=os.path.join(tmp_path, "libmutant.so"),
                       extra_flags=("-Wno-unused-parameter", "-Wno-unused-variable"))
    caught = []
    with oracle.using(lib):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
    assert caught, "no pin caught mutant " + name
