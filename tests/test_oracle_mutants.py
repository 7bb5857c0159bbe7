"""The pins catch plausible mistakes: each planted mistake in a copy of the
oracle source (a dropped term, a wrong sign or index, a transposed operand, a
missing scale, an off-by-one window) must fail at least one pin.  CPU only;
the mutated copies are built in a temporary directory and never shipped."""
import os

import pytest

import oracle
import pins

MUTANTS = {
    "bias_dropped": ("if (rpb) bias =", "if (0) bias ="),
    "bias_sign": ("(ky - y + k - 1)) * nb + (kx - x + k - 1)",
                  "(y - ky + k - 1)) * nb + (x - kx + k - 1)"),
    "bias_axes_swapped": ("(ky - y + k - 1)) * nb + (kx - x + k - 1)",
                          "(kx - x + k - 1)) * nb + (ky - y + k - 1)"),
    "bias_unscaled": ("logit[a * k + c] = (dot + bias) * scale;",
                      "logit[a * k + c] = dot * scale + bias;"),
    "no_scale": ("const double scale = 1.0 / sqrt((double)d);", "const double scale = 1.0;"),
    "window_off_by_one": ("int s = i - k / 2;", "int s = i - k / 2 + 1;"),
    "dot_drops_a_term": ("for (int t = 0; t < d; ++t) dot +=", "for (int t = 1; t < d; ++t) dot +="),
    "value_rows_flipped": ("(map + (int64_t)(sy + a) * W + (sx + c)) * d",
                           "(map + (int64_t)(sy + (k - 1 - a)) * W + (sx + c)) * d"),
    "normaliser_off": ("const double w = logit[a * k + c] / z;",
                       "const double w = logit[a * k + c] / (z + 1e-3);"),
    "key_query_mixup": ("const double *kj = kk + (map + (int64_t)ky * W + kx) * d;",
                        "const double *kj = q + (map + (int64_t)ky * W + kx) * d;"),
    "lse_without_max": ("if (lse) *lse = m + log(z);", "if (lse) *lse = log(z);"),
    "lse_log2": ("if (lse) *lse = m + log(z);", "if (lse) *lse = m + log2(z);"),
    # the sampled form's split of a linear query index
    "sampled_batch_head_swapped": (
        "const int h = (int)((p / ((int64_t)W * H)) % heads);\n"
        "            const int64_t b = p / ((int64_t)W * H * heads);",
        "const int h = (int)(p / ((int64_t)W * H * B));\n"
        "            const int64_t b = (p / ((int64_t)W * H)) % B;"),
    "sampled_row_col_swapped": (
        "const int x = (int)(p % W);\n            const int y = (int)((p / W) % H);",
        "const int y = (int)(p % H);\n            const int x = (int)((p / H) % W);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation site not found: %s" % name
    path = os.path.join(str(tmp_path), "mut_%s.c" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_oracle(path, os.path.join(str(tmp_path), "libmut_%s.so" % name))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passes every pin" % name
