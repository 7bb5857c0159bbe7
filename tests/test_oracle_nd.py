"""The N-axis oracle (NA1D, NA3D, SASA) against its pins, and planted
mistakes in a copy of its source that some pin must catch.  CPU only."""
import os

import pytest

import oracle
import pins_nd


@pytest.mark.parametrize("pin", pins_nd.ALL_PINS_ND, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default_nd(), oracle.default())


MUTANTS = {
    "sasa_clamps_too": ("    if (mode == 0) {\n        if (s < 0) s = 0;",
                        "    if (1) {\n        if (s < 0) s = 0;"),
    "padding_left_out_of_softmax": ("        logit[j] = (dot + bias) * scale;",
                                    "        logit[j] = inside ? (dot + bias) * scale : -INFINITY;"),
    "bias_axes_swapped": ("bias = rpb[(((int64_t)h * nb[0] + r0) * nb[1] + r1) * nb[2] + r2];",
                          "bias = rpb[(((int64_t)h * nb[0] + r2) * nb[1] + r1) * nb[2] + r0];"),
    "bias_sign": ("const int64_t r0 = p0 - pos[0] + s->k[0] - 1",
                  "const int64_t r0 = pos[0] - p0 + s->k[0] - 1"),
    "window_axis_mixup": ("st[a] = na_nd_window_start(pos[a], s->k[a], s->L[a], s->mode);",
                          "st[a] = na_nd_window_start(pos[a], s->k[a], s->L[2 - a], s->mode);"),
    "no_scale": ("const double scale = 1.0 / sqrt((double)d);", "const double scale = 1.0;"),
    "index_split_swapped": ("    pos[2] = (int)(p % s->L[2]);\n    p /= s->L[2];\n    pos[1] = (int)(p % s->L[1]);",
                            "    pos[1] = (int)(p % s->L[2]);\n    p /= s->L[2];\n    pos[2] = (int)(p % s->L[1]);"),
    "padded_value_read": ("            continue;\n        const double *vj",
                          "            p0 = p0 < 0 ? 0 : p0;\n        const double *vj"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.ND_SOURCE).read()
    assert src.count(old) == 1, "mutation site not found: %s" % name
    if name == "padded_value_read":  # make the mutated line compile: p0 must be assignable
        src = src.replace("        const int p0 = st[0] + c0, p1 = st[1] + c1, p2 = st[2] + c2;\n"
                          "        if (p0 < 0",
                          "        int p0 = st[0] + c0; const int p1 = st[1] + c1, p2 = st[2] + c2;\n"
                          "        if (p0 < 0")
    path = os.path.join(str(tmp_path), "mut_%s.c" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_oracle(path, os.path.join(str(tmp_path), "libmut_%s.so" % name))
    orc = oracle.OracleND(lib)
    failed = []
    for pin in pins_nd.ALL_PINS_ND:
        try:
            pin(orc, oracle.default())
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passes every pin" % name
