"""The NA2D gradient oracle against its pins, and planted mistakes in a copy
of its source that some pin must catch.  CPU only."""
import os

import pytest

import oracle
import pins_bwd


@pytest.mark.parametrize("pin", pins_bwd.ALL_PINS_BWD, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default_bwd())


MUTANTS = {
    "softmax_grad_drops_delta": ("ds[e] = p[e] * (ds[e] - go);", "ds[e] = p[e] * ds[e];"),
    "dq_unscaled": ("dq[iq * d + t] += ds[e] * kk[j * d + t] * scale;",
                    "dq[iq * d + t] += ds[e] * kk[j * d + t];"),
    "dq_uses_values": ("dq[iq * d + t] += ds[e] * kk[j * d + t] * scale;",
                       "dq[iq * d + t] += ds[e] * v[j * d + t] * scale;"),
    "dk_uses_weights": ("dk[j * d + t] += ds[e] * qi[t] * scale;",
                        "dk[j * d + t] += p[e] * qi[t] * scale;"),
    "dv_uses_softmax_grad": ("dv[j * d + t] += p[e] * gi[t];", "dv[j * d + t] += ds[e] * gi[t];"),
    "drpb_axes_swapped": ("drpb_map[(sy + a - y + k - 1) * nb + (sx + c - x + k - 1)] += ds[e] * scale;",
                          "drpb_map[(sx + c - x + k - 1) * nb + (sy + a - y + k - 1)] += ds[e] * scale;"),
    "drpb_sign": ("drpb_map[(sy + a - y + k - 1) * nb + (sx + c - x + k - 1)] += ds[e] * scale;",
                  "drpb_map[(y - sy - a + k - 1) * nb + (x - sx - c + k - 1)] += ds[e] * scale;"),
    "weights_not_normalised": ("for (int e = 0; e < n; ++e) p[e] /= z;",
                               "for (int e = 0; e < n; ++e) p[e] /= 1.0;"),
    "window_off_by_one": ("    int s = i - k / 2;", "    int s = i - k / 2 + 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.BWD_SOURCE).read()
    assert src.count(old) == 1, "mutation site not found: %s" % name
    path = os.path.join(str(tmp_path), "mut_%s.c" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    orc = oracle.OracleBwd(oracle.compile_oracle(path, os.path.join(str(tmp_path), "libmut.so")))
    failed = []
    for pin in pins_bwd.ALL_PINS_BWD:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passes every pin" % name
