"""Plausible mistakes planted in the oracle must each fail at least one pin.

Each mutant is a textual edit of the oracle's C source, compiled to a
temporary library on the CPU and run through every pin in ``pins.py``. This
shows the pins are not just the oracle agreeing with itself.
"""
import os

import pytest

import oracle

from pins import failing_pins

# (name, original text, replacement); each original must occur in the source.
MUTANTS = [
    ("adjoint_exponent_sign", "const double theta = 2.0 * M_PI * (j->kx[m] * xn",
     "const double theta = -2.0 * M_PI * (j->kx[m] * xn"),
    ("adjoint_missing_two", "const double theta = 2.0 * M_PI * (j->kx[m] * xn",
     "const double theta = M_PI * (j->kx[m] * xn"),
    ("adjoint_dropped_kz", " + j->kz[m] * zn);", ");"),
    ("adjoint_y_z_swapped", "j->ky[m] * yn + j->kz[m] * zn", "j->ky[m] * zn + j->kz[m] * yn"),
    ("adjoint_kx_ky_swapped", "(j->kx[m] * xn + j->ky[m] * yn", "(j->ky[m] * xn + j->kx[m] * yn"),
    ("mac_real_sign", "sum_re += j->in_re[m] * c - j->in_im[m] * s;",
     "sum_re += j->in_re[m] * c + j->in_im[m] * s;"),
    ("mac_imag_operand", "sum_im += j->in_re[m] * s + j->in_im[m] * c;",
     "sum_im += j->in_im[m] * s + j->in_re[m] * c;"),
    ("sin_cos_swapped", "const double c = cos(theta), s = sin(theta);\n            /* (D_re",
     "const double c = sin(theta), s = cos(theta);\n            /* (D_re"),
    ("last_sample_dropped", "for (long m = 0; m < j->M; ++m) {\n            const double theta",
     "for (long m = 0; m + 1 < j->M; ++m) {\n            const double theta"),
    ("forward_exponent_sign", "sum_re += j->in_re[n] * c + j->in_im[n] * s;",
     "sum_re += j->in_re[n] * c - j->in_im[n] * s;"),
    ("forward_imag_sign", "sum_im += j->in_im[n] * c - j->in_re[n] * s;",
     "sum_im += j->in_im[n] * c + j->in_re[n] * s;"),
    ("accumulator_not_reset", "double sum_re = 0.0, sum_im = 0.0;\n        for (long m",
     "static __thread double sum_re = 0.0, sum_im = 0.0;\n        for (long m"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, "mutation site not unique/absent: %s" % name
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(source.replace(old, new))
    lib_path = str(tmp_path / ("libmut_%s.so" % name))
    oracle.build(str(src), lib_path)
    lib = oracle.load(lib_path)
    bad = failing_pins(lib)
    assert bad, "mutant %s passed every pin" % name


def test_unmutated_source_passes_every_pin(tmp_path):
    lib_path = str(tmp_path / "libclean.so")
    oracle.build(oracle.SOURCE, lib_path)
    assert failing_pins(oracle.load(lib_path)) == []
    assert os.path.exists(lib_path)
