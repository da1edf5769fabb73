"""Host check of the kernels' fp64 exponentials (specv_math.h), built with g++.

The draw sums fp64 exps of (z - max)/T. A relative error e in them moves the
draw's CDF edges by about e of the mass, so a draw flips only when u*S lies
within that of an edge: about 2e per token with weight above it, 2.6e-8 per
draw for e = 1e-13 at 1.3e5 tokens, against an allowed 1e-4 of cases (and each
such flip has a margin far below 1e-5). The header states 1e-13 for the
polynomial form (the decision's ratio) and 2.5e-13 for the table form (the
draw), whose table entries are correctly rounded.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_specv_amd", "csrc")


@pytest.fixture(scope="module")
def exp_report(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("exp") / "exp_check"
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "native", "exp_check.cpp"),
                    "-o", str(out), "-lm"], check=True)
    text = subprocess.run([str(out)], check=True, capture_output=True, text=True).stdout
    return dict(line.split(None, 1) for line in text.strip().splitlines())


@pytest.mark.parametrize("form,bound", [("", 1e-13), ("tab_", 2.5e-13)])
def test_relative_error_bound(exp_report, form, bound):
    assert float(exp_report[form + "max_rel_err"].split()[0]) < bound


@pytest.mark.parametrize("form", ["", "tab_"])
def test_special_values(exp_report, form):
    assert float(exp_report[form + "exp0"]) == 1.0
    assert float(exp_report[form + "exp_minus_inf"]) == 0.0
    assert float(exp_report[form + "exp_nan"]) == 0.0
    assert float(exp_report[form + "exp_below"]) == 0.0
    assert float(exp_report[form + "exp_far_below"]) == 0.0


@pytest.mark.parametrize("form,bound", [("", 2.0e-323), ("tab_", 6.0e-321)])
def test_subnormal_range(exp_report, form, bound):
    # Below -708 the results are subnormal or tiny normals: the polynomial form
    # stays within a few units of the smallest subnormal (4.9e-324) of the
    # exact value, the table form within its relative bound of the largest of
    # them (2.5e-13 * 2.2e-308).
    assert float(exp_report[form + "subnormal_abs_err"].split()[0]) <= bound


def test_table_correctly_rounded(exp_report):
    assert float(exp_report["table_max_ulp"]) <= 0.5
