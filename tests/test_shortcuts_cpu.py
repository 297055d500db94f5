"""The flush kernels' arithmetic shortcuts, checked on the CPU.

The HIP flush computes the group scale RN(range / L) in three operations and
each code from a Newton-refined reciprocal, falling back to the IEEE
quotient within 2^-16 of a tie (see ``shortcut_check.c``).  Bit-exactness
with the quantizer ([Metal post] "Three ways to be off by one bit") rests on
both; this test runs the exhaustive scale check over every binary32 range in
[2^-24, 2^18) and the sampled near-tie check of the code shortcut, plus
negative controls showing the same checks catch the plain reciprocal
without its correction or its fallback.
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "shortcut_check.c")


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("shortcut") / "shortcut_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall",
                    "-Wextra", "-Werror", "-o", exe, SRC, "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    lines = {}
    for line in res.stdout.splitlines():
        fields = dict(re.findall(r"(\w+)=(\S+)", line))
        head = line.split()[0] if line.split()[0] != "control" else "control " + line.split()[1]
        key = (head, fields.get("bits"), fields.get("meta"))
        lines[key] = fields
    return res.returncode, lines


def test_scale_shortcut_is_the_ieee_quotient_for_every_range(report):
    rc, lines = report
    for bits in ("4", "2"):
        f = lines[("scale", bits, None)]
        # {0} and every binary32 in [2^-24, 2^18): 42 binades of 2^23 values
        assert int(f["checked"]) == 42 * 2 ** 23 + 1
        assert int(f["mismatches"]) == 0


@pytest.mark.parametrize("meta", ["f32", "f16"])
@pytest.mark.parametrize("bits", ["4", "2"])
def test_reciprocal_code_matches_ieee_near_ties(report, bits, meta):
    rc, lines = report
    f = lines[("code", bits, meta)]
    assert int(f["mismatches"]) == 0
    assert int(f["lemma_violations"]) == 0
    assert float(f["worst_gap"]) < 2.0 ** -17
    # both branches are exercised in quantity
    assert int(f["taken"]) > 10 ** 7 and int(f["fallback"]) > 10 ** 7


def test_negative_controls_fail(report):
    rc, lines = report
    assert rc == 0
    assert int(lines[("control scale_without_correction", None, None)]["mismatches"]) > 0
    assert int(lines[("control code", "4", "f32")]["mismatches"]) > 0
