"""The scale sweep divides each weight by a candidate's mantissa scale with a
reciprocal and two fused multiply-adds instead of a full IEEE division
sequence.  Markstein's theorem says the result is still the correctly
rounded quotient (no overflow, normal result); this test checks the same
sequence on the host CPU against IEEE division over every significand of
the divisor and 20M random pairs in the exponent range the sweep uses."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_fma_division_is_correctly_rounded():
    src = os.path.join(HERE, "c", "div_rn_check.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "div_rn_check")
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-o", exe, src, "-lm"],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    bad, n = int(out[0]), int(out[1])
    assert n > 60_000_000
    assert bad == 0, "%d of %d quotients differ from IEEE division" % (bad, n)
