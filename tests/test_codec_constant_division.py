"""The prompt packer divides the codec's range by 2^b - 1 as a product with
the rounded reciprocal plus one fma correction.  This checks, for every fp32
range in [0, 2^17] and b = 8, 4, 2, 1 (the widths of the tier codec
variants), that the result equals the IEEE quotient
(the definition the oracle uses) bit for bit."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_constant_division_equals_ieee_for_every_range(tmp_path):
    exe = str(tmp_path / "div_by_const")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "exhaustive", "div_by_const.c"), "-lm"], check=True)
    procs = [subprocess.Popen([exe, str(q)], stdout=subprocess.PIPE, text=True) for q in (255, 15, 3, 1)]
    for q, p in zip((255, 15, 3, 1), procs):
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0 and out.strip() == "0", f"divisor {q}: {out.strip()} values differ"
