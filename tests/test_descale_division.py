"""The fp8 KV append divides by the per-tensor descale with one exact
reciprocal and an FMA correction instead of a division per element.  This
host check (C, gcc, contraction off) runs that arithmetic over every bf16
value for powers of two near every exponent of 2^-60 .. 2^60, their
neighbours and random descales of that range, and requires the E4M3 code of
every quotient to equal that of the IEEE quotient (and the binary32
quotient itself wherever it is at least 2^-10).  The GPU append tests check
the kernel's codes against the oracle."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_division_matches_ieee(tmp_path):
    exe = str(tmp_path / "descale_division_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "native", "descale_division_check.c"), "-lm"], check=True)
    r = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "0 mismatches" in r.stdout
