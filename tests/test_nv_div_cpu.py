"""CPU check of the NVFP4-style quantizers' quotient (csrc/nv_div.h: one
reciprocal per block, then two fma corrections) against IEEE fp32 division,
bit for bit: the header's sequence is compiled with g++ and run over the
divisors d = dec(S) s_g of every E4M3 code and many tensor scales, with zeros,
subnormals, quotients within a few ulps of every E2M1 decision point and
random quotients (tests/nv_div_check.cpp): bit-exact wherever the quotient
is at least 2^-3 in magnitude, and the same E2M1 code everywhere (a
subnormal x can make the remainder underflow, and the last bits of a tiny
quotient then differ). The plain product x y, without the corrections, must
fail the same check, so the check can tell."""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "fp4_quantized_diffusion_amd", "csrc")


def build_and_run(tmp_path, extra=(), n_sg=400):
    exe = str(tmp_path / ("nv_div_check" + "".join(extra).replace("-", "_")))
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wno-unknown-pragmas",
           f"-I{CSRC}", *extra, os.path.join(HERE, "nv_div_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    out = subprocess.run([exe, str(n_sg)], check=True, capture_output=True, text=True).stdout
    m = re.search(r"cases (\d+) mismatches (\d+) code_mismatches (\d+)", out)
    assert m, out
    return int(m.group(1)), int(m.group(2)), int(m.group(3)), out


def test_quotient_is_ieee_division(tmp_path):
    """Bit-exact wherever |x / d| >= 2^-3 (where a code can be non-zero), the
    same E2M1 code everywhere."""
    cases, bad, bad_code, out = build_and_run(tmp_path)
    assert cases > 10_000_000, out
    assert bad == 0 and bad_code == 0, out


def test_uncorrected_product_is_caught(tmp_path):
    cases, bad, bad_code, out = build_and_run(tmp_path, ("-DPLANT_NO_CORRECTION",), n_sg=40)
    assert bad > 0, out
