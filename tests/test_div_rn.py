"""Host check of the reciprocal-and-FMA division that the fp8 tiled GEMMs use
when they requantise h per 128 columns (expert_ffn_layer_gemm_amd/csrc/common.hpp,
div_rn_by): against IEEE fp32 division, bit for bit wherever the e4m3 code can
depend on it (tests/csrc/div_rn_check.c states the cases)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_division_matches_ieee(tmp_path):
    exe = tmp_path / "div_rn_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "csrc", "div_rn_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    r = subprocess.run([str(exe), "1000000"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
