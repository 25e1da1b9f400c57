"""Host build of the HIP library's own fp64 exp2 and of the fp32 streaming pass's
table method (2^(a/256) from a table of 2^(j/256) and a degree-2 series), checked
against libm's long-double exp2 (CPU only; needs hipcc, not a GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_exp2_f64_accuracy(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = str(tmp_path / "exp2_check")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "speculative_sampling_verify_02_amd", "csrc"),
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "native", "exp2_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    max_ulp, mean_rel, n = float(out[0]), float(out[1]), int(out[2])
    assert n > 3_000_000
    assert max_ulp < 2.0, max_ulp
    assert abs(mean_rel) < 1e-16, mean_rel
    assert out[3] == "0" and out[4] in ("nan", "-nan") and out[5] == "1"
    # the table method: truncation of the degree-2 series at |r ln2 / 256| <= ln2 / 512
    # is (ln2 / 512)^3 / 6 = 4.2e-10 relative; the table entries add ~1e-16
    tab_max_rel, tab_n = float(out[6]), int(out[7])
    assert tab_n == 2_000_000
    assert tab_max_rel < 4.5e-10, tab_max_rel
