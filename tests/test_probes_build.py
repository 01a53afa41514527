"""The measurement probes under tests/probes/ still compile for gfx950 (device and host code, no link, nothing run):
they back figures quoted for the MFMA precision and issue-rate choices, so they must stay buildable from the
current library headers. CPU only (hipcc cross-compiles)."""
import os
import subprocess

import pytest

from long_context_sparse_sa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = ["mfma_fp8_precision.hip", "mfma_shape_rate.hip"]


@pytest.mark.slow
@pytest.mark.parametrize("probe", PROBES)
def test_probe_compiles(probe, tmp_path):
    src = os.path.join(ROOT, "tests", "probes", probe)
    cmd = [B.hipcc(), *B.FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form", "-c", src, "-o", str(tmp_path / "probe.o")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
