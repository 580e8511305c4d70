"""The binding must share torch's HIP runtime whatever the import order."""
import subprocess
import sys

import pytest


@pytest.mark.gpu
def test_library_first_then_torch_runs_on_gpu():
    code = (
        "import exact_attention_14_amd as fa\n"
        "import torch\n"
        "q = torch.randn(1, 1, 64, 64, device='cuda', dtype=torch.bfloat16)\n"
        "o, l = fa.fwd(q, q, q)\n"
        "torch.cuda.synchronize()\n"
        "print('ok', bool(torch.isfinite(o.float()).all()))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "ok True" in r.stdout
