"""The binding on the GPU when the library is loaded before torch is imported:
it must bind to the HIP runtime torch uses (one runtime in the process), so
that a call on torch's tensors and stream succeeds. Run in a child process,
where nothing has imported torch yet."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {root!r})
import w8a8_fp8_linear_amd as w8
w8.lib()
import torch
x = torch.ones(4, 256, dtype=torch.bfloat16, device="cuda")
q, s = w8.quantize_per_token(x)
torch.cuda.synchronize()
# every row is all ones: scale fl32(1 / 448), every code 448 (0x7E)
assert torch.all(q.cpu() == 0x7E), q
assert torch.all(s.cpu() == torch.tensor(1.0 / 448.0, dtype=torch.float32)), s
print("ok")
"""


def test_library_loaded_before_torch():
    print("[binding] library loaded before torch, child process", flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-2000:] + res.stderr[-3000:]
