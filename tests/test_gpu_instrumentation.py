"""The library's optional instrumentation, switched by environment variables:
BPT_LOG=1 prints each call's plan to stderr, BPT_ROCTX=1 brackets every phase
with a roctx range (recorded by ``rocprofv3 --marker-trace``). Run in a child
process so the switches are read afresh; the results must not change."""
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, hashlib
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import torch
import workloads as wl
from harness import Inputs, run_gpu
sh = wl.SMALL["llama8b-small"]
out = run_gpu(Inputs(sh, norm_std=0.2))
h = hashlib.sha256()
for k in ("y", "dx"):
    h.update(out[k].tobytes())
for k in sorted(out["grads"]):
    h.update(out["grads"][k].tobytes())
print("digest", h.hexdigest(), flush=True)
"""


def _run(env_extra):
    env = dict(os.environ, **env_extra)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    proc = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=300)
    assert proc.returncode == 0, proc.stderr[-3000:]
    digest = [l for l in proc.stdout.splitlines() if l.startswith("digest")]
    assert digest, proc.stdout[-2000:]
    return digest[-1], proc.stderr


def test_log_and_markers_do_not_change_results():
    base, err0 = _run({"BPT_LOG": "0", "BPT_ROCTX": "0"})
    logged, err1 = _run({"BPT_LOG": "1", "BPT_ROCTX": "1"})
    assert logged == base
    assert "[bpt]" not in err0
    assert "[bpt] bpt_layer_forward: b=1 s=656 h=512 heads=4/2 d=128" in err1
    assert "[bpt] bpt_layer_backward:" in err1
