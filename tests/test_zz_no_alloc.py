"""The allocation-free forward (bpt_layer_forward_noalloc: the library's static
device scratch instead of a caller workspace) against the workspace forward
(bpt_layer_forward), through the C ABI: two calls in a row, the second with a
smaller layer, so the second runs on scratch that still holds the first
call's contents. Both paths run the same kernels on the same inputs, so y and
the saved state must agree bit for bit; y is also held to the oracle bar."""
import sys

import numpy as np
import pytest

import workloads as wl
from harness import TOL, Inputs, rel_l2, run_oracle, to_device, to_host64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_forward_matches_workspace_forward():
    import memory_efficient_long_amd as bpt
    bpt.load_library()
    cap = bpt.bpt_layer_noalloc_scratch_bytes()
    for name in ["llama8b-small", "bf16-d64-gqa-rope"]:   # second: smaller scratch use
        sh = wl.SMALL[name]
        cfg = bpt.LayerConfig.from_shape(sh)
        d = cfg.desc()
        need = bpt.bpt_layer_workspace_size(d, False)
        _say(f"[noalloc] {name}: forward scratch {need} of {cap} bytes")
        assert 0 < need <= cap
        inp = Inputs(sh, norm_std=0.2)
        x = to_device(inp.x)
        w = {k: to_device(v) for k, v in inp.w.items()}
        y_ref, saved_ref = bpt.forward(cfg, x, w)
        y = torch.full_like(y_ref, float("nan"))
        saved = torch.zeros_like(saved_ref)
        st = bpt.bpt_layer_forward_noalloc(d, x, w, y, saved)
        assert st == 0, bpt.bpt_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        assert torch.equal(saved[:bpt.bpt_layer_saved_size(d)],
                           saved_ref[:bpt.bpt_layer_saved_size(d)])
        err = rel_l2(to_host64(y), run_oracle(inp, backward=False)["y"])
        _say(f"  y rel L2 vs oracle {err:.2e}")
        assert err <= TOL[sh.dtype]


def test_noalloc_forward_refuses_layers_beyond_the_scratch():
    import memory_efficient_long_amd as bpt
    sh = wl.WORKLOADS["gpt1b-s8k"]
    cfg = bpt.LayerConfig.from_shape(sh)
    d = cfg.desc()
    assert bpt.bpt_layer_workspace_size(d, False) > bpt.bpt_layer_noalloc_scratch_bytes()
    x = torch.zeros(sh.batch, sh.seq_len, sh.hidden, dtype=torch.bfloat16, device="cuda")
    w = {k: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
         for k, s in wl.weight_shapes(sh).items()}
    y = torch.full_like(x, 3.0)
    saved = torch.zeros(bpt.bpt_layer_saved_size(d), dtype=torch.uint8, device="cuda")
    st = bpt.bpt_layer_forward_noalloc(d, x, w, y, saved)
    torch.cuda.synchronize()
    assert st == 2 and "static scratch" in bpt.bpt_last_error()
    assert torch.all(y == 3.0)
