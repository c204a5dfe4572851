"""GPU parity of the layer stack with checkpointing every k layers (through
the C ABI) against the float64 oracle's stack (oracle.bpt_oracle.stack).

* Three bf16 layers (GPT-1B family, reduced) for k in {0, 1, 2, 3}: every
  schedule gives the same bits (the rebuilt segments recompute the same
  values) and matches the oracle per tensor and per row / tile.
* Two fp32 layers against the oracle at the fp32 bar.
* The reinforcement-learning small-hidden shape (3 layers, h = 128, one head):
  at s = 8000 against the oracle; at its full s = 128000 the schedules agree
  bit for bit and the values are finite.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from harness import TOL, compare, over_bar, to_device, to_host64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(sh, L, k, ws_host, x_host, dy_host):
    import memory_efficient_long_amd as bpt
    cfg = bpt.StackConfig(bpt.LayerConfig.from_shape(sh), L, k)
    x = to_device(x_host)
    ws = [{n: to_device(v) for n, v in w.items()} for w in ws_host]
    y, saved = bpt.stack_forward(cfg, x, ws)
    dx, grads = bpt.stack_backward(cfg, x, ws, saved, to_device(dy_host))
    torch.cuda.synchronize()
    return y, dx, grads


def _oracle(sh, ws_host, x_host, dy_host):
    from oracle import bpt_oracle as orc
    return orc.stack(x_host.f64(), [{n: v.f64() for n, v in w.items()} for w in ws_host],
                     orc.spec_of(sh), dy=dy_host.f64())


def _check_vs_oracle(sh, gpu, ref, x_host, dy_host):
    y, dx, grads = gpu
    res = {"y": to_host64(y), "dx": to_host64(dx)}
    errs = compare({**res, "grads": {}}, {"y": ref["y"], "dx": ref["dx"], "grads": {}}, sh.dtype,
                   dy=dy_host.f64())
    for li, g in enumerate(grads):
        for name, v in g.items():
            e = compare({"y": res["y"], "dx": res["dx"], "grads": {name[1:]: to_host64(v)}},
                        {"y": ref["y"], "dx": ref["dx"], "grads": {name[1:]: ref["grads"][li][name[1:]]}},
                        sh.dtype)
            errs[f"L{li}.{name}"] = e[name]
            errs[f"L{li}.{name}@tile"] = e[name + "@tile"]
    return errs


def test_stack_bf16_checkpoint_schedules_match_oracle():
    sh = wl.SMALL["gpt1b-small"]
    L = 3
    ws_host = wl.make_stack_weights(sh, L, bias_std=0.2, norm_std=0.2)
    x_host, dy_host = wl.make_x(sh), wl.make_dy(sh)
    ref = _oracle(sh, ws_host, x_host, dy_host)
    base = None
    for k in (0, 1, 2, 3):
        _say(f"[stack] {sh.name} L={L} k={k}")
        out = _run(sh, L, k, ws_host, x_host, dy_host)
        if base is None:
            base = out
            errs = _check_vs_oracle(sh, out, ref, x_host, dy_host)
            _say(f"  errs { {e: f'{v:.2e}' for e, v in errs.items()} }")
            bad = over_bar(errs, sh.dtype)
            assert not bad, bad
        else:
            assert torch.equal(out[0], base[0]) and torch.equal(out[1], base[1]), k
            for ga, gb in zip(out[2], base[2]):
                for n in ga:
                    assert torch.equal(ga[n], gb[n]), (k, n)


def test_stack_fp32_matches_oracle():
    sh = wl.SMALL["gpt-small-fp32-ragged"]
    L = 2
    ws_host = wl.make_stack_weights(sh, L, bias_std=0.2, norm_std=0.2)
    x_host, dy_host = wl.make_x(sh), wl.make_dy(sh)
    ref = _oracle(sh, ws_host, x_host, dy_host)
    errs = _check_vs_oracle(sh, _run(sh, L, 1, ws_host, x_host, dy_host), ref, x_host, dy_host)
    _say(f"[stack fp32] errs { {e: f'{v:.2e}' for e, v in errs.items()} }")
    bad = over_bar(errs, sh.dtype)
    assert not bad, bad


@pytest.mark.timeout(900)
def test_rl_small_hidden_stack():
    L = wl.RL_SMALL_H_LAYERS
    red = wl.RL_SMALL_H.replace(name="rl-small-h-s8k", seq_len=8000)
    ws_host = wl.make_stack_weights(red, L, bias_std=0.2, norm_std=0.2)
    x_host, dy_host = wl.make_x(red), wl.make_dy(red)
    _say(f"[rl] {red.name} L={L} s={red.seq_len} h={red.hidden}")
    ref = _oracle(red, ws_host, x_host, dy_host)
    errs = _check_vs_oracle(red, _run(red, L, 1, ws_host, x_host, dy_host), ref, x_host, dy_host)
    _say(f"  errs { {e: f'{v:.2e}' for e, v in errs.items()} }")
    bad = over_bar(errs, red.dtype)
    assert not bad, bad
    full = wl.RL_SMALL_H
    _say(f"[rl] {full.name} L={L} s={full.seq_len}: schedules k = 1 and 3 agree")
    ws_full = wl.make_stack_weights(full, L)
    x_full, dy_full = wl.make_x(full), wl.make_dy(full)
    a = _run(full, L, 1, ws_full, x_full, dy_full)
    b = _run(full, L, 3, ws_full, x_full, dy_full)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert bool(torch.isfinite(a[0].float()).all()) and bool(torch.isfinite(a[1].float()).all())
