"""Shared test plumbing: seeded inputs (from ``workloads``) copied to the GPU,
calls through the C ABI, oracle runs, and the comparison metric.

The HIP side is reached only through ``memory_efficient_long_amd`` (ctypes over
libbpt.so); the oracle side only through ``oracle``. Nothing here computes any
part of the layer.
"""
from __future__ import annotations

import numpy as np

import workloads as wl

# Parity bars (relative L2 per tensor, computed in float64).
TOL = {"f32": 1e-5, "bf16": 1e-2}


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


class Inputs:
    """Seeded host tensors for one workload (storage-rounded values)."""

    def __init__(self, sh: wl.LayerShape, dy_rows=None, bias_std=0.0, norm_std=0.0):
        self.sh = sh
        self.x = wl.make_x(sh)
        self.w = wl.make_weights(sh, bias_std=bias_std, norm_std=norm_std)
        self.dy = wl.make_dy(sh, rows=dy_rows)
        self.dy_rows = dy_rows

    def oracle_weights(self):
        return {k: v.f64() for k, v in self.w.items()}


def to_device(t: wl.Tensor, device="cuda"):
    import torch
    if t.dtype == "bf16":
        host = torch.from_numpy(t.storage.view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(t.storage)
    return host.to(device).contiguous()


def to_host64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(inp: Inputs, backward=True, cfg=None, device="cuda"):
    """Forward (and backward) through the C ABI. Returns float64 numpy results."""
    import torch
    import memory_efficient_long_amd as bpt
    cfg = cfg or bpt.LayerConfig.from_shape(inp.sh)
    x = to_device(inp.x, device)
    w = {k: to_device(v, device) for k, v in inp.w.items()}
    y, saved = bpt.forward(cfg, x, w)
    out = {"y": y}
    if backward:
        dy = to_device(inp.dy, device)
        dx, grads = bpt.backward(cfg, x, w, saved, dy)
        out["dx"] = dx
        out["grads"] = grads
    torch.cuda.synchronize()
    res = {"y": to_host64(out["y"])}
    if backward:
        res["dx"] = to_host64(out["dx"])
        res["grads"] = {k[1:]: to_host64(v) for k, v in out["grads"].items()}
    return res


def run_oracle(inp: Inputs, backward=True, rows=None):
    from oracle import bpt_oracle as orc
    sp = orc.spec_of(inp.sh)
    x = inp.x.f64()
    w = inp.oracle_weights()
    dy = None
    if backward:
        dy = inp.dy.f64()
        if rows is not None:
            dy = dy[:, rows]
    return orc.layer(x, w, sp, dy=dy, rows=rows)


def compare(gpu, ref, dtype, rows=None, residual_x=None, dy=None):
    """Per-tensor relative L2 of every output; returns {name: err}."""
    errs = {}
    gy = gpu["y"] if rows is None else gpu["y"][:, rows]
    errs["y"] = rel_l2(gy, ref["y"])
    if residual_x is not None:
        rx = residual_x if rows is None else residual_x[:, rows]
        errs["y-x"] = rel_l2(gy - rx, ref["y"] - rx)
    if "dx" in ref:
        errs["dx"] = rel_l2(gpu["dx"], ref["dx"])
        if dy is not None:
            errs["dx-dy"] = rel_l2(gpu["dx"] - dy, ref["dx"] - dy)
        for k, v in ref["grads"].items():
            errs["d" + k] = rel_l2(gpu["grads"][k], v)
    return errs
