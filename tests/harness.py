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
# Local bars, as a multiple of the tensor bar: the error of every row of y and
# dx (and of their non-residual parts), and of every 32 x 32 tile of a weight
# gradient (32-element segment of a vector), divided by the norm an average
# row / tile of the reference has (||ref|| * sqrt(block size / tensor size)).
# A wrong row or tile has a local error of order one; for a single head's
# attention tile feeding a row through the projections, about
# 1 / sqrt(3 heads-worth of terms) or more, far above LOCAL_FACTOR x TOL.
LOCAL_FACTOR = 5.0
TILE = 32


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def local_max(got, ref, rowwise: bool) -> float:
    """Largest block error relative to the norm of an average reference block.
    rowwise: blocks are the rows of [..., h] (y, dx); otherwise 32 x 32 tiles of
    a matrix or 32-element segments of a vector (padded with zeros)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    if rowwise:
        d2 = diff.reshape(-1, diff.shape[-1])
        num = np.sqrt((d2 * d2).sum(axis=1))
        nblk, bsz = d2.shape[0], d2.shape[1]
    else:
        if diff.ndim == 1:
            diff = diff[None, :]
        m, n = diff.shape
        pm, pn = -m % TILE if m > 1 else 0, -n % TILE
        dp = np.pad(diff, ((0, pm), (0, pn)))
        bm = TILE if m > 1 else 1
        blk = dp.reshape(dp.shape[0] // bm, bm, dp.shape[1] // TILE, TILE)
        num = np.sqrt((blk * blk).sum(axis=(1, 3))).ravel()
        nblk, bsz = num.size, bm * TILE
    den = np.linalg.norm(ref) * np.sqrt(bsz / max(ref.size, 1))
    if den == 0.0:
        return 0.0 if num.max(initial=0.0) == 0.0 else float("inf")
    return float(num.max(initial=0.0) / den)


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


def compare(gpu, ref, dtype, rows=None, residual_x=None, dy=None, local=True):
    """Per-tensor relative L2 of every output, {name: err}; with ``local``
    also the largest row / tile error, under "name@row" / "name@tile"."""
    errs = {}

    def put(name, got, want, rowwise):
        errs[name] = rel_l2(got, want)
        if local:
            errs[name + ("@row" if rowwise else "@tile")] = local_max(got, want, rowwise)

    gy = gpu["y"] if rows is None else gpu["y"][:, rows]
    put("y", gy, ref["y"], True)
    if residual_x is not None:
        rx = residual_x if rows is None else residual_x[:, rows]
        put("y-x", gy - rx, ref["y"] - rx, True)
    if "dx" in ref:
        put("dx", gpu["dx"], ref["dx"], True)
        if dy is not None:
            put("dx-dy", gpu["dx"] - dy, ref["dx"] - dy, True)
        for k, v in ref["grads"].items():
            put("d" + k, gpu["grads"][k], v, False)
    return errs


def over_bar(errs, dtype, bars=None):
    """{name: err} of every entry above its bar: TOL[dtype] per tensor,
    LOCAL_FACTOR x that per row / tile; ``bars`` overrides the tensor bar by
    name (the local bar follows it)."""
    bad = {}
    for k, v in errs.items():
        base = k.split("@")[0]
        bar = (bars or {}).get(base, TOL[dtype])
        if "@" in k:
            bar *= LOCAL_FACTOR
        if not v <= bar:
            bad[k] = (v, bar)
    return bad
