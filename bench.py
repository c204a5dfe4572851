#!/usr/bin/env python3
"""Benchmark of the fused Blockwise Parallel Transformer layer on one MI355X.

One step = forward + recompute-based backward of one layer over one batch of
seeded synthetic input, everything resident in HBM before the timed region.
Default workload: the GPT-1B-shaped layer at s = 131072 (h = 2048, 16 heads x
128, GeLU FFN 8192, bf16 storage with fp32 accumulation, query block 2048,
KV block 4096).

Prints ONE JSON line: tokens/s (the metric), ms/step, model TFLOP/s and the
fraction of the bf16 MFMA peak, the roofline of the dominant kernel (timed live
with HIP events on the launch stream by the library's timing hooks), bytes per
token kept for the backward, and the CPU oracle timed on the host's cores on a
bounded sample (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def attn_pairs(s: int, causal: bool, window: int = 0) -> int:
    """Visible (query, key) pairs per head: causal rows see i + 1 keys, or
    min(i + 1, W) with a sliding window W."""
    if not causal:
        return s * s
    if window and window < s:
        return window * (window + 1) // 2 + (s - window) * window
    return s * (s + 1) // 2


def model_flops(sh) -> dict:
    """Model FLOPs of one layer (multiply-add = 2), causal attention counted on
    the visible pairs only; a step is forward + backward = 3 x forward."""
    s, h, H, Hkv, d, f = sh.seq_len, sh.hidden, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.ffn_dim
    n_ffn = 3 if sh.ffn == "swiglu" else 2
    lin = 2 * s * h * (H + 2 * Hkv) * d + 2 * s * H * d * h + 2 * s * h * f * n_ffn
    w = getattr(sh, "window", 0)
    attn = 4 * d * H * attn_pairs(s, sh.causal, w)
    fwd = (lin + attn) * sh.batch
    pairs = attn_pairs(s, sh.causal, w) * sh.batch
    return {"fwd": fwd, "step": 3 * fwd,
            # attention units (see ROOFLINE_UNITS): forward QK^T and PV, 4d per
            # visible pair and head; backward dV, dP, dK and dQ, 8d
            "attn_fwd": 4 * d * H * pairs, "attn_bwd": 8 * d * H * pairs,
            # what the kernels run, with the recomputed products: the forward
            # 4d; dK/dV recomputes S (+2d); the dQ pass recomputes S and dP (+4d)
            "hw_attn_fwd": 4 * d * H * pairs, "hw_attn_bwd": 14 * d * H * pairs}


# Roofline units: the attention forward kernel alone, and the attention
# backward as the pair of kernels it is split into (dK/dV pass, then dQ pass).
ROOFLINE_UNITS = {"attn_fwd": ["attn_fwd"], "attn_bwd": ["attn_bwd_dkdv", "attn_bwd_dq"]}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def gpu_sysfs_dir(dev):
    """sysfs directory of the device (found by its PCI address), or None where
    the device's clock table is not readable."""
    try:
        import torch
        p = torch.cuda.get_device_properties(dev)
        bus = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    except Exception:
        return None
    d = os.path.join("/sys/bus/pci/devices", bus)
    return d if os.access(os.path.join(d, "pp_dpm_sclk"), os.R_OK) else None


def parse_sclk(text: str):
    """Current shader clock in MHz from a pp_dpm_sclk table (the starred
    level, e.g. "1: 2400Mhz *"), or None."""
    import re
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
            if m:
                return float(m.group(1))
    return None


class ClockSampler:
    """Reads the device's current shader clock from sysfs every `period` s on
    a host thread while the timed steps run (default clocks and power; the
    reading is what the driver reports, logged beside the timing)."""

    def __init__(self, dev, period: float = 0.05):
        import threading
        self.dir = gpu_sysfs_dir(dev)
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True) if self.dir else None

    def _run(self):
        path = os.path.join(self.dir, "pp_dpm_sclk")
        while not self._stop.is_set():
            try:
                with open(path) as fh:
                    v = parse_sclk(fh.read())
            except OSError:
                return
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self._thr:
            self._thr.start()
        return self

    def __exit__(self, *exc):
        if self._thr:
            self._stop.set()
            self._thr.join()

    def summary(self):
        if not self.samples:
            return None
        v = self.samples
        return {"source": "sysfs pp_dpm_sclk", "samples": len(v), "mean_mhz": round(sum(v) / len(v), 1),
                "min_mhz": min(v), "max_mhz": max(v)}


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from memory_efficient_long_amd.profiling import kernel_source_hash
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(sh, sample_len: int) -> dict:
    """Time the CPU oracle (float64, all host BLAS threads) on the same layer
    at a shorter sequence and scale its model-FLOP rate to tokens/s of the full
    workload."""
    import numpy as np
    import workloads as wl
    from oracle import bpt_oracle as orc
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    samp = sh.replace(seq_len=sample_len, q_block=sample_len, kv_block=sample_len)
    x = wl.make_x(samp).f64()
    w = {k: v.f64() for k, v in wl.make_weights(samp).items()}
    dy = wl.make_dy(samp).f64()
    t0 = time.perf_counter()
    orc.layer(x, w, orc.spec_of(samp), dy=dy)
    dt = time.perf_counter() - t0
    rate = model_flops(samp)["step"] / dt
    full = model_flops(sh)
    tokens_per_s = rate / (full["step"] / (sh.seq_len * sh.batch))
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"float64 oracle forward+backward of the same layer at s={sample_len} "
                       f"({dt:.1f} s, {rate / 1e9:.1f} GFLOP/s); model-FLOP rate scaled to the "
                       f"per-token FLOPs at s={sh.seq_len}")}


def _peak_activation_bytes(sh) -> dict:
    """One forward + backward of the layer with torch-allocated saved buffer
    and workspaces; returns the library's exact sizes and torch's peak
    allocation above what was live before (inputs, weights, gradients, y, dx)."""
    import numpy as np
    import torch
    import memory_efficient_long_amd as bpt
    import workloads as wl
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn(sh.batch, sh.seq_len, sh.hidden, device=dev, generator=gen).to(dt)
    w = {k: (torch.randn(s, device=dev, generator=gen) * 0.02).to(dt)
         for k, s in wl.weight_shapes(sh).items()}
    dy = torch.randn_like(x)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    cfg = bpt.LayerConfig.from_shape(sh)
    grads = {k: torch.empty(s, dtype=torch.float32, device=dev)
             for k, s in bpt.grad_shapes(cfg, w).items()}
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    _, saved = bpt.forward(cfg, x, w, y=y)
    bpt.backward(cfg, x, w, saved, dy, dx=dx, grads=grads)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev) - base
    d = cfg.desc()
    lib = (bpt.bpt_layer_saved_size(d) + max(bpt.bpt_layer_workspace_size(d, False),
                                              bpt.bpt_layer_workspace_size(d, True)))
    del saved, x, w, dy, y, dx, grads
    torch.cuda.empty_cache()
    return {"s": sh.seq_len, "head_chunk": sh.head_chunk, "library_bytes": lib,
            "torch_peak_bytes": int(peak)}


def memory_sweep() -> int:
    """Peak activation memory over s at the GPT-1B shape (affine fit) and
    over the head chunk at the Llama-8B shape."""
    import numpy as np
    import workloads as wl
    base = wl.WORKLOADS["gpt1b-s128k"]
    pts = []
    for s in (16384, 32768, 65536, 131072):
        print(f"[memory] gpt1b s={s}", file=sys.stderr, flush=True)
        pts.append(_peak_activation_bytes(base.replace(seq_len=s)))
    ss = np.array([p["s"] for p in pts], dtype=np.float64)
    fit = {}
    for key in ("library_bytes", "torch_peak_bytes"):
        v = np.array([p[key] for p in pts], dtype=np.float64)
        slope, icpt = np.polyfit(ss, v, 1)
        resid = np.max(np.abs(v - (slope * ss + icpt)) / v)
        fit[key] = {"bytes_per_token": round(slope, 1),
                    "sbh_per_token": round(slope / base.hidden, 3),
                    "intercept_bytes": round(icpt), "max_rel_residual": float(resid)}
    chunks = []
    llama = wl.WORKLOADS["llama8b-s64k"]
    for u in (4, 8, 16, 32):
        print(f"[memory] llama8b head_chunk={u}", file=sys.stderr, flush=True)
        chunks.append(_peak_activation_bytes(llama.replace(head_chunk=u)))
    stack = []
    st_shape = base.replace(seq_len=16384)
    for k in (0, 1, 2, 4, 8):
        print(f"[memory] gpt1b stack L=8 k={k}", file=sys.stderr, flush=True)
        stack.append(_stack_peak_bytes(st_shape, 8, k))
    print(json.dumps({"memory_sweep": {"gpt1b": pts, "affine_fit": fit,
                                       "llama8b_head_chunk": chunks,
                                       "gpt1b_s16k_stack_L8": stack}}), flush=True)
    return 0


def _stack_peak_bytes(sh, L, k) -> dict:
    """Peak of a stack forward + backward: the library's saved + workspace
    bytes, the checkpoint-every-k prediction (L/k) c + k A with c one
    activation and A one layer's rebuilt input and saved state, and torch's
    peak allocation above the inputs, weights and gradients."""
    import torch
    import memory_efficient_long_amd as bpt
    import workloads as wl
    dev = torch.device("cuda:0")
    cfg = bpt.StackConfig(bpt.LayerConfig.from_shape(sh), L, k)
    d = cfg.desc()
    gen = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn(sh.batch, sh.seq_len, sh.hidden, device=dev, generator=gen).to(torch.bfloat16)
    ws = [{n: (torch.randn(s, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
           for n, s in wl.weight_shapes(sh).items()} for _ in range(L)]
    dy = torch.randn_like(x)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    y, saved = bpt.stack_forward(cfg, x, ws)
    dx, grads = bpt.stack_backward(cfg, x, ws, saved, dy)
    torch.cuda.synchronize()
    gbytes = sum(v.numel() * 4 for g in grads for v in g.values())
    peak = torch.cuda.max_memory_allocated(dev) - base - gbytes - 2 * x.numel() * 2
    lib = bpt.bpt_stack_saved_size(d) + max(bpt.bpt_stack_workspace_size(d, False),
                                            bpt.bpt_stack_workspace_size(d, True))
    c = x.numel() * 2
    A = c + bpt.bpt_layer_saved_size(cfg.layer.desc())
    pred = (L / k * c + k * A) if k else None
    del x, ws, dy, y, saved, dx, grads
    torch.cuda.empty_cache()
    return {"k": k, "library_bytes": lib, "torch_peak_bytes": int(peak),
            "pages_M_k_bytes": pred}


def bench_stack(args, sh, L, k) -> int:
    """One step = forward + backward of a stack of L layers (own weights
    each) with checkpointing every k layers, inputs resident in HBM."""
    import numpy as np
    import torch
    import memory_efficient_long_amd as bpt
    import workloads as wl
    dev = torch.device("cuda:0")

    def to_dev(t):
        if t.dtype == "bf16":
            return torch.from_numpy(t.storage.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.storage).to(dev)

    cfg = bpt.StackConfig(bpt.LayerConfig.from_shape(sh), L, k)
    d = cfg.desc()
    x, dy = to_dev(wl.make_x(sh)), to_dev(wl.make_dy(sh))
    ws = [{n: to_dev(v) for n, v in w.items()} for w in wl.make_stack_weights(sh, L)]
    y, dx = torch.empty_like(x), torch.empty_like(x)
    saved = torch.empty(max(bpt.bpt_stack_saved_size(d), 256), dtype=torch.uint8, device=dev)
    wsf = torch.empty(bpt.bpt_stack_workspace_size(d, False), dtype=torch.uint8, device=dev)
    wsb = torch.empty(bpt.bpt_stack_workspace_size(d, True), dtype=torch.uint8, device=dev)
    grads = [{n: torch.empty(s, dtype=torch.float32, device=dev)
              for n, s in bpt.grad_shapes(cfg.layer, w).items()} for w in ws]
    stream = torch.cuda.current_stream()

    def step():
        st = bpt.bpt_stack_forward(d, x, ws, y, saved, wsf, stream)
        st = st or bpt.bpt_stack_backward(d, x, ws, saved, dy, dx, grads, wsb, False, stream)
        if st:
            raise bpt.BptError(st, "stack")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    attn = ["attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"]
    bpt.bpt_timing_enable(attn)
    bpt.bpt_timing_read(reset=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    timing = bpt.bpt_timing_read(reset=True)
    bpt.bpt_timing_enable([])
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    fl = model_flops(sh)
    model = L * fl["step"]
    peak = PEAK_BF16_TFLOPS if sh.dtype == "bf16" else PEAK_F32_TFLOPS
    tokens = sh.seq_len * sh.batch
    # the dominant unit, as for one layer (k >= 1 runs each layer's attention
    # forward twice per step)
    unit_ms = {u: sum(timing[c][0] for c in cs) for u, cs in ROOFLINE_UNITS.items()}
    dom = max(unit_ms, key=unit_ms.get)
    n_launch = timing[ROOFLINE_UNITS[dom][0]][1]
    avg_ms = sum(timing[c][0] / max(timing[c][1], 1) for c in ROOFLINE_UNITS[dom])
    achieved = fl[dom] / (avg_ms * 1e-3) / 1e12 if avg_ms > 0 else 0.0
    saved_b = bpt.bpt_stack_saved_size(d)
    peak_b = saved_b + max(wsf.numel(), wsb.numel())
    out = {
        "metric": "BPT layer stack fwd+bwd tokens/s (checkpointing every k layers)",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": sh.name, "n_layers": L, "checkpoint_every": k,
                   "seq_len": sh.seq_len, "hidden": sh.hidden, "n_heads": sh.n_heads,
                   "head_dim": sh.head_dim, "ffn_dim": sh.ffn_dim, "q_block": sh.q_block,
                   "kv_block": sh.kv_block},
        "model_tflops": round(model / (ms * 1e-3) / 1e12, 2),
        "mfma_peak_frac": round(model / (ms * 1e-3) / 1e12 / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": " + ".join(c + "_dma_kernel" for c in ROOFLINE_UNITS[dom]),
                     "avg_launch_ms": round(avg_ms, 3), "launches_per_step": n_launch / args.steps},
        "memory": {"saved_bytes_per_token": saved_b / tokens,
                   "saved_sbh": round(saved_b / (tokens * sh.hidden), 3),
                   "peak_bytes_per_token": peak_b / tokens,
                   "peak_sbh": round(peak_b / (tokens * sh.hidden), 3)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_lm_head(args) -> int:
    """One step = LM-head loss + gradients (dz, dW_head) over all rows, inputs
    resident in HBM: by default the fused call (each chunk's logits computed
    once and kept in fp32 for its dlogits), with --lm-two-calls the forward
    and backward calls (the backward recomputes the logits)."""
    import numpy as np
    import torch
    import memory_efficient_long_amd as bpt
    import workloads as wl
    sh = wl.LM_HEADS[args.workload]
    if args.lm_chunk_rows:
        sh = sh.replace(chunk_rows=args.lm_chunk_rows)
    dev = torch.device("cuda:0")

    def to_dev(t):
        if t.dtype == "bf16":
            return torch.from_numpy(t.storage.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.storage).to(dev)

    cfg = bpt.LmHeadConfig(sh.rows, sh.hidden, sh.vocab, sh.chunk_rows, sh.dtype)
    d = cfg.desc()
    z, w = to_dev(wl.make_z(sh)), to_dev(wl.make_w_head(sh))
    t = torch.from_numpy(wl.make_targets(sh)).to(dev)
    valid = max(int((t >= 0).sum()), 1)
    g = torch.full((sh.rows,), 1.0 / valid, dtype=torch.float32, device=dev)  # mean loss
    loss = torch.empty(sh.rows, dtype=torch.float32, device=dev)
    saved = torch.empty(bpt.bpt_lm_head_saved_size(d), dtype=torch.uint8, device=dev)
    wsf = torch.empty(bpt.bpt_lm_head_workspace_size(d, False), dtype=torch.uint8, device=dev)
    fused = not args.lm_two_calls
    if fused:
        wsf = wsb = torch.empty(bpt.bpt_lm_head_workspace_size(d, 2), dtype=torch.uint8, device=dev)
    else:
        wsb = torch.empty(bpt.bpt_lm_head_workspace_size(d, True), dtype=torch.uint8, device=dev)
    dz = torch.empty_like(z)
    dw = torch.empty(sh.hidden, sh.vocab, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        if fused:
            st = bpt.bpt_lm_head_forward_backward(d, z, w, t, g, loss, saved, dz, dw, wsf,
                                                  False, stream)
        else:
            st = bpt.bpt_lm_head_forward(d, z, w, t, loss, saved, wsf, stream)
            st = st or bpt.bpt_lm_head_backward(d, z, w, t, saved, g, dz, dw, wsb, False, stream)
        if st:
            raise bpt.BptError(st, "lm head")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    bpt.bpt_timing_enable(["lm_head", "rowwise"])
    bpt.bpt_timing_read(reset=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    timing = bpt.bpt_timing_read(reset=True)
    bpt.bpt_timing_enable([])
    step_ms = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.mean(step_ms))
    n, h, V = sh.rows, sh.hidden, sh.vocab
    model = 6 * n * h * V          # logits, dz and dW products (2nhV each)
    hw = (6 if fused else 8) * n * h * V   # two calls: + the logits recomputed
    gm, gn = timing["lm_head"]
    achieved = model / (gm / args.steps * 1e-3) / 1e12 if gm > 0 else 0.0
    peak = PEAK_BF16_TFLOPS if sh.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": "blockwise LM head + cross-entropy fwd+bwd tokens/s",
        "value": round(n / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": sh.name, "rows": n, "hidden": h, "vocab": V,
                   "chunk_rows": sh.chunk_rows,
                   "path": "fused forward+backward" if fused else "forward, then backward"},
        "model_tflops": round(model / (ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": ("gemm_dma_kernel (LM head: logits with the log-sum-exp and "
                                "fp32-logit epilogue, dz, dW)") if fused else
                               ("gemm_dma_kernel (LM head: logits with the log-sum-exp epilogue, "
                                "recomputed logits with the dlogit epilogue, dz, dW)"),
                     "avg_launch_ms": round(gm / max(gn, 1), 3),
                     "launches_per_step": gn / args.steps,
                     "kernel_ms_per_step": round(gm / args.steps, 3),
                     "flops_unit": "6*h*V per row (model)" + ("" if fused else
                                   "; 8*h*V per row run (logits recomputed)"),
                     "hardware_flops_per_step": hw},
        "rowwise_ms_per_step": round(timing["rowwise"][0] / args.steps, 3),
        "memory": {"saved_bytes_per_token": bpt.bpt_lm_head_saved_size(d) / n,
                   "workspace_bytes": max(wsf.numel(), wsb.numel()),
                   "chunk_logits_fp32_bytes_held": 4 * cfg.chunk_rows * V if fused else 0,
                   "logits_fp32_bytes_not_held": 4 * n * V},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import lm_head_oracle as lmo
        rows = min(n, 2048)
        samp = sh.replace(rows=rows)
        zz, ww = wl.make_z(samp).f64(), wl.make_w_head(samp).f64()
        tt = wl.make_targets(samp)
        gg = np.full(rows, 1.0 / rows)
        t0 = time.perf_counter()
        lmo.lm_head_ce(zz, ww, tt, gg)
        dt = time.perf_counter() - t0
        try:
            import threadpoolctl
            threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        out["cpu_baseline"] = {"value": rows / dt, "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"float64 oracle forward+backward on the first {rows} "
                                         f"rows ({dt:.1f} s); rows are independent, so the rate "
                                         f"is per row"}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt1b-s128k")
    ap.add_argument("--head-chunk", type=int, default=0, metavar="U",
                    help="query heads per attention stage (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-len", type=int, default=8192)
    ap.add_argument("--lm-chunk-rows", type=int, default=0,
                    help="LM head: rows per chunk (default: the workload's)")
    ap.add_argument("--lm-two-calls", action="store_true",
                    help="LM head: time the forward and backward calls instead of the fused call")
    ap.add_argument("--breakdown", action="store_true",
                    help="also time GEMM and row-wise kernel classes (adds events)")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="causal sliding window of W keys (local attention)")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="attention dropout probability (masks regenerated in the backward)")
    ap.add_argument("--stack", type=int, default=0, metavar="L",
                    help="time a stack of L layers of the workload's shape instead of one layer")
    ap.add_argument("--checkpoint-every", type=int, default=1, metavar="K",
                    help="stack checkpoint interval (0: keep every layer's saved state)")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="only measure peak activation bytes over s (GPT-1B shape) and head chunk "
                         "(Llama-8B shape) and print one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES (HBM counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy}))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(see DESIGN.md for how the layer would shard).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import memory_efficient_long_amd as bpt
    from memory_efficient_long_amd import accounting as acc
    import workloads as wl

    bpt.load_library()
    if args.memory_sweep:
        return memory_sweep()
    if args.workload in wl.LM_HEADS:
        return bench_lm_head(args)
    if args.workload == wl.RL_SMALL_H.name:
        return bench_stack(args, wl.RL_SMALL_H, args.stack or wl.RL_SMALL_H_LAYERS,
                           args.checkpoint_every)
    if args.stack:
        sh = wl.WORKLOADS[args.workload]
        if args.head_chunk:
            sh = sh.replace(head_chunk=args.head_chunk)
        return bench_stack(args, sh, args.stack, args.checkpoint_every)
    sh = wl.WORKLOADS[args.workload]
    if args.head_chunk:
        sh = sh.replace(head_chunk=args.head_chunk)
    if args.window:
        sh = sh.replace(window=args.window)
    if args.dropout:
        sh = sh.replace(dropout_p=args.dropout, seed=1234)
    cfg = bpt.LayerConfig.from_shape(sh)
    desc = cfg.desc()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(t):
        if t.dtype == "bf16":
            return torch.from_numpy(t.storage.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.storage).to(dev)

    print(f"[bench] generating inputs for {sh.name}", file=sys.stderr, flush=True)
    x = to_dev(wl.make_x(sh))
    w = {k: to_dev(v) for k, v in wl.make_weights(sh).items()}
    dy = to_dev(wl.make_dy(sh))
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    saved_bytes = bpt.bpt_layer_saved_size(desc)
    ws_f_bytes = bpt.bpt_layer_workspace_size(desc, False)
    ws_b_bytes = bpt.bpt_layer_workspace_size(desc, True)
    saved = torch.empty(saved_bytes, dtype=torch.uint8, device=dev)
    ws_f = torch.empty(ws_f_bytes, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(ws_b_bytes, dtype=torch.uint8, device=dev)
    grads = {k: torch.empty(s, dtype=torch.float32, device=dev)
             for k, s in bpt.grad_shapes(cfg, w).items()}
    stream = torch.cuda.current_stream()

    def fwd():
        st = bpt.bpt_layer_forward(desc, x, w, y, saved, ws_f, stream)
        if st:
            raise bpt.BptError(st, "forward")

    def bwd():
        st = bpt.bpt_layer_backward(desc, x, w, saved, dy, dx, grads, ws_b, False, stream)
        if st:
            raise bpt.BptError(st, "backward")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    attn_classes = ["attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"]
    classes = attn_classes + (["gemm", "rowwise"] if args.breakdown else [])
    bpt.bpt_timing_enable(classes)
    bpt.bpt_timing_read(reset=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler(dev) as clocks:
        t0 = time.perf_counter()
        for e0, e1, e2 in evs:
            e0.record(stream)
            fwd()
            e1.record(stream)
            bwd()
            e2.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    timing = bpt.bpt_timing_read(reset=True)
    bpt.bpt_timing_enable([])
    fwd_ms = [a.elapsed_time(b) for a, b, _ in evs]
    bwd_ms = [b.elapsed_time(c) for _, b, c in evs]
    step_ms = [a.elapsed_time(c) for a, _, c in evs]
    ms_per_step = float(np.mean(step_ms))
    print(f"[bench] step {ms_per_step:.2f} ms (wall {wall_ms:.2f}); fwd {np.mean(fwd_ms):.2f} "
          f"bwd {np.mean(bwd_ms):.2f}; timing {timing}", file=sys.stderr, flush=True)

    # Sustained MFMA rate of this device (a register-only MFMA kernel), the
    # practical ceiling next to the datasheet peak.
    practical = bpt.bpt_mfma_peak_probe(stream) if sh.dtype == "bf16" else None

    fl = model_flops(sh)
    tokens = sh.seq_len * sh.batch
    tflops = fl["step"] / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if sh.dtype == "bf16" else PEAK_F32_TFLOPS

    # Dominant unit: the attention forward kernel or the backward pair, by
    # measured time. achieved = the unit's algorithmic FLOPs per launch over
    # the sum of its kernels' average launch durations (HIP events on the
    # launch stream, recorded by the library around each launch).
    unit_ms = {u: sum(timing[c][0] for c in cs) for u, cs in ROOFLINE_UNITS.items()}
    dom = max(unit_ms, key=unit_ms.get)
    kernels = ROOFLINE_UNITS[dom]
    launches = timing[kernels[0]][1] / args.steps          # launches of the unit per step
    avg = {c: timing[c][0] / max(timing[c][1], 1) for c in kernels}
    avg_ms = sum(avg.values())
    per_launch_flops = fl[dom] / max(launches, 1)
    achieved = per_launch_flops / (avg_ms * 1e-3) / 1e12 if avg_ms > 0 else 0.0
    # bf16 with head_dim 64 / 128 runs the direct-to-LDS attention kernels.
    dma = sh.dtype == "bf16" and sh.head_dim in (64, 128)
    names = {c: c + ("_dma_kernel" if dma else "_kernel") for c in kernels}
    traffic = None
    if sh.head_chunk == wl.WORKLOADS[args.workload].head_chunk:  # counters at the default chunk
        parts = [load_traffic(names[c], sh.name) for c in kernels]
        traffic = sum(parts) if all(v is not None for v in parts) else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic,
                "traffic_gb_per_s": (round(traffic / (avg_ms * 1e-3) / 1e9, 1)
                                     if traffic and avg_ms > 0 else None),
                "kernel": " + ".join(names[c] for c in kernels),
                "avg_launch_ms": round(avg_ms, 3),
                "kernel_avg_launch_ms": {names[c]: round(avg[c], 3) for c in kernels},
                "launches_per_step": launches,
                "flops_unit": ("4*d per visible (query, key) pair and head" if dom == "attn_fwd"
                               else "8*d per visible (query, key) pair and head"),
                "algorithmic_flops_per_launch": per_launch_flops,
                "hardware_flops_per_launch": fl["hw_" + dom] / max(launches, 1)}

    breakdown = {c: {"ms_per_step": round(v[0] / args.steps, 3), "launches_per_step": v[1] / args.steps}
                 for c, v in timing.items() if v[1]}
    out = {
        "metric": "fused BPT layer fwd+bwd tokens/s and % MFMA bf16 peak at s=131072",
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": sh.name, "batch": sh.batch, "seq_len": sh.seq_len,
                   "hidden": sh.hidden, "n_heads": sh.n_heads, "n_kv_heads": sh.n_kv_heads,
                   "head_dim": sh.head_dim, "ffn_dim": sh.ffn_dim, "ffn": sh.ffn, "norm": sh.norm,
                   "causal": sh.causal, "rope_base": sh.rope_base, "q_block": sh.q_block,
                   "kv_block": sh.kv_block, "head_chunk": sh.head_chunk,
                   "window": sh.window, "dropout_p": sh.dropout_p},
        "ms_per_step_median": round(float(np.median(step_ms)), 3),
        "ms_per_step_min": round(float(np.min(step_ms)), 3),
        "model_tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "mfma_practical_peak_tflops": round(practical, 1) if practical else None,
        "mfma_practical_frac": round(tflops / practical, 4) if practical else None,
        "fwd_ms": round(float(np.mean(fwd_ms)), 3),
        "bwd_ms": round(float(np.mean(bwd_ms)), 3),
        "gpu_sclk": clocks.summary(),
        "kernel_ms_per_step": breakdown,
        "memory": {"saved_bytes_per_token": saved_bytes / tokens,
                   "saved_sbh": round(saved_bytes / (tokens * sh.hidden), 3),
                   "peak_bytes_per_token": (saved_bytes + max(ws_f_bytes, ws_b_bytes)) / tokens,
                   "peak_sbh": round((saved_bytes + max(ws_f_bytes, ws_b_bytes)) / (tokens * sh.hidden), 3),
                   # the pages' per-layer predictions at this shape, in sbh
                   "pages_sbh": {k: round(acc.sbh_per_layer(sh.hidden, sh.n_heads, sh.seq_len, k), 2)
                                 for k in ("bpt", "flash", "vanilla")},
                   # cross-check: everything this process allocated on the GPU
                   # (inputs, weights, gradients, saved state, workspaces)
                   "torch_max_allocated_bytes": int(torch.cuda.max_memory_allocated(dev))},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle, s={args.cpu_sample_len})", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(sh, args.cpu_sample_len)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
