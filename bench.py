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


def attn_pairs(s: int, causal: bool) -> int:
    return s * (s + 1) // 2 if causal else s * s


def model_flops(sh) -> dict:
    """Model FLOPs of one layer (multiply-add = 2), causal attention counted on
    the visible pairs only; a step is forward + backward = 3 x forward."""
    s, h, H, Hkv, d, f = sh.seq_len, sh.hidden, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.ffn_dim
    n_ffn = 3 if sh.ffn == "swiglu" else 2
    lin = 2 * s * h * (H + 2 * Hkv) * d + 2 * s * H * d * h + 2 * s * h * f * n_ffn
    attn = 4 * d * H * attn_pairs(s, sh.causal)
    fwd = (lin + attn) * sh.batch
    pairs = attn_pairs(s, sh.causal) * sh.batch
    # Algorithmic attention FLOPs per kernel: forward QK^T and PV (4d per
    # visible pair and head); backward dV, dP, dK in the dK/dV pass (6d) and dQ
    # in the dQ pass (2d). "hw_" adds the recomputed products each kernel runs.
    return {"fwd": fwd, "step": 3 * fwd,
            "attn_fwd": 4 * d * H * pairs, "attn_bwd_dkdv": 6 * d * H * pairs,
            "attn_bwd_dq": 2 * d * H * pairs,
            "hw_attn_fwd": 4 * d * H * pairs, "hw_attn_bwd_dkdv": 8 * d * H * pairs,
            "hw_attn_bwd_dq": 6 * d * H * pairs}


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
            "sample": (f"float64 oracle forward+backward of the same layer at s={sample_len} "
                       f"({dt:.1f} s, {rate / 1e9:.1f} GFLOP/s); model-FLOP rate scaled to the "
                       f"per-token FLOPs at s={sh.seq_len}")}


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
    ap.add_argument("--breakdown", action="store_true",
                    help="also time GEMM and row-wise kernel classes (adds events)")
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
    import workloads as wl

    bpt.load_library()
    sh = wl.WORKLOADS[args.workload]
    if args.head_chunk:
        sh = sh.replace(head_chunk=args.head_chunk)
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

    # Dominant kernel: the attention kernel with the largest measured time.
    dom = max(attn_classes, key=lambda c: timing[c][0])
    dom_ms, dom_n = timing[dom]
    avg_ms = dom_ms / max(dom_n, 1)
    per_launch_flops = fl[dom] / max(dom_n / args.steps, 1)
    achieved = per_launch_flops / (avg_ms * 1e-3) / 1e12 if avg_ms > 0 else 0.0
    # bf16 with head_dim 64 / 128 runs the direct-to-LDS attention kernels.
    dma = sh.dtype == "bf16" and sh.head_dim in (64, 128)
    kernel_name = dom + ("_dma_kernel" if dma else "_kernel")
    traffic = (load_traffic(kernel_name, sh.name)
               if sh.head_chunk == wl.WORKLOADS[args.workload].head_chunk else None)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                # counters are taken at the workload's own head chunk
                "traffic": traffic,
                "traffic_gb_per_s": (round(traffic / (avg_ms * 1e-3) / 1e9, 1)
                                     if traffic and avg_ms > 0 else None),
                "kernel": kernel_name,
                "avg_launch_ms": round(avg_ms, 3), "launches_per_step": dom_n / args.steps,
                "algorithmic_flops_per_launch": per_launch_flops,
                "hardware_flops_per_launch": fl["hw_" + dom] / max(dom_n / args.steps, 1)}

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
                   "kv_block": sh.kv_block, "head_chunk": sh.head_chunk},
        "ms_per_step_median": round(float(np.median(step_ms)), 3),
        "ms_per_step_min": round(float(np.min(step_ms)), 3),
        "model_tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "mfma_practical_peak_tflops": round(practical, 1) if practical else None,
        "mfma_practical_frac": round(tflops / practical, 4) if practical else None,
        "fwd_ms": round(float(np.mean(fwd_ms)), 3),
        "bwd_ms": round(float(np.mean(bwd_ms)), 3),
        "kernel_ms_per_step": breakdown,
        "memory": {"saved_bytes_per_token": saved_bytes / tokens,
                   "saved_sbh": round(saved_bytes / (tokens * sh.hidden), 3),
                   "peak_bytes_per_token": (saved_bytes + max(ws_f_bytes, ws_b_bytes)) / tokens,
                   "peak_sbh": round((saved_bytes + max(ws_f_bytes, ws_b_bytes)) / (tokens * sh.hidden), 3),
                   "pages_bpt_sbh": 2, "pages_flashattention_ffn_sbh": 8,
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
