"""Host-side tests of the C ABI (no GPU work is launched).

* libbpt.so loads and exports every function include/bpt.h declares.
* The ctypes mirrors of the structs match the C layout (sizeof / offsetof from
  a small program compiled with gcc against the header).
* Descriptor validation returns the documented status before any launch.
* saved and workspace sizes are affine in s and hold no s * ffn_dim term.
"""
import ctypes
import os
import re
import subprocess

import pytest

import memory_efficient_long_amd as bpt
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpt.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bpt_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = bpt.load_library()
    names = _declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", bpt.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bpt_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "bpt.h"
#define F(S, m) printf(#S "." #m " %zu\n", offsetof(S, m));
int main(void) {
  printf("desc %zu\nweights %zu\ngrads %zu\n", sizeof(bpt_layer_desc),
         sizeof(bpt_layer_weights), sizeof(bpt_layer_grads));
  F(bpt_layer_desc, batch) F(bpt_layer_desc, head_chunk) F(bpt_layer_desc, rope_base)
  F(bpt_layer_desc, norm_eps) F(bpt_layer_grads, accumulate) F(bpt_layer_weights, n2_b)
  F(bpt_layer_desc, window) F(bpt_layer_desc, dropout_p) F(bpt_layer_desc, seed)
  F(bpt_stack_desc, n_layers) F(bpt_lm_head_desc, chunk_rows)
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    lines = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True,
                                                          text=True, check=True).stdout.split("\n")
                 if l)
    assert int(lines["desc"]) == ctypes.sizeof(bpt.BptLayerDesc)
    assert int(lines["weights"]) == ctypes.sizeof(bpt.BptLayerWeights)
    assert int(lines["grads"]) == ctypes.sizeof(bpt.BptLayerGrads)
    for key, (cls, field) in {"bpt_layer_desc.batch": (bpt.BptLayerDesc, "batch"),
                              "bpt_layer_desc.head_chunk": (bpt.BptLayerDesc, "head_chunk"),
                              "bpt_layer_desc.rope_base": (bpt.BptLayerDesc, "rope_base"),
                              "bpt_layer_desc.norm_eps": (bpt.BptLayerDesc, "norm_eps"),
                              "bpt_layer_grads.accumulate": (bpt.BptLayerGrads, "accumulate"),
                              "bpt_layer_weights.n2_b": (bpt.BptLayerWeights, "n2_b"),
                              "bpt_layer_desc.window": (bpt.BptLayerDesc, "window"),
                              "bpt_layer_desc.dropout_p": (bpt.BptLayerDesc, "dropout_p"),
                              "bpt_layer_desc.seed": (bpt.BptLayerDesc, "seed"),
                              "bpt_stack_desc.n_layers": (bpt.BptStackDesc, "n_layers"),
                              "bpt_lm_head_desc.chunk_rows": (bpt.BptLmHeadDesc, "chunk_rows")}.items():
        assert int(lines[key]) == getattr(cls, field).offset, key


def _desc(name="gpt1b-s8k", **kw):
    d = bpt.LayerConfig.from_shape(wl.WORKLOADS[name]).desc()
    for k, v in kw.items():
        setattr(d, k, v)
    if "hidden" in kw and "n_heads" not in kw and kw["hidden"] % d.head_dim == 0:
        d.n_heads = d.n_kv_heads = d.head_chunk = kw["hidden"] // d.head_dim
    return d


@pytest.mark.parametrize("name", list(wl.WORKLOADS) + list(wl.SMALL))
def test_workloads_validate(name):
    sh = wl.WORKLOADS.get(name) or wl.SMALL[name]
    d = bpt.LayerConfig.from_shape(sh).desc()
    assert bpt.bpt_layer_validate(d) == 0, bpt.bpt_last_error()
    assert bpt.bpt_layer_saved_size(d) > 0
    assert bpt.bpt_layer_workspace_size(d, False) > 0
    assert bpt.bpt_layer_workspace_size(d, True) > 0


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 1, 1), ("abi_version", 3, 1), ("dtype", 7, 1), ("norm", 3, 1), ("ffn", 9, 1), ("causal", 2, 1),
    ("seq_len", 8200, 1), ("seq_len", 0, 1), ("hidden", 2000, 1), ("n_kv_heads", 3, 1),
    ("head_dim", 96, 3), ("ffn_dim", 100, 1), ("q_block", 1000, 1), ("kv_block", 3000, 1),
    ("head_chunk", 3, 1), ("head_chunk", 0, 1), ("norm_eps", float("nan"), 1),
    # the norm kernels take rows of at most 16384 elements
    ("hidden", 32768, 3),
    ("window", -1, 1), ("dropout_p", 1.0, 1), ("dropout_p", -0.1, 1), ("dropout_p", 0.999, 1),
])
def test_invalid_descriptors(field, value, status):
    d = _desc(**{field: value})
    assert bpt.bpt_layer_validate(d) == status
    assert bpt.bpt_last_error()
    assert bpt.bpt_layer_saved_size(d) == 0
    assert bpt.bpt_layer_workspace_size(d, True) == 0


def test_gqa_head_chunk_rule():
    # head_chunk must hold whole GQA groups (32 query / 8 KV heads: group 4).
    assert bpt.bpt_layer_validate(_desc("llama8b-s64k", head_chunk=4)) == 0
    assert bpt.bpt_layer_validate(_desc("llama8b-s64k", head_chunk=2)) == 1
    assert bpt.bpt_layer_validate(_desc("gpt-tiny-fp32", head_dim=64, hidden=128)) == 0
    assert bpt.bpt_layer_validate(_desc("gpt-tiny-fp32", head_dim=128, hidden=256)) == 3


def test_forward_backward_reject_bad_arguments_before_launch():
    lib = bpt.load_library()
    d = _desc()
    w = bpt.BptLayerWeights(w_qkv=0x1000, w_o=0x1000, w_1=0x1000, w_2=0x1000, n1_g=0x1000,
                            n2_g=0x1000)
    ws_need = bpt.bpt_layer_workspace_size(d, False)
    fake = 0x10000
    # NULL x
    assert lib.bpt_layer_forward(ctypes.byref(d), None, ctypes.byref(w), fake, fake, fake,
                                 ws_need, None) == 1
    # misaligned y
    assert lib.bpt_layer_forward(ctypes.byref(d), fake, ctypes.byref(w), fake + 2, fake, fake,
                                 ws_need, None) == 1
    # workspace too small
    assert lib.bpt_layer_forward(ctypes.byref(d), fake, ctypes.byref(w), fake, fake, fake,
                                 ws_need - 1, None) == 2
    # missing weight matrix
    w2 = bpt.BptLayerWeights(w_qkv=0x1000, w_o=None, w_1=0x1000, w_2=0x1000, n1_g=0x1000,
                             n2_g=0x1000)
    assert lib.bpt_layer_forward(ctypes.byref(d), fake, ctypes.byref(w2), fake, fake, fake,
                                 ws_need, None) == 1
    # RMSNorm with a shift
    dr = _desc("llama8b-s64k")
    wr = bpt.BptLayerWeights(w_qkv=0x1000, w_o=0x1000, w_1=0x1000, w_2=0x1000, w_3=0x1000,
                             n1_g=0x1000, n2_g=0x1000, n1_b=0x1000)
    assert lib.bpt_layer_forward(ctypes.byref(dr), fake, ctypes.byref(wr), fake, fake, fake,
                                 bpt.bpt_layer_workspace_size(dr, False), None) == 1
    # backward: NULL grads table, bad accumulate flag, small workspace
    wsb = bpt.bpt_layer_workspace_size(d, True)
    assert lib.bpt_layer_backward(ctypes.byref(d), fake, ctypes.byref(w), fake, fake, fake, None,
                                  fake, wsb, None) == 1
    g = bpt.BptLayerGrads(accumulate=5)
    assert lib.bpt_layer_backward(ctypes.byref(d), fake, ctypes.byref(w), fake, fake, fake,
                                  ctypes.byref(g), fake, wsb, None) == 1
    g = bpt.BptLayerGrads(accumulate=0)
    assert lib.bpt_layer_backward(ctypes.byref(d), fake, ctypes.byref(w), fake, fake, fake,
                                  ctypes.byref(g), fake, wsb - 256, None) == 2
    assert bpt.bpt_status_string(2) == "workspace too small"


@pytest.mark.parametrize("backward", [False, True])
def test_memory_is_affine_in_s_without_s_times_ffn(backward):
    base = wl.WORKLOADS["gpt1b-s128k"]

    def ws(s, f):
        d = bpt.LayerConfig.from_shape(base.replace(seq_len=s, ffn_dim=f)).desc()
        return bpt.bpt_layer_workspace_size(d, backward), bpt.bpt_layer_saved_size(d)

    sizes = [ws(s, 8192) for s in (16384, 32768, 65536, 131072)]
    for i in range(2):
        assert [sizes[j][i] for j in range(4)] == sorted(sizes[j][i] for j in range(4))
        d1 = sizes[1][i] - sizes[0][i]
        d2 = (sizes[2][i] - sizes[1][i]) / 2
        d3 = (sizes[3][i] - sizes[2][i]) / 4
        assert abs(d1 - d2) <= 4096 and abs(d2 - d3) <= 4096     # linear in s (alignment slack)
    # The FFN width changes the workspace by the same amount at every s: the
    # FFN scratch covers one group of query blocks, never s x ffn_dim.
    df_small = ws(16384, 16384)[0] - ws(16384, 8192)[0]
    df_large = ws(131072, 16384)[0] - ws(131072, 8192)[0]
    assert df_small == df_large
    # Saved state is exactly O (bf16) plus one fp32 LSE per row and head.
    sh = base
    assert sizes[3][1] == sh.seq_len * sh.n_heads * sh.head_dim * 2 + sh.n_heads * sh.seq_len * 4


@pytest.mark.parametrize("head_chunk", [4, 8, 32])
def test_gqa_workspace_is_affine_in_s(head_chunk):
    """GQA with few KV heads per chunk adds the dK/dV split partials and the
    gathered chunk weights; the backward workspace stays affine in s."""
    base = wl.WORKLOADS["llama8b-s64k"].replace(head_chunk=head_chunk)

    def ws(s):
        d = bpt.LayerConfig.from_shape(base.replace(seq_len=s)).desc()
        return bpt.bpt_layer_workspace_size(d, True)

    sizes = [ws(s) for s in (16384, 32768, 65536, 131072)]
    d1 = sizes[1] - sizes[0]
    d2 = (sizes[2] - sizes[1]) / 2
    d3 = (sizes[3] - sizes[2]) / 4
    assert abs(d1 - d2) <= 8192 and abs(d2 - d3) <= 8192
    assert d1 > 0


def test_weight_set_matches_printed_parameter_counts(repo_root):
    """12h^2 + 13h per GPT layer ("Training memory", §3 parameters and §4/§5
    printed values)."""
    import json
    gold = json.load(open(os.path.join(repo_root, "tests", "golden", "page3_printed_values.json")))
    for h, count in gold["params_per_gpt_layer"].items():
        h = int(h)
        sh = wl.WORKLOADS["gpt1b-s8k"].replace(hidden=h, n_heads=h // 128, n_kv_heads=h // 128,
                                               head_dim=min(128, h), ffn_dim=4 * h)
        n = sum(int(__import__("numpy").prod(s)) for s in wl.weight_shapes(sh).values())
        assert n == count == 12 * h * h + 13 * h


def test_bench_refuses_more_than_one_gpu():
    """The benchmark is single-GPU: asking for more exits non-zero with a
    message instead of running (and reporting) anything."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode != 0
    assert "one GPU" in proc.stderr
    assert proc.stdout.strip() == ""


def test_lm_head_workspace_modes():
    """The fused LM-head call's workspace holds the forward's and the
    backward's plus one chunk's fp32 logits and log-sum-exps (each region
    rounded up to 256 bytes); other modes are refused with 0."""
    def up(n):
        return (n + 255) // 256 * 256
    for rows, h, v, c in [(1000, 128, 512, 256), (37, 64, 64, 64), (131072, 2048, 50304, 8192)]:
        cfg = bpt.LmHeadConfig(rows=rows, hidden=h, vocab=v, chunk_rows=c)
        cc = min(c, (rows + 63) // 64 * 64)
        f, b, fb = (bpt.bpt_lm_head_workspace_size(cfg, m) for m in (0, 1, 2))
        assert f == up(cc * (v // 32) * 8) + up(cc * 4)
        assert b == up(cc * v * 2)
        assert fb == f + b + up(cc * v * 4) + up(cc * 4)
        assert bpt.bpt_lm_head_workspace_size(cfg, 3) == 0
        assert bpt.bpt_lm_head_workspace_size(cfg, -1) == 0


def test_lm_head_fused_binding_checks(monkeypatch):
    """The fused call's binding refuses mismatched tensors before any launch;
    saved may be None, dz and dw_head not both."""
    torch = pytest.importorskip("torch")
    lib = bpt.load_library()
    calls = []
    monkeypatch.setattr(lib, "bpt_lm_head_forward_backward", lambda *a: calls.append(1) or 0)
    monkeypatch.setattr(bpt, "DEVICE_TYPE", "cpu")
    cfg = bpt.LmHeadConfig(rows=100, hidden=64, vocab=128, chunk_rows=64)
    d = cfg.desc()
    z = torch.zeros(100, 64, dtype=torch.bfloat16)
    w = torch.zeros(64, 128, dtype=torch.bfloat16)
    t = torch.zeros(100, dtype=torch.int32)
    g = torch.zeros(100, dtype=torch.float32)
    loss = torch.zeros(100, dtype=torch.float32)
    dz = torch.zeros_like(z)
    dw = torch.zeros(64, 128, dtype=torch.float32)
    ws = torch.zeros(bpt.bpt_lm_head_workspace_size(d, 2), dtype=torch.uint8)
    saved = torch.zeros(bpt.bpt_lm_head_saved_size(d), dtype=torch.uint8)
    st = _Stream()
    assert bpt.bpt_lm_head_forward_backward(d, z, w, t, g, loss, saved, dz, dw, ws, stream=st) == 0
    assert bpt.bpt_lm_head_forward_backward(d, z, w, t, g, loss, None, None, dw, ws, stream=st) == 0
    assert len(calls) == 2
    bad = {
        "ws-short": dict(ws=ws[:-1]),
        "ws-of-backward": dict(ws=torch.zeros(bpt.bpt_lm_head_workspace_size(d, 1),
                                              dtype=torch.uint8)),
        "loss-short": dict(loss=loss[:-1]),
        "dloss-missing": dict(g=None),
        "dloss-bf16": dict(g=g.bfloat16()),
        "saved-short": dict(saved=saved[:-4]),
        "no-grads": dict(dz=None, dw=None),
        "dw-bf16": dict(dw=dw.bfloat16()),
        "targets-int64": dict(t=t.long()),
    }
    for name, change in bad.items():
        a = dict(z=z, w=w, t=t, g=g, loss=loss, saved=saved, dz=dz, dw=dw, ws=ws)
        a.update(change)
        with pytest.raises(ValueError):
            bpt.bpt_lm_head_forward_backward(d, a["z"], a["w"], a["t"], a["g"], a["loss"],
                                             a["saved"], a["dz"], a["dw"], a["ws"], stream=st)
        assert len(calls) == 2, name


def test_bench_clock_reading_parses_the_current_level():
    """The bench logs the shader clock from the driver's level table: the
    starred line is the current level; a table with none gives no reading."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    assert bench.parse_sclk("0: 500Mhz\n1: 1750Mhz *\n2: 2400Mhz\n") == 1750.0
    assert bench.parse_sclk("S: 133Mhz\n0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.parse_sclk("") is None


@pytest.mark.parametrize("q_block", [512, 1024, 2048, 4096, 8192])
def test_ffn_scratch_is_a_group_of_query_blocks(q_block):
    """At s = 8192 the FFN scratch (the part of the backward workspace that
    grows with ffn_dim: pre-activation, activation and its gradient, plus the
    64 column-sum partial rows) covers one group of whole query blocks of at
    most s / 2 rows; only a single query block spanning the sequence makes
    it s rows ("Blockwise Parallel Transformer...", §3.2: the FFN runs per
    query block)."""
    base = wl.WORKLOADS["gpt1b-s8k"].replace(q_block=q_block)
    s = base.seq_len

    def ws(f):
        return bpt.bpt_layer_workspace_size(
            bpt.LayerConfig.from_shape(base.replace(ffn_dim=f)).desc(), True)

    df = 8192
    grow = ws(2 * df) - ws(df)
    rows = s if q_block == s else s // 2
    # three [rows, f] bf16 buffers (a, u, da) and 64 fp32 partial rows
    assert grow <= 3 * rows * df * 2 + 64 * df * 4 + 3 * 256
    if q_block < s:
        assert grow < 3 * s * df * 2


# ----------------------------------------------------------------- binding checks
class _Stream:
    cuda_stream = 0


def _binding_args(torch, sh):
    cfg = bpt.LayerConfig.from_shape(sh)
    d = cfg.desc()
    dt = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
    n = (sh.batch, sh.seq_len, sh.hidden)
    w = {k: torch.zeros(s, dtype=dt) for k, s in wl.weight_shapes(sh).items()}
    return dict(
        d=d, x=torch.zeros(n, dtype=dt), y=torch.zeros(n, dtype=dt), dy=torch.zeros(n, dtype=dt),
        dx=torch.zeros(n, dtype=dt), w=w,
        saved=torch.zeros(bpt.bpt_layer_saved_size(d), dtype=torch.uint8),
        wsf=torch.zeros(bpt.bpt_layer_workspace_size(d, False), dtype=torch.uint8),
        wsb=torch.zeros(bpt.bpt_layer_workspace_size(d, True), dtype=torch.uint8),
        grads={"d" + k: torch.zeros(s, dtype=torch.float32) for k, s in wl.weight_shapes(sh).items()})


def _mutations(torch):
    return {
        "x-fp32-under-bf16": lambda a: a.update(x=a["x"].float()),
        "x-transposed-view": lambda a: a.update(x=a["x"].transpose(1, 2).contiguous().transpose(1, 2)),
        "y-short": lambda a: a.update(y=a["y"][:, :-1]),
        "dy-short": lambda a: a.update(dy=a["dy"][:, :-16]),
        "dx-wrong-dtype": lambda a: a.update(dx=a["dx"].float()),
        "saved-short": lambda a: a.update(saved=a["saved"][:-1]),
        "ws-short": lambda a: a.update(wsf=a["wsf"][:-1], wsb=a["wsb"][:-1]),
        "w_o-short": lambda a: a["w"].update(w_o=a["w"]["w_o"][:-1]),
        "w_1-transposed-shape": lambda a: a["w"].update(w_1=a["w"]["w_1"].t().contiguous()),
        "w_qkv-wrong-dtype": lambda a: a["w"].update(w_qkv=a["w"]["w_qkv"].float()),
        "rmsnorm-with-shift": lambda a: a["w"].update(n1_b=torch.zeros_like(a["w"]["n1_g"])),
        "unknown-weight": lambda a: a["w"].update(w_9=a["w"]["w_1"]),
        "grad-bf16": lambda a: a["grads"].update(dw_1=a["grads"]["dw_1"].bfloat16()),
        "grad-wrong-shape": lambda a: a["grads"].update(dw_2=a["grads"]["dw_1"]),
    }


def _call(kind, a):
    if kind == "forward":
        return bpt.bpt_layer_forward(a["d"], a["x"], a["w"], a["y"], a["saved"], a["wsf"],
                                     stream=_Stream())
    return bpt.bpt_layer_backward(a["d"], a["x"], a["w"], a["saved"], a["dy"], a["dx"],
                                  a["grads"], a["wsb"], stream=_Stream())


@pytest.mark.parametrize("kind", ["forward", "backward"])
def test_binding_checks_tensors_before_any_launch(kind, monkeypatch):
    """The binding refuses tensors that do not match the descriptor (device,
    dtype, contiguity, element count, weight and gradient shapes, saved and
    workspace sizes) with ValueError and never reaches the library's compute
    entry points, which would otherwise read or write outside the tensors."""
    torch = pytest.importorskip("torch")
    lib = bpt.load_library()
    calls = []
    monkeypatch.setattr(lib, "bpt_layer_forward", lambda *a: calls.append("f") or 0)
    monkeypatch.setattr(lib, "bpt_layer_backward", lambda *a: calls.append("b") or 0)
    sh = wl.SMALL["llama8b-small"]   # bf16, RMSNorm, SwiGLU, GQA
    # Host tensors are refused outright (the library takes device pointers).
    with pytest.raises(ValueError, match="cuda"):
        _call(kind, _binding_args(torch, sh))
    assert not calls
    # With host tensors admitted, matching arguments reach the (stubbed) call.
    monkeypatch.setattr(bpt, "DEVICE_TYPE", "cpu")
    assert _call(kind, _binding_args(torch, sh)) == 0
    assert calls == [kind[0]]
    calls.clear()
    relevant = {"forward": {"dy-short", "dx-wrong-dtype", "grad-bf16", "grad-wrong-shape"},
                "backward": {"y-short"}}[kind]
    for name, mutate in _mutations(torch).items():
        if name in relevant:
            continue
        a = _binding_args(torch, sh)
        mutate(a)
        with pytest.raises(ValueError):
            _call(kind, a)
            pytest.fail(f"{name}: accepted")
        assert not calls, name


def test_noalloc_forward_refuses_layers_beyond_its_scratch():
    """The allocation-free forward checks its static scratch size on the host
    and returns BPT_EWORKSPACE before any device work (the GPT-1B-shaped layer
    at s = 8192 needs more than the 64 MiB it holds)."""
    lib = bpt.load_library()
    d = _desc()
    assert bpt.bpt_layer_workspace_size(d, False) > bpt.bpt_layer_noalloc_scratch_bytes()
    assert bpt.bpt_layer_noalloc_scratch_bytes() == 64 << 20
    w = bpt.BptLayerWeights(w_qkv=0x1000, w_o=0x1000, w_1=0x1000, w_2=0x1000, n1_g=0x1000,
                            n2_g=0x1000)
    fake = 0x10000
    assert lib.bpt_layer_forward_noalloc(ctypes.byref(d), fake, ctypes.byref(w), fake, fake,
                                         None) == 2
    assert "static scratch" in bpt.bpt_last_error()
    # argument errors come first, as in bpt_layer_forward
    assert lib.bpt_layer_forward_noalloc(ctypes.byref(d), None, ctypes.byref(w), fake, fake,
                                         None) == 1


@pytest.mark.parametrize("L,k", [(1, 1), (3, 0), (3, 1), (3, 2), (3, 3), (8, 2), (8, 3)])
def test_stack_memory_follows_checkpoint_every_k(L, k):
    """Saved bytes: (ceil(L / k) - 1) checkpoints of one activation c for
    k >= 1 (the first segment's is x), or L - 1 activations and L saved
    states for k = 0. Backward peak (saved + workspace) for k >= 1:
    (ceil(L / k) - 1) c + k rebuilt layers (input + saved state) + scratch and
    gradient activations + the layer workspace: the (L/k) c + k A of
    "Training memory", §3 (checkpoint every k layers)."""
    sh = wl.WORKLOADS["gpt1b-s8k"]
    layer = bpt.LayerConfig.from_shape(sh)
    d = bpt.StackConfig(layer, L, k).desc()
    assert bpt.bpt_stack_validate(d) == 0
    ld = layer.desc()
    c = sh.seq_len * sh.hidden * 2
    sv = -(-bpt.bpt_layer_saved_size(ld) // 256) * 256
    lw = max(bpt.bpt_layer_workspace_size(ld, False), bpt.bpt_layer_workspace_size(ld, True))
    saved = bpt.bpt_stack_saved_size(d)
    wsb = bpt.bpt_stack_workspace_size(d, True)
    if k == 0:
        assert saved == (L - 1) * c + L * sv
        assert wsb == 2 * c + bpt.bpt_layer_workspace_size(ld, True)
    else:
        n_ck = -(-L // k) - 1
        assert saved == n_ck * c
        assert saved + wsb == (n_ck + (k - 1) + 1 + 2) * c + k * sv + lw
    assert bpt.bpt_stack_workspace_size(d, False) == 2 * c + (sv if k else 0) + \
        bpt.bpt_layer_workspace_size(ld, False)


def test_stack_descriptor_rules():
    layer = bpt.LayerConfig.from_shape(wl.WORKLOADS["gpt1b-s8k"])
    assert bpt.bpt_stack_validate(bpt.StackConfig(layer, 0, 0).desc()) == 1
    assert bpt.bpt_stack_validate(bpt.StackConfig(layer, 3, 4).desc()) == 1
    assert bpt.bpt_stack_validate(bpt.StackConfig(layer, 3, -1).desc()) == 1
    bad = dataclasses_replace(layer, q_block=1000)
    assert bpt.bpt_stack_validate(bpt.StackConfig(bad, 3, 1).desc()) == 1
    assert bpt.bpt_stack_saved_size(bpt.StackConfig(layer, 3, 4).desc()) == 0


def dataclasses_replace(obj, **kw):
    import dataclasses
    return dataclasses.replace(obj, **kw)


def test_window_needs_causal():
    assert bpt.bpt_layer_validate(_desc(window=64)) == 0
    assert bpt.bpt_layer_validate(_desc(window=1 << 30)) == 0      # wider than s: plain causal
    assert bpt.bpt_layer_validate(_desc(window=64, causal=0)) == 1
