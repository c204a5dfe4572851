"""Python binding of the MI355X Blockwise Parallel Transformer layer library.

The compute runs in ``libbpt.so`` (HIP kernels for gfx950, built in-tree by
``memory_efficient_long_amd.build``); this module only marshals arguments
through the C ABI declared in ``include/bpt.h``. The functions carry the C
names (``bpt_layer_forward`` ...). PyTorch supplies device memory and the
stream. There is no fallback: if the library is missing, importing the binding
raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

__all__ = [
    "LayerConfig", "BptLayerDesc", "BptLayerWeights", "BptLayerGrads", "BptError",
    "load_library", "bpt_layer_validate", "bpt_layer_saved_size", "bpt_layer_workspace_size",
    "bpt_layer_forward", "bpt_layer_backward", "bpt_status_string", "bpt_last_error",
    "forward", "backward", "WEIGHT_NAMES", "GRAD_NAMES", "bpt_timing_enable", "bpt_timing_read",
    "bpt_mfma_peak_probe",
    "KERNEL_CLASSES", "check_forward_args", "check_backward_args", "weight_shapes_of",
    "bpt_layer_forward_noalloc", "bpt_layer_noalloc_scratch_bytes",
    "LmHeadConfig", "BptLmHeadDesc", "bpt_lm_head_validate", "bpt_lm_head_saved_size",
    "bpt_lm_head_workspace_size", "bpt_lm_head_forward", "bpt_lm_head_backward",
    "bpt_lm_head_forward_backward", "lm_head_forward", "lm_head_backward",
    "lm_head_forward_backward", "check_lm_head_args",
    "StackConfig", "BptStackDesc", "bpt_stack_validate", "bpt_stack_saved_size",
    "bpt_stack_workspace_size", "bpt_stack_forward", "bpt_stack_backward", "stack_forward",
    "stack_backward",
]

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libbpt.so")
ABI_VERSION = 2

DTYPES = {"f32": 0, "bf16": 1}
NORMS = {"layernorm": 0, "rmsnorm": 1}
FFNS = {"relu": 0, "gelu": 1, "swiglu": 2}

WEIGHT_NAMES = ["w_qkv", "b_qkv", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2", "w_3",
                "n1_g", "n1_b", "n2_g", "n2_b"]
GRAD_NAMES = ["dw_qkv", "db_qkv", "dw_o", "db_o", "dw_1", "db_1", "dw_2", "db_2", "dw_3",
              "dn1_g", "dn1_b", "dn2_g", "dn2_b"]


class BptLayerDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
        ("ffn", ctypes.c_int32), ("causal", ctypes.c_int32), ("use_rope", ctypes.c_int32),
        ("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("hidden", ctypes.c_int64),
        ("n_heads", ctypes.c_int64), ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("ffn_dim", ctypes.c_int64), ("q_block", ctypes.c_int64), ("kv_block", ctypes.c_int64),
        ("head_chunk", ctypes.c_int64), ("rope_base", ctypes.c_double),
        ("norm_eps", ctypes.c_float), ("window", ctypes.c_int32),
        ("dropout_p", ctypes.c_float), ("reserved", ctypes.c_int32), ("seed", ctypes.c_uint64),
    ]


class BptLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


class BptLayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_NAMES] + [
        ("accumulate", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class BptStackDesc(ctypes.Structure):
    _fields_ = [("layer", BptLayerDesc), ("n_layers", ctypes.c_int64),
                ("checkpoint_every", ctypes.c_int64)]


class BptLmHeadDesc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("hidden", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("chunk_rows", ctypes.c_int64)]


class BptError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load_library()
        msg = lib.bpt_status_string(status).decode()
        detail = lib.bpt_last_error().decode()
        super().__init__(f"{where}: {msg} (status {status}){': ' + detail if detail else ''}")
        self.status = status


_LIB: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libbpt.so (once; BPT_LIBRARY overrides the path). Raises if it has
    not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or os.environ.get("BPT_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m memory_efficient_long_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.bpt_layer_validate.argtypes = [P(BptLayerDesc)]
    lib.bpt_layer_validate.restype = ctypes.c_int
    lib.bpt_layer_saved_size.argtypes = [P(BptLayerDesc)]
    lib.bpt_layer_saved_size.restype = ctypes.c_size_t
    lib.bpt_layer_workspace_size.argtypes = [P(BptLayerDesc), ctypes.c_int32]
    lib.bpt_layer_workspace_size.restype = ctypes.c_size_t
    lib.bpt_layer_forward.argtypes = [P(BptLayerDesc), ctypes.c_void_p, P(BptLayerWeights),
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
    lib.bpt_layer_forward.restype = ctypes.c_int
    lib.bpt_layer_backward.argtypes = [P(BptLayerDesc), ctypes.c_void_p, P(BptLayerWeights),
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       P(BptLayerGrads), ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
    lib.bpt_layer_backward.restype = ctypes.c_int
    lib.bpt_layer_forward_noalloc.argtypes = [P(BptLayerDesc), ctypes.c_void_p,
                                              P(BptLayerWeights), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]
    lib.bpt_layer_forward_noalloc.restype = ctypes.c_int
    lib.bpt_layer_noalloc_scratch_bytes.argtypes = []
    lib.bpt_layer_noalloc_scratch_bytes.restype = ctypes.c_size_t
    SP = P(BptStackDesc)
    lib.bpt_stack_validate.argtypes = [SP]
    lib.bpt_stack_validate.restype = ctypes.c_int
    lib.bpt_stack_saved_size.argtypes = [SP]
    lib.bpt_stack_saved_size.restype = ctypes.c_size_t
    lib.bpt_stack_workspace_size.argtypes = [SP, ctypes.c_int32]
    lib.bpt_stack_workspace_size.restype = ctypes.c_size_t
    lib.bpt_stack_forward.argtypes = [SP, ctypes.c_void_p, P(BptLayerWeights), ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]
    lib.bpt_stack_forward.restype = ctypes.c_int
    lib.bpt_stack_backward.argtypes = [SP, ctypes.c_void_p, P(BptLayerWeights), ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, P(BptLayerGrads),
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.bpt_stack_backward.restype = ctypes.c_int
    LP = P(BptLmHeadDesc)
    lib.bpt_lm_head_validate.argtypes = [LP]
    lib.bpt_lm_head_validate.restype = ctypes.c_int
    lib.bpt_lm_head_saved_size.argtypes = [LP]
    lib.bpt_lm_head_saved_size.restype = ctypes.c_size_t
    lib.bpt_lm_head_workspace_size.argtypes = [LP, ctypes.c_int32]
    lib.bpt_lm_head_workspace_size.restype = ctypes.c_size_t
    vp = ctypes.c_void_p
    lib.bpt_lm_head_forward.argtypes = [LP, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bpt_lm_head_forward.restype = ctypes.c_int
    lib.bpt_lm_head_backward.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                         ctypes.c_size_t, vp]
    lib.bpt_lm_head_backward.restype = ctypes.c_int
    lib.bpt_lm_head_forward_backward.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                                 vp, ctypes.c_size_t, vp]
    lib.bpt_lm_head_forward_backward.restype = ctypes.c_int
    lib.bpt_status_string.argtypes = [ctypes.c_int]
    lib.bpt_status_string.restype = ctypes.c_char_p
    lib.bpt_last_error.argtypes = []
    lib.bpt_last_error.restype = ctypes.c_char_p
    lib.bpt_mfma_peak_probe.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.bpt_mfma_peak_probe.restype = ctypes.c_int
    lib.bpt_timing_enable.argtypes = [ctypes.c_uint32]
    lib.bpt_timing_enable.restype = ctypes.c_int
    lib.bpt_timing_read.argtypes = [P(ctypes.c_double), P(ctypes.c_int64), ctypes.c_int32]
    lib.bpt_timing_read.restype = ctypes.c_int
    _LIB = lib
    return lib


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and options of one layer (mirrors bpt_layer_desc)."""
    seq_len: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    dtype: str = "bf16"
    norm: str = "layernorm"
    ffn: str = "gelu"
    causal: bool = True
    rope_base: Optional[float] = None
    q_block: int = 1024
    kv_block: int = 2048
    head_chunk: Optional[int] = None
    batch: int = 1
    norm_eps: float = 1e-5
    window: int = 0
    dropout_p: float = 0.0
    seed: int = 0

    @staticmethod
    def from_shape(sh) -> "LayerConfig":
        return LayerConfig(seq_len=sh.seq_len, hidden=sh.hidden, n_heads=sh.n_heads,
                           n_kv_heads=sh.n_kv_heads, head_dim=sh.head_dim, ffn_dim=sh.ffn_dim,
                           dtype=sh.dtype, norm=sh.norm, ffn=sh.ffn, causal=sh.causal,
                           rope_base=sh.rope_base, q_block=sh.q_block, kv_block=sh.kv_block,
                           head_chunk=sh.head_chunk, batch=sh.batch, norm_eps=sh.norm_eps,
                           window=getattr(sh, "window", 0),
                           dropout_p=getattr(sh, "dropout_p", 0.0), seed=getattr(sh, "seed", 0))

    def desc(self) -> BptLayerDesc:
        return BptLayerDesc(
            abi_version=ABI_VERSION, dtype=DTYPES[self.dtype], norm=NORMS[self.norm],
            ffn=FFNS[self.ffn], causal=int(self.causal), use_rope=int(self.rope_base is not None),
            batch=self.batch, seq_len=self.seq_len, hidden=self.hidden, n_heads=self.n_heads,
            n_kv_heads=self.n_kv_heads, head_dim=self.head_dim, ffn_dim=self.ffn_dim,
            q_block=self.q_block, kv_block=self.kv_block,
            head_chunk=self.head_chunk if self.head_chunk else self.n_heads,
            rope_base=float(self.rope_base or 0.0), norm_eps=self.norm_eps, window=self.window,
            dropout_p=self.dropout_p, reserved=0, seed=self.seed)


def _desc(d) -> BptLayerDesc:
    return d.desc() if isinstance(d, LayerConfig) else d


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ----------------------------------------------------------------- C-named wrappers
def bpt_layer_validate(desc) -> int:
    return load_library().bpt_layer_validate(ctypes.byref(_desc(desc)))


def bpt_layer_saved_size(desc) -> int:
    return load_library().bpt_layer_saved_size(ctypes.byref(_desc(desc)))


def bpt_layer_workspace_size(desc, backward: bool) -> int:
    return load_library().bpt_layer_workspace_size(ctypes.byref(_desc(desc)), int(backward))


def bpt_status_string(status: int) -> str:
    return load_library().bpt_status_string(status).decode()


def bpt_last_error() -> str:
    return load_library().bpt_last_error().decode()


KERNEL_CLASSES = ["attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq", "gemm", "rowwise", "lm_head"]


def bpt_timing_enable(classes) -> int:
    """Enable HIP-event timing for the named kernel classes (empty: disable)."""
    mask = 0
    for c in classes:
        mask |= 1 << KERNEL_CLASSES.index(c)
    return load_library().bpt_timing_enable(mask)


def bpt_timing_read(reset: bool = True) -> Dict[str, tuple]:
    """{class: (total_ms, launches)} since the last reset (waits for the events)."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    st = load_library().bpt_timing_read(ms, cnt, int(reset))
    if st:
        raise BptError(st, "bpt_timing_read")
    return {c: (ms[i], cnt[i]) for i, c in enumerate(KERNEL_CLASSES)}


def bpt_mfma_peak_probe(stream=None) -> float:
    """Sustained dense bf16 MFMA TFLOP/s of the current device (measured)."""
    out = ctypes.c_double(0.0)
    st = load_library().bpt_mfma_peak_probe(ctypes.byref(out), _stream_handle(stream))
    if st:
        raise BptError(st, "bpt_mfma_peak_probe")
    return out.value


def _weights_struct(weights: Dict[str, "object"]) -> BptLayerWeights:
    return BptLayerWeights(**{n: _ptr(weights.get(n)) for n in WEIGHT_NAMES})


# ----------------------------------------------------------------- argument checks
# The C ABI takes raw device pointers and trusts the sizes implied by the
# descriptor, so a short, mistyped or strided tensor would make the kernels read
# or write outside it. Every tensor is checked here before the library is
# called; a failed check raises ValueError and launches nothing.
DEVICE_TYPE = "cuda"
_TORCH_DTYPE_NAMES = {0: "float32", 1: "bfloat16"}


def weight_shapes_of(desc) -> Dict[str, tuple]:
    """Shape of every weight the descriptor admits (w_3 only for SwiGLU;
    norm shifts only for LayerNorm)."""
    d = _desc(desc)
    h, f, hd = d.hidden, d.ffn_dim, d.n_heads * d.head_dim
    qkv = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim
    shapes = {"w_qkv": (h, qkv), "b_qkv": (qkv,), "w_o": (hd, h), "b_o": (h,), "w_1": (h, f),
              "b_1": (f,), "w_2": (f, h), "b_2": (h,), "n1_g": (h,), "n2_g": (h,)}
    if d.ffn == FFNS["swiglu"]:
        shapes["w_3"] = (h, f)
    if d.norm == NORMS["layernorm"]:
        shapes["n1_b"] = (h,)
        shapes["n2_b"] = (h,)
    return shapes


def _check_tensor(t, name, device, dtype=None, numel=None, shape=None, min_bytes=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device.type != DEVICE_TYPE:
        raise ValueError(f"{name} must be a {DEVICE_TYPE} tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements (got {t.numel()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {min_bytes}")


def _check_weights(d, weights, device):
    shapes = weight_shapes_of(d)
    dt = _TORCH_DTYPE_NAMES[d.dtype]
    unknown = set(weights) - set(WEIGHT_NAMES)
    if unknown:
        raise ValueError(f"unknown weight names {sorted(unknown)}")
    for n in WEIGHT_NAMES:
        t = weights.get(n)
        if t is None:
            continue
        if n not in shapes:
            raise ValueError(f"{n} is not used by this layer (must be absent)")
        _check_tensor(t, n, device, dtype=dt, shape=shapes[n])


def check_forward_args(desc, x, weights, y, saved, workspace, need_workspace=True) -> None:
    """Raise ValueError unless every tensor matches the descriptor."""
    d = _desc(desc)
    if d.dtype not in _TORCH_DTYPE_NAMES:
        raise ValueError("descriptor dtype")
    n = d.batch * d.seq_len * d.hidden
    dt = _TORCH_DTYPE_NAMES[d.dtype]
    _check_tensor(x, "x", None, dtype=dt, numel=n)
    dev = x.device
    _check_tensor(y, "y", dev, dtype=dt, numel=n)
    _check_weights(d, weights, dev)
    _check_tensor(saved, "saved", dev, min_bytes=bpt_layer_saved_size(d))
    if need_workspace:
        _check_tensor(workspace, "workspace", dev, min_bytes=bpt_layer_workspace_size(d, False))


def check_backward_args(desc, x, weights, saved, dy, dx, grads, workspace) -> None:
    """Raise ValueError unless every tensor matches the descriptor."""
    d = _desc(desc)
    if d.dtype not in _TORCH_DTYPE_NAMES:
        raise ValueError("descriptor dtype")
    n = d.batch * d.seq_len * d.hidden
    dt = _TORCH_DTYPE_NAMES[d.dtype]
    _check_tensor(x, "x", None, dtype=dt, numel=n)
    dev = x.device
    _check_tensor(dy, "dy", dev, dtype=dt, numel=n)
    _check_tensor(dx, "dx", dev, dtype=dt, numel=n)
    _check_weights(d, weights, dev)
    _check_tensor(saved, "saved", dev, min_bytes=bpt_layer_saved_size(d))
    _check_tensor(workspace, "workspace", dev, min_bytes=bpt_layer_workspace_size(d, True))
    shapes = weight_shapes_of(d)
    unknown = set(grads) - set(GRAD_NAMES)
    if unknown:
        raise ValueError(f"unknown gradient names {sorted(unknown)}")
    for g, t in grads.items():
        if t is None:
            continue
        if g[1:] not in shapes:
            raise ValueError(f"{g} is not used by this layer (must be absent)")
        _check_tensor(t, g, dev, dtype="float32", shape=shapes[g[1:]])


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def bpt_layer_forward(desc, x, weights, y, saved, workspace, stream=None) -> int:
    """Raw call: every argument is a device tensor (weights: dict by name),
    checked against the descriptor first (ValueError, nothing launched)."""
    d = _desc(desc)
    check_forward_args(d, x, weights, y, saved, workspace)
    w = _weights_struct(weights)
    return load_library().bpt_layer_forward(
        ctypes.byref(d), _ptr(x), ctypes.byref(w), _ptr(y), _ptr(saved), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))


def bpt_layer_forward_noalloc(desc, x, weights, y, saved, stream=None) -> int:
    """Raw call of the allocation-free forward (the library's static scratch
    replaces the workspace); tensors are checked as for bpt_layer_forward."""
    d = _desc(desc)
    check_forward_args(d, x, weights, y, saved, None, need_workspace=False)
    w = _weights_struct(weights)
    return load_library().bpt_layer_forward_noalloc(
        ctypes.byref(d), _ptr(x), ctypes.byref(w), _ptr(y), _ptr(saved), _stream_handle(stream))


def bpt_layer_noalloc_scratch_bytes() -> int:
    return load_library().bpt_layer_noalloc_scratch_bytes()


def bpt_layer_backward(desc, x, weights, saved, dy, dx, grads, workspace, accumulate=False,
                       stream=None) -> int:
    """Raw call: grads is a dict of fp32 device tensors by GRAD_NAMES (missing = not
    computed); every tensor is checked against the descriptor first (ValueError, nothing
    launched)."""
    d = _desc(desc)
    check_backward_args(d, x, weights, saved, dy, dx, grads, workspace)
    w = _weights_struct(weights)
    g = BptLayerGrads(**{n: _ptr(grads.get(n)) for n in GRAD_NAMES}, accumulate=int(accumulate),
                      reserved=0)
    return load_library().bpt_layer_backward(
        ctypes.byref(d), _ptr(x), ctypes.byref(w), _ptr(saved), _ptr(dy), _ptr(dx),
        ctypes.byref(g), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(stream))


# ----------------------------------------------------------------- conveniences
def _alloc_bytes(n: int, device):
    import torch
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


def forward(cfg: LayerConfig, x, weights, y=None, saved=None, workspace=None, stream=None):
    """y, saved = forward(cfg, x, weights): allocates what is not passed."""
    import torch
    d = cfg.desc()
    st = bpt_layer_validate(d)
    if st:
        raise BptError(st, "bpt_layer_validate")
    if y is None:
        y = torch.empty_like(x)
    if saved is None:
        saved = _alloc_bytes(bpt_layer_saved_size(d), x.device)
    if workspace is None:
        workspace = _alloc_bytes(bpt_layer_workspace_size(d, False), x.device)
    st = bpt_layer_forward(d, x, weights, y, saved, workspace, stream)
    if st:
        raise BptError(st, "bpt_layer_forward")
    return y, saved


def grad_shapes(cfg: LayerConfig, weights) -> Dict[str, tuple]:
    return {"d" + n: tuple(weights[n].shape) for n in WEIGHT_NAMES if weights.get(n) is not None}


def backward(cfg: LayerConfig, x, weights, saved, dy, dx=None, grads=None, workspace=None,
             accumulate=False, stream=None):
    """dx, grads = backward(...): fp32 gradients for every weight present."""
    import torch
    d = cfg.desc()
    if dx is None:
        dx = torch.empty_like(x)
    if grads is None:
        grads = {k: torch.empty(s, dtype=torch.float32, device=x.device)
                 for k, s in grad_shapes(cfg, weights).items()}
    if workspace is None:
        workspace = _alloc_bytes(bpt_layer_workspace_size(d, True), x.device)
    st = bpt_layer_backward(d, x, weights, saved, dy, dx, grads, workspace, accumulate, stream)
    if st:
        raise BptError(st, "bpt_layer_backward")
    return dx, grads


# ----------------------------------------------------------------- LM head with cross-entropy
@dataclasses.dataclass(frozen=True)
class LmHeadConfig:
    """Shape of the blockwise LM head (mirrors bpt_lm_head_desc)."""
    rows: int
    hidden: int
    vocab: int
    chunk_rows: int = 8192
    dtype: str = "bf16"

    def desc(self) -> BptLmHeadDesc:
        return BptLmHeadDesc(abi_version=ABI_VERSION, dtype=DTYPES[self.dtype], rows=self.rows,
                             hidden=self.hidden, vocab=self.vocab, chunk_rows=self.chunk_rows)


def _lm_desc(d) -> BptLmHeadDesc:
    return d.desc() if isinstance(d, LmHeadConfig) else d


def bpt_lm_head_validate(desc) -> int:
    return load_library().bpt_lm_head_validate(ctypes.byref(_lm_desc(desc)))


def bpt_lm_head_saved_size(desc) -> int:
    return load_library().bpt_lm_head_saved_size(ctypes.byref(_lm_desc(desc)))


def bpt_lm_head_workspace_size(desc, backward) -> int:
    """backward: False / 0 forward, True / 1 backward, 2 the fused call."""
    return load_library().bpt_lm_head_workspace_size(ctypes.byref(_lm_desc(desc)), int(backward))


def check_lm_head_args(desc, z, w_head, targets, saved, workspace, backward, loss=None,
                       dloss=None, dz=None, dw_head=None) -> None:
    """Raise ValueError unless every tensor matches the LM-head descriptor
    (backward: 0 forward, 1 backward, 2 the fused call, whose saved may be None)."""
    d = _lm_desc(desc)
    if d.dtype not in _TORCH_DTYPE_NAMES:
        raise ValueError("descriptor dtype")
    dt = _TORCH_DTYPE_NAMES[d.dtype]
    _check_tensor(z, "z", None, dtype=dt, numel=d.rows * d.hidden)
    dev = z.device
    _check_tensor(w_head, "w_head", dev, dtype=dt, shape=(d.hidden, d.vocab))
    _check_tensor(targets, "targets", dev, dtype="int32", numel=d.rows)
    mode = int(backward)
    if saved is not None or mode != 2:
        _check_tensor(saved, "saved", dev, min_bytes=bpt_lm_head_saved_size(d))
    _check_tensor(workspace, "workspace", dev, min_bytes=bpt_lm_head_workspace_size(d, mode))
    if mode != 1:
        _check_tensor(loss, "loss", dev, dtype="float32", numel=d.rows)
    if mode == 0:
        return
    _check_tensor(dloss, "dloss", dev, dtype="float32", numel=d.rows)
    if dz is None and dw_head is None:
        raise ValueError("dz and dw_head are both None")
    if dz is not None:
        _check_tensor(dz, "dz", dev, dtype=dt, numel=d.rows * d.hidden)
    if dw_head is not None:
        _check_tensor(dw_head, "dw_head", dev, dtype="float32", shape=(d.hidden, d.vocab))


def bpt_lm_head_forward(desc, z, w_head, targets, loss, saved, workspace, stream=None) -> int:
    """Raw call (device tensors, checked first)."""
    d = _lm_desc(desc)
    check_lm_head_args(d, z, w_head, targets, saved, workspace, False, loss=loss)
    return load_library().bpt_lm_head_forward(
        ctypes.byref(d), _ptr(z), _ptr(w_head), _ptr(targets), _ptr(loss), _ptr(saved),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_handle(stream))


def bpt_lm_head_backward(desc, z, w_head, targets, saved, dloss, dz, dw_head, workspace,
                         accumulate=False, stream=None) -> int:
    """Raw call (device tensors, checked first); dz or dw_head may be None."""
    d = _lm_desc(desc)
    check_lm_head_args(d, z, w_head, targets, saved, workspace, True, dloss=dloss, dz=dz,
                       dw_head=dw_head)
    return load_library().bpt_lm_head_backward(
        ctypes.byref(d), _ptr(z), _ptr(w_head), _ptr(targets), _ptr(saved), _ptr(dloss), _ptr(dz),
        _ptr(dw_head), int(accumulate), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))


def bpt_lm_head_forward_backward(desc, z, w_head, targets, dloss, loss, saved, dz, dw_head,
                                 workspace, accumulate=False, stream=None) -> int:
    """Raw fused call (device tensors, checked first); saved, dz or dw_head may be None."""
    d = _lm_desc(desc)
    check_lm_head_args(d, z, w_head, targets, saved, workspace, 2, loss=loss, dloss=dloss, dz=dz,
                       dw_head=dw_head)
    return load_library().bpt_lm_head_forward_backward(
        ctypes.byref(d), _ptr(z), _ptr(w_head), _ptr(targets), _ptr(dloss), _ptr(loss),
        _ptr(saved), _ptr(dz), _ptr(dw_head), int(accumulate), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))


def lm_head_forward(cfg: LmHeadConfig, z, w_head, targets, stream=None):
    """loss, saved = lm_head_forward(cfg, z, w_head, targets): allocates outputs."""
    import torch
    d = cfg.desc()
    st = bpt_lm_head_validate(d)
    if st:
        raise BptError(st, "bpt_lm_head_validate")
    loss = torch.empty(cfg.rows, dtype=torch.float32, device=z.device)
    saved = _alloc_bytes(bpt_lm_head_saved_size(d), z.device)
    ws = _alloc_bytes(bpt_lm_head_workspace_size(d, False), z.device)
    st = bpt_lm_head_forward(d, z, w_head, targets, loss, saved, ws, stream)
    if st:
        raise BptError(st, "bpt_lm_head_forward")
    return loss, saved


def lm_head_backward(cfg: LmHeadConfig, z, w_head, targets, saved, dloss, dz=None, dw_head=None,
                     accumulate=False, stream=None):
    """dz, dw_head = lm_head_backward(...): allocates what is not passed."""
    import torch
    d = cfg.desc()
    if dz is None:
        dz = torch.empty_like(z)
    if dw_head is None:
        dw_head = torch.empty(cfg.hidden, cfg.vocab, dtype=torch.float32, device=z.device)
    ws = _alloc_bytes(bpt_lm_head_workspace_size(d, True), z.device)
    st = bpt_lm_head_backward(d, z, w_head, targets, saved, dloss, dz, dw_head, ws, accumulate,
                              stream)
    if st:
        raise BptError(st, "bpt_lm_head_backward")
    return dz, dw_head


def lm_head_forward_backward(cfg: LmHeadConfig, z, w_head, targets, dloss, stream=None):
    """loss, saved, dz, dw_head = lm_head_forward_backward(...): loss and gradients in one
    call (the logits computed once per chunk); allocates every output."""
    import torch
    d = cfg.desc()
    st = bpt_lm_head_validate(d)
    if st:
        raise BptError(st, "bpt_lm_head_validate")
    loss = torch.empty(cfg.rows, dtype=torch.float32, device=z.device)
    saved = _alloc_bytes(bpt_lm_head_saved_size(d), z.device)
    dz = torch.empty_like(z)
    dw_head = torch.empty(cfg.hidden, cfg.vocab, dtype=torch.float32, device=z.device)
    ws = _alloc_bytes(bpt_lm_head_workspace_size(d, 2), z.device)
    st = bpt_lm_head_forward_backward(d, z, w_head, targets, dloss, loss, saved, dz, dw_head, ws,
                                      False, stream)
    if st:
        raise BptError(st, "bpt_lm_head_forward_backward")
    return loss, saved, dz, dw_head


# ----------------------------------------------------------------- stack of layers
@dataclasses.dataclass(frozen=True)
class StackConfig:
    """n_layers layers of one shape with checkpointing every k layers
    (mirrors bpt_stack_desc; k = 0 keeps every layer's saved state)."""
    layer: LayerConfig
    n_layers: int
    checkpoint_every: int = 1

    def desc(self) -> BptStackDesc:
        return BptStackDesc(layer=self.layer.desc(), n_layers=self.n_layers,
                            checkpoint_every=self.checkpoint_every)


def _stack_desc(d) -> BptStackDesc:
    return d.desc() if isinstance(d, StackConfig) else d


def bpt_stack_validate(desc) -> int:
    return load_library().bpt_stack_validate(ctypes.byref(_stack_desc(desc)))


def bpt_stack_saved_size(desc) -> int:
    return load_library().bpt_stack_saved_size(ctypes.byref(_stack_desc(desc)))


def bpt_stack_workspace_size(desc, backward: bool) -> int:
    return load_library().bpt_stack_workspace_size(ctypes.byref(_stack_desc(desc)), int(backward))


def _check_stack(d, x, weights_list, saved, workspace, backward):
    if len(weights_list) != d.n_layers:
        raise ValueError(f"{len(weights_list)} weight tables for {d.n_layers} layers")
    n = d.layer.batch * d.layer.seq_len * d.layer.hidden
    dt = _TORCH_DTYPE_NAMES.get(d.layer.dtype)
    if dt is None:
        raise ValueError("descriptor dtype")
    _check_tensor(x, "x", None, dtype=dt, numel=n)
    for wdict in weights_list:
        _check_weights(d.layer, wdict, x.device)
    if bpt_stack_saved_size(d):
        _check_tensor(saved, "saved", x.device, min_bytes=bpt_stack_saved_size(d))
    _check_tensor(workspace, "workspace", x.device,
                  min_bytes=bpt_stack_workspace_size(d, backward))
    return n, dt


def bpt_stack_forward(desc, x, weights_list, y, saved, workspace, stream=None) -> int:
    """Raw call: weights_list holds one weight dict per layer (checked first)."""
    d = _stack_desc(desc)
    n, dt = _check_stack(d, x, weights_list, saved, workspace, False)
    _check_tensor(y, "y", x.device, dtype=dt, numel=n)
    ws_arr = (BptLayerWeights * d.n_layers)(*[_weights_struct(w) for w in weights_list])
    return load_library().bpt_stack_forward(
        ctypes.byref(d), _ptr(x), ws_arr, _ptr(y), _ptr(saved), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))


def bpt_stack_backward(desc, x, weights_list, saved, dy, dx, grads_list, workspace,
                       accumulate=False, stream=None) -> int:
    """Raw call: grads_list holds one dict of fp32 gradients per layer."""
    d = _stack_desc(desc)
    n, dt = _check_stack(d, x, weights_list, saved, workspace, True)
    _check_tensor(dy, "dy", x.device, dtype=dt, numel=n)
    _check_tensor(dx, "dx", x.device, dtype=dt, numel=n)
    if len(grads_list) != d.n_layers:
        raise ValueError(f"{len(grads_list)} gradient tables for {d.n_layers} layers")
    shapes = weight_shapes_of(d.layer)
    for grads in grads_list:
        for g, tns in grads.items():
            if tns is None:
                continue
            if g not in GRAD_NAMES or g[1:] not in shapes:
                raise ValueError(f"{g} is not a gradient of this layer")
            _check_tensor(tns, g, x.device, dtype="float32", shape=shapes[g[1:]])
    g_arr = (BptLayerGrads * d.n_layers)(*[
        BptLayerGrads(**{k: _ptr(gr.get(k)) for k in GRAD_NAMES}, accumulate=int(accumulate),
                      reserved=0) for gr in grads_list])
    ws_arr = (BptLayerWeights * d.n_layers)(*[_weights_struct(w) for w in weights_list])
    return load_library().bpt_stack_backward(
        ctypes.byref(d), _ptr(x), ws_arr, _ptr(saved), _ptr(dy), _ptr(dx), g_arr, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))


def _alloc_aligned_bytes(n: int, device):
    """A byte tensor whose data pointer is 256-byte aligned (torch's caching
    allocator returns such blocks)."""
    t = _alloc_bytes(n, device)
    if t.data_ptr() % 256:
        raise RuntimeError("allocation not 256-byte aligned")
    return t


def stack_forward(cfg: StackConfig, x, weights_list, stream=None):
    """y, saved = stack_forward(cfg, x, weights_list): allocates what it needs."""
    import torch
    d = cfg.desc()
    st = bpt_stack_validate(d)
    if st:
        raise BptError(st, "bpt_stack_validate")
    y = torch.empty_like(x)
    saved = _alloc_aligned_bytes(bpt_stack_saved_size(d), x.device)
    ws = _alloc_aligned_bytes(bpt_stack_workspace_size(d, False), x.device)
    st = bpt_stack_forward(d, x, weights_list, y, saved, ws, stream)
    if st:
        raise BptError(st, "bpt_stack_forward")
    return y, saved


def stack_backward(cfg: StackConfig, x, weights_list, saved, dy, stream=None):
    """dx, grads_list = stack_backward(...): fp32 gradients for every layer."""
    import torch
    d = cfg.desc()
    dx = torch.empty_like(x)
    grads_list = [{k: torch.empty(s, dtype=torch.float32, device=x.device)
                   for k, s in grad_shapes(cfg.layer, w).items()} for w in weights_list]
    ws = _alloc_aligned_bytes(bpt_stack_workspace_size(d, True), x.device)
    st = bpt_stack_backward(d, x, weights_list, saved, dy, dx, grads_list, ws, False, stream)
    if st:
        raise BptError(st, "bpt_stack_backward")
    return dx, grads_list
