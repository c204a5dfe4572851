"""GPU checks of the HIP layer (through the C ABI) against closed forms and
exact invariants, independent of the oracle's layer code:

* Causal prefix ("Blockwise Parallel Transformer for Long Context Large
  Models", §3.4: a causal row sees only keys at or before it): the output on
  the first n positions does not depend on later positions, so
  y(x[:n]) = y(x)[:n]. Bit for bit when n is a multiple of the 128-row query
  tile (every kernel then runs the same arithmetic on those rows); within
  rounding otherwise (a wave's rare rescale of the running maximum is decided
  over its 32 rows, some of which differ).
* Zero query projection: every score is 0, so each row's softmax is uniform
  over the keys it may see (BPT §3.4, Eq. 3 with equal scores). The saved
  base-2 log-sum-exp is then exactly log2(number of visible keys), and the
  attention output is the running mean of V.
* Head permutation: relabelling the heads (query heads with their KV group,
  and the matching rows of W_o) leaves y unchanged up to the order of the
  O-projection's sum.
* NaN propagation: a NaN input row makes its own output NaN, leaves the rows
  of earlier query tiles bit-identical, and the backward still returns.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from harness import Inputs, rel_l2, run_gpu, to_device, to_host64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _truncated(t: wl.Tensor, n: int) -> wl.Tensor:
    return wl.Tensor(t.f32[:, :n].copy(), t.storage[:, :n].copy(), t.dtype)


def _forward(sh, x, w):
    import memory_efficient_long_amd as bpt
    cfg = bpt.LayerConfig.from_shape(sh)
    xd = to_device(x)
    wd = {k: to_device(v) for k, v in w.items()}
    y, saved = bpt.forward(cfg, xd, wd)
    torch.cuda.synchronize()
    return y, saved


PREFIX = ["llama8b-small", "gpt1b-small", "bf16-d64-gqa-rope-window-dropout", "f32-d64-window"]


@pytest.mark.parametrize("name", PREFIX)
@pytest.mark.parametrize("n", [256, 208])
def test_causal_prefix(name, n):
    sh = wl.SMALL[name]
    _say(f"[prefix] {name} s={sh.seq_len} n={n}")
    inp = Inputs(sh, bias_std=0.2 if sh.has_bias else 0.0, norm_std=0.2)
    y_full, _ = _forward(sh, inp.x, inp.w)
    short = sh.replace(seq_len=n, q_block=128 if n % 128 == 0 else n // 2, kv_block=n)
    y_short, _ = _forward(short, _truncated(inp.x, n), inp.w)
    head = y_full[:, :n]
    if n % 128 == 0:
        assert torch.equal(y_short, head)
        return
    err = rel_l2(to_host64(y_short), to_host64(head))
    _say(f"  rel L2 {err:.2e}")
    assert err <= (1e-6 if sh.dtype == "f32" else 2e-3), err


def _saved_o_lse(sh, saved):
    """The saved state: O [b, s, H d] in the storage dtype, then (at the next
    256-byte boundary) the base-2 log-sum-exp [b, H, s] in fp32."""
    b, s, H, d = sh.batch, sh.seq_len, sh.n_heads, sh.head_dim
    esz = 2 if sh.dtype == "bf16" else 4
    o_bytes = b * s * H * d * esz
    raw = saved[:o_bytes]
    o = (raw.view(torch.bfloat16) if sh.dtype == "bf16" else raw.view(torch.float32))
    off = (o_bytes + 255) // 256 * 256
    lse = saved[off:off + b * H * s * 4].view(torch.float32)
    return to_host64(o).reshape(b, s, H, d), to_host64(lse).reshape(b, H, s)


ZERO_Q = ["llama8b-small", "gpt1b-small-chunked", "bf16-d64-noncausal", "bf16-d128-window",
          "f32-d64-window", "f32-d64-gqa-rope-noncausal"]


@pytest.mark.parametrize("name", ZERO_Q)
def test_zero_query_projection_closed_form(name):
    from oracle import bpt_oracle as orc
    sh = wl.SMALL[name]
    H, Hkv, d, s = sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.seq_len
    _say(f"[zero q] {name} s={s} H={H}/{Hkv} d={d} causal={sh.causal} window={sh.window}")
    inp = Inputs(sh, bias_std=0.2 if sh.has_bias else 0.0, norm_std=0.2)
    w = dict(inp.w)
    w["w_qkv"] = wl.scaled(w["w_qkv"], 0.0, cols=slice(0, H * d))
    if "b_qkv" in w:
        w["b_qkv"] = wl.scaled(w["b_qkv"], 0.0, cols=slice(0, H * d))
    _, saved = _forward(sh, inp.x, w)
    o, lse = _saved_o_lse(sh, saved)
    i = np.arange(s)
    if not sh.causal:
        count = np.full(s, s, dtype=np.float64)
    elif sh.window:
        count = np.minimum(i + 1, sh.window).astype(np.float64)
    else:
        count = (i + 1).astype(np.float64)
    want = np.broadcast_to(np.log2(count), lse.shape)
    err_lse = float(np.max(np.abs(lse - want) / np.maximum(want, 1.0)))
    # running mean of V (float64, from the storage-rounded inputs)
    sp = orc.spec_of(sh)
    x = inp.x.f64()[0]
    g1 = w["n1_g"].f64()
    b1 = w["n1_b"].f64() if "n1_b" in w else None
    xn, _, _ = orc.norm_forward(x, g1, b1, sp.norm, sp.eps)
    wv = w["w_qkv"].f64()[:, (H + Hkv) * d:]
    bv = w["b_qkv"].f64()[(H + Hkv) * d:] if "b_qkv" in w else 0.0
    v = (xn @ wv + bv).reshape(s, Hkv, d)
    csum = np.cumsum(v, axis=0)
    if not sh.causal:
        mean = np.broadcast_to(csum[-1] / s, v.shape)
    else:
        lo = np.maximum(i - sh.window, -1) if sh.window else np.full(s, -1)
        before = np.where(lo[:, None, None] >= 0, csum[np.maximum(lo, 0)], 0.0)
        mean = (csum - before) / count[:, None, None]
    ref = np.repeat(mean, H // Hkv, axis=1)          # query head hq reads KV head hq // G
    err_o = rel_l2(o[0], ref)
    _say(f"  lse max rel err {err_lse:.2e}; O rel L2 {err_o:.2e}")
    assert err_lse <= 1e-6, err_lse
    assert err_o <= (1e-5 if sh.dtype == "f32" else 1e-2), err_o


def _permute_heads(sh, w, perm_kv):
    """Relabel KV head k as perm_kv[k] (with its query group, in order) and
    permute the rows of W_o the same way."""
    H, Hkv, d = sh.n_heads, sh.n_kv_heads, sh.head_dim
    G = H // Hkv
    qperm = np.concatenate([np.arange(G) + G * k for k in perm_kv])   # new head j <- old qperm[j]
    cols_q = np.concatenate([np.arange(d) + d * h for h in qperm])
    cols_k = H * d + np.concatenate([np.arange(d) + d * k for k in perm_kv])
    cols_v = (H + Hkv) * d + np.concatenate([np.arange(d) + d * k for k in perm_kv])
    cols = np.concatenate([cols_q, cols_k, cols_v])
    out = dict(w)
    t = w["w_qkv"]
    out["w_qkv"] = wl.Tensor(t.f32[:, cols].copy(), t.storage[:, cols].copy(), t.dtype)
    if "b_qkv" in w:
        t = w["b_qkv"]
        out["b_qkv"] = wl.Tensor(t.f32[cols].copy(), t.storage[cols].copy(), t.dtype)
    t = w["w_o"]
    out["w_o"] = wl.Tensor(t.f32[cols_q].copy(), t.storage[cols_q].copy(), t.dtype)
    return out


@pytest.mark.parametrize("name", ["llama8b-small", "gpt1b-small-chunked", "f32-d64-window"])
def test_head_permutation_invariance(name):
    sh = wl.SMALL[name]
    _say(f"[heads] {name} H={sh.n_heads}/{sh.n_kv_heads}")
    inp = Inputs(sh, bias_std=0.2 if sh.has_bias else 0.0, norm_std=0.2)
    y0, _ = _forward(sh, inp.x, inp.w)
    perm = np.arange(sh.n_kv_heads)[::-1].copy()
    y1, _ = _forward(sh, inp.x, _permute_heads(sh, inp.w, perm))
    err = rel_l2(to_host64(y1), to_host64(y0))
    _say(f"  rel L2 {err:.2e}")
    assert err <= (1e-6 if sh.dtype == "f32" else 2e-3), err


@pytest.mark.parametrize("name", ["gpt1b-small", "f32-d64-window"])
def test_nan_input_row(name):
    sh = wl.SMALL[name]
    j = 300
    _say(f"[nan] {name} s={sh.seq_len} row {j}")
    inp = Inputs(sh, bias_std=0.2 if sh.has_bias else 0.0, norm_std=0.2)
    clean = run_gpu(inp, backward=False)["y"]
    vals = inp.x.f32.copy()
    vals[:, j, :] = np.nan
    inp.x = wl.Tensor(vals, vals.copy() if sh.dtype == "f32" else
                      wl.round_to_bf16_bits(vals), sh.dtype)
    got = run_gpu(inp)           # forward and backward must return
    y = got["y"]
    q0 = 128 * (j // 128)        # rows of earlier query tiles never see key j
    assert np.array_equal(y[:, :q0], clean[:, :q0])
    assert np.all(np.isnan(y[:, j]))
    assert np.isnan(got["dx"]).any()
