"""CPU oracle for one Blockwise Parallel Transformer layer: forward and backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. The HIP
library never calls it, and it shares no code with the HIP path (it imports
nothing from the package).

What it computes
----------------
"Blockwise Parallel Transformer for Long Context Large Models", §3.1 (reader
orientation) and §3.4 (the final remarks on exactness): BPT only reschedules a
standard transformer layer (blockwise attention with an online softmax, then the
feed-forward network per query block) and produces the same outputs up to
floating-point rounding. The oracle is therefore the standard layer written out
plainly, in float64:

* pre-norm residual layer, h1 = x + Attn(Norm1(x)) W_o + b_o and
  y = h1 + FFN(Norm2(h1));
* attention per head is softmax(Q K^T / sqrt(d)) V (§3.4, "Blockwise
  Self-Attention with Online Softmax", the scaled dot-product formula), with the
  softmax taken explicitly over each full score row: shift by the row maximum,
  exponentiate, divide by the row sum (the numerically stable form given there);
* causal masking sets scores with key index > query index to -inf (§3.4, the
  chunk-bias function of the implementation walkthrough);
* FFN(z) = act(z W1 + b1) W2 + b2 (§2, the position-wise FFN equation) with
  act = ReLU, exact-erf GeLU, or SwiGLU silu(z W_gate) * (z W_up) as used by the
  Llama-shaped workloads ("Untied Ulysses: Memory-Efficient Context Parallelism
  via Headwise Chunking", §5 experimental setup: Llama3-8B);
* grouped-query attention maps query head q to KV head q // G (Untied Ulysses,
  §3.4, the GQA scheduling discussion), and RoPE rotates the pairs (2i, 2i+1)
  of Q and K by p * base^(-2i/d) at position p.

The backward follows the per-operation rules of "Training memory: model states,
activations and checkpointing", §2 ("every operation keeps what its backward
pass needs"): linear dW = x^T dy; element-wise g'(x) * dy; softmax
dz = p * (pbar - <p, pbar>); LayerNorm via the normalised input and row
statistics; products of two activations differentiate against the other
factor; the residual copies the gradient to both branches. The running-max
``stop_gradient`` of the BPT implementation (§3.4) makes the max a pure shift,
so the exact softmax gradient applies.

Readings where the pages are silent (each also listed in the design doc): pre-norm
placement; W_o included; biases only on the GPT-shaped workloads; exact-erf
GeLU; eps = 1e-5 with biased variance; interleaved RoPE pairs; no dropout;
kv head = q // G; batch elements are independent sequences.

Parity pins live in ``tests/test_oracle_*.py``: an independent composition of
PyTorch library routines with autograd, central finite differences, an
independent blockwise online-softmax recurrence (Algorithm 1), closed forms and
invariants. Every function here is pinned by at least one of them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
from scipy.special import erf

__all__ = ["Spec", "spec_of", "layer", "stack", "norm_forward", "norm_backward", "rope_rotate",
           "attention_probs", "philox4x32_10", "dropout_keep", "dropout_threshold"]


@dataclasses.dataclass(frozen=True)
class Spec:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    norm: str                      # "layernorm" | "rmsnorm"
    ffn: str                       # "relu" | "gelu" | "swiglu"
    causal: bool = True
    rope_base: Optional[float] = None
    eps: float = 1e-5
    window: int = 0                # causal sliding window W (0: none)
    dropout_p: float = 0.0         # attention-probability dropout (0: none)
    seed: int = 0                  # 64-bit seed of the dropout masks


def spec_of(shape) -> Spec:
    """Spec from any object carrying the layer's shape attributes."""
    return Spec(shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
                shape.norm, shape.ffn, shape.causal, shape.rope_base,
                getattr(shape, "norm_eps", 1e-5), getattr(shape, "window", 0),
                getattr(shape, "dropout_p", 0.0), getattr(shape, "seed", 0))


# --------------------------------------------------------------------------- norms
def norm_forward(x, g, b, kind, eps):
    """LayerNorm (mean, biased variance) or RMSNorm over the last axis.
    Returns (output, normalised input xhat, per-row reciprocal std)."""
    if kind == "layernorm":
        mu = x.mean(axis=-1, keepdims=True)
        var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
        rstd = 1.0 / np.sqrt(var + eps)
        xhat = (x - mu) * rstd
        out = xhat * g + (b if b is not None else 0.0)
    elif kind == "rmsnorm":
        rstd = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
        xhat = x * rstd
        out = xhat * g
    else:
        raise ValueError(kind)
    return out, xhat, rstd


def norm_backward(dout, xhat, rstd, g, kind):
    """Gradient of norm_forward w.r.t. its input, scale and shift (Training
    memory, §2: LayerNorm keeps its input and per-row statistics)."""
    gx = dout * g
    if kind == "layernorm":
        dx = rstd * (gx - gx.mean(axis=-1, keepdims=True)
                     - xhat * (gx * xhat).mean(axis=-1, keepdims=True))
        dshift = dout.sum(axis=0)
    else:
        dx = rstd * (gx - xhat * (gx * xhat).mean(axis=-1, keepdims=True))
        dshift = None
    dscale = (dout * xhat).sum(axis=0)
    return dx, dscale, dshift


# --------------------------------------------------------------------------- RoPE
def rope_rotate(t, positions, base, sign=+1.0):
    """Rotate the pairs (2i, 2i+1) of the last axis of t [n, heads, d] by
    sign * p * base^(-2i/d), p the row's position. sign=-1 is the inverse
    (transpose) rotation, used by the backward."""
    d = t.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    ang = sign * np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    even, odd = t[..., 0::2], t[..., 1::2]
    out = np.empty_like(t)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


# --------------------------------------------------------------------------- attention
def attention_probs(q_h, k_h, rows, causal, window=0):
    """Softmax(q k^T / sqrt(d)) for query rows ``rows`` (positions) against keys
    0..n-1, one explicit score row at a time: shift by the row max, exponentiate,
    normalise by the row sum. The positional bias is -inf for keys after the
    query (causal) and, with a window W, for keys W or more positions before
    it ("Blockwise Parallel Transformer", §3.4: a bias from the absolute
    positions of the query and key, -inf where a key is not visible)."""
    d = q_h.shape[-1]
    n = k_h.shape[0]
    scores = (q_h @ k_h.T) / np.sqrt(d)
    rr = np.asarray(rows)[:, None]
    jj = np.arange(n)[None, :]
    if causal:
        scores = np.where(rr >= jj, scores, -np.inf)
    if window:
        scores = np.where(rr - jj < window, scores, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    return e / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------- dropout
# Dropout on the attention probabilities ("Training memory", §3: the layer's
# dropout after the softmax, whose s x s mask FlashAttention regenerates from
# the saved random-number state instead of storing it). The mask comes from a
# counter-based generator, Philox4x32 with 10 rounds (Salmon, Moraes, Dror and
# Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11), so any block of
# (query, key) pairs can be regenerated on its own: element (i, j) of head h in
# sequence b uses the counter (i // 4, j // 4, h, b) under the key (low, high
# 32 bits of the seed) and byte 4 (i % 4) + (j % 4) of the 16 output bytes
# (word i % 4, little-endian byte j % 4); it is kept iff that byte is at least
# t = round(256 p), so the effective drop probability is t / 256 and kept
# probabilities are scaled by 256 / (256 - t).
_PHILOX_M = (np.uint64(0xD2511F53), np.uint64(0xCD9E8D57))
_PHILOX_W = (np.uint64(0x9E3779B9), np.uint64(0xBB67AE85))
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 bijection of the 128-bit counters (c0..c3, arrays of
    uint32 values) under the key (k0, k1): ten rounds of two 32 x 32 -> 64-bit
    products, xors with the other counter words and the round key, and a Weyl
    increment of the key."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _U32 for c in (c0, c1, c2, c3))
    k0, k1 = np.uint64(k0) & _U32, np.uint64(k1) & _U32
    for _ in range(10):
        p0 = _PHILOX_M[0] * c0
        p1 = _PHILOX_M[1] * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _U32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _U32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + _PHILOX_W[0]) & _U32
        k1 = (k1 + _PHILOX_W[1]) & _U32
    return c0, c1, c2, c3


def dropout_threshold(p):
    return int(round(256.0 * float(p)))


def dropout_keep(rows, n_keys, head, batch, seed, thr):
    """Boolean keep mask [len(rows), n_keys] for query positions ``rows``."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    ii, jj = np.broadcast_arrays(i, j)
    words = philox4x32_10(ii // 4, jj // 4, np.full(ii.shape, head), np.full(ii.shape, batch),
                          int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    w = np.choose((ii % 4).astype(np.int64), words)
    byte = (w >> (np.uint64(8) * (jj % 4).astype(np.uint64))) & np.uint64(0xFF)
    return byte >= np.uint64(thr)


# Query rows per explicit score matrix. The softmax is defined row by row, so
# evaluating the rows in groups changes nothing but the size of the temporary
# (a group x keys matrix instead of rows x keys); with the causal mask a group
# needs only the keys up to its last row, since every later key has weight
# exactly zero (exp(-inf) = 0) for all of its rows.
ROW_GROUP = 2048


def _row_groups(rows, n, causal):
    """(slice of ``rows``, number of keys) for each group of query rows."""
    for a in range(0, len(rows), ROW_GROUP):
        sl = slice(a, min(a + ROW_GROUP, len(rows)))
        nk = int(rows[sl.stop - 1]) + 1 if causal else n
        yield sl, nk


# --------------------------------------------------------------------------- FFN
def _gelu(a):
    return 0.5 * a * (1.0 + erf(a / np.sqrt(2.0)))


def _gelu_grad(a):
    cdf = 0.5 * (1.0 + erf(a / np.sqrt(2.0)))
    pdf = np.exp(-0.5 * a * a) / np.sqrt(2.0 * np.pi)
    return cdf + a * pdf


def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


# --------------------------------------------------------------------------- layer
def _get(w, name, shape=None):
    v = w.get(name)
    if v is None:
        return None
    return np.asarray(v, dtype=np.float64)


def _sequence(x, w, sp: Spec, rows, dy, batch=0):
    """One sequence. x [s, h]; rows sorted positions where y is produced and
    where the cotangent dy [len(rows), h] lives (zero elsewhere)."""
    s, h = x.shape
    H, Hkv, d = sp.n_heads, sp.n_kv_heads, sp.head_dim
    G = H // Hkv
    r = len(rows)
    # Positions >= n can influence none of the requested rows when causal.
    n = rows[-1] + 1 if sp.causal else s
    xs = x[:n]

    wqkv = _get(w, "w_qkv")
    wq, wk, wv = wqkv[:, :H * d], wqkv[:, H * d:(H + Hkv) * d], wqkv[:, (H + Hkv) * d:]
    bqkv = _get(w, "b_qkv")
    if bqkv is None:
        bqkv = np.zeros(wqkv.shape[1])
    bq, bk, bv = bqkv[:H * d], bqkv[H * d:(H + Hkv) * d], bqkv[(H + Hkv) * d:]
    w_o, b_o = _get(w, "w_o"), _get(w, "b_o")
    w1, b1, w2, b2, w3 = (_get(w, k) for k in ("w_1", "b_1", "w_2", "b_2", "w_3"))
    g1, sh1, g2, sh2 = (_get(w, k) for k in ("n1_g", "n1_b", "n2_g", "n2_b"))

    # Norm1 and the QKV projection (K, V for every position that can be attended).
    xn, xhat1, rstd1 = norm_forward(xs, g1, sh1, sp.norm, sp.eps)
    q = (xn[rows] @ wq + bq).reshape(r, H, d)
    k = (xn @ wk + bk).reshape(n, Hkv, d)
    v = (xn @ wv + bv).reshape(n, Hkv, d)
    if sp.rope_base is not None:
        q = rope_rotate(q, rows, sp.rope_base)
        k = rope_rotate(k, np.arange(n), sp.rope_base)

    thr = dropout_threshold(sp.dropout_p)
    dscale = 256.0 / (256.0 - thr)

    def dropped(p, sl, nk, hq):
        """P with the dropout mask applied (kept entries scaled); P itself
        when there is no dropout."""
        if not thr:
            return p
        return p * dropout_keep(rows[sl], nk, hq, batch, sp.seed, thr) * dscale

    attn = np.empty((r, H, d))
    for hq in range(H):
        kv = hq // G
        for sl, nk in _row_groups(rows, n, sp.causal):
            p = attention_probs(q[sl, hq], k[:nk, kv], rows[sl], sp.causal, sp.window)
            attn[sl, hq] = dropped(p, sl, nk, hq) @ v[:nk, kv]
    attn2 = attn.reshape(r, H * d)

    h1 = x[rows] + attn2 @ w_o + (b_o if b_o is not None else 0.0)
    z, xhat2, rstd2 = norm_forward(h1, g2, sh2, sp.norm, sp.eps)
    if sp.ffn == "swiglu":
        gate = z @ w1 + (b1 if b1 is not None else 0.0)
        up = z @ w3
        u = gate * _sigmoid(gate) * up
    else:
        a = z @ w1 + (b1 if b1 is not None else 0.0)
        u = np.maximum(a, 0.0) if sp.ffn == "relu" else _gelu(a)
    y = h1 + u @ w2 + (b2 if b2 is not None else 0.0)
    if dy is None:
        return {"y": y}

    # ------------------------------------------------------------- backward
    dy = np.asarray(dy, dtype=np.float64)
    grads = {}
    grads["w_2"] = u.T @ dy
    if b2 is not None:
        grads["b_2"] = dy.sum(axis=0)
    du = dy @ w2.T
    if sp.ffn == "swiglu":
        sg = _sigmoid(gate)
        dgate = du * up * sg * (1.0 + gate * (1.0 - sg))
        dup = du * gate * sg
        grads["w_1"] = z.T @ dgate
        grads["w_3"] = z.T @ dup
        if b1 is not None:
            grads["b_1"] = dgate.sum(axis=0)
        dz = dgate @ w1.T + dup @ w3.T
    else:
        da = du * ((a > 0.0).astype(np.float64) if sp.ffn == "relu" else _gelu_grad(a))
        grads["w_1"] = z.T @ da
        if b1 is not None:
            grads["b_1"] = da.sum(axis=0)
        dz = da @ w1.T
    dh1_norm, grads["n2_g"], dn2b = norm_backward(dz, xhat2, rstd2, g2, sp.norm)
    if dn2b is not None:
        grads["n2_b"] = dn2b
    dh1 = dy + dh1_norm                       # residual copies the gradient

    grads["w_o"] = attn2.T @ dh1
    if b_o is not None:
        grads["b_o"] = dh1.sum(axis=0)
    dattn = (dh1 @ w_o.T).reshape(r, H, d)

    dq = np.zeros((r, H, d))
    dk = np.zeros((n, Hkv, d))
    dv = np.zeros((n, Hkv, d))
    for hq in range(H):
        kv = hq // G
        for sl, nk in _row_groups(rows, n, sp.causal):
            p = attention_probs(q[sl, hq], k[:nk, kv], rows[sl], sp.causal, sp.window)
            pd = dropped(p, sl, nk, hq)
            # the product with V used the dropped probabilities: its gradient
            # reaches P through the same mask and scale
            dpd = dattn[sl, hq] @ v[:nk, kv].T
            dv[:nk, kv] += pd.T @ dattn[sl, hq]
            dp = dpd if pd is p else dropped(dpd, sl, nk, hq)
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[sl, hq] = ds @ k[:nk, kv] / np.sqrt(d)
            dk[:nk, kv] += ds.T @ q[sl, hq] / np.sqrt(d)
    if sp.rope_base is not None:
        dq = rope_rotate(dq, rows, sp.rope_base, sign=-1.0)
        dk = rope_rotate(dk, np.arange(n), sp.rope_base, sign=-1.0)
    dq2, dk2, dv2 = dq.reshape(r, H * d), dk.reshape(n, Hkv * d), dv.reshape(n, Hkv * d)

    dwqkv = np.zeros_like(wqkv)
    dwqkv[:, :H * d] = xn[rows].T @ dq2
    dwqkv[:, H * d:(H + Hkv) * d] = xn.T @ dk2
    dwqkv[:, (H + Hkv) * d:] = xn.T @ dv2
    grads["w_qkv"] = dwqkv
    if _get(w, "b_qkv") is not None:
        grads["b_qkv"] = np.concatenate([dq2.sum(axis=0), dk2.sum(axis=0), dv2.sum(axis=0)])
    dxn = dk2 @ wk.T + dv2 @ wv.T
    dxn[rows] += dq2 @ wq.T

    dx_norm, grads["n1_g"], dn1b = norm_backward(dxn, xhat1, rstd1, g1, sp.norm)
    if dn1b is not None:
        grads["n1_b"] = dn1b
    dx = np.zeros((s, h))
    dx[:n] = dx_norm
    dx[rows] += dh1
    return {"y": y, "dx": dx, "grads": grads}


def layer(x, w: Dict[str, np.ndarray], sp: Spec, dy=None, rows=None):
    """The layer's forward and, when ``dy`` is given, its backward.

    x: [b, s, h]. w: weights by name (w_qkv [h,(H+2Hkv)d] packed Q|K|V with head
    k in columns [k d, (k+1) d) of each part; w_o [H d, h]; w_1 [h, f];
    w_2 [f, h]; w_3 [h, f] (SwiGLU up; w_1 is the gate); optional b_qkv, b_o,
    b_1, b_2; n1_g, n2_g and, for LayerNorm, n1_b, n2_b).

    rows: positions at which y is returned (default: all). dy: cotangent of y,
    [b, s, h] when rows is None, else [b, len(rows), h] (zero at every other
    position). Returns {"y": [b, r, h]} and, with dy, "dx" [b, s, h] and
    "grads" with the same names as w (summed over the batch).
    """
    x = np.asarray(x, dtype=np.float64)
    b, s, _ = x.shape
    rows = np.arange(s) if rows is None else np.asarray(sorted(set(int(i) for i in rows)))
    ys, dxs, grads = [], [], {}
    for bi in range(b):
        out = _sequence(x[bi], w, sp, rows, None if dy is None else dy[bi], batch=bi)
        ys.append(out["y"])
        if dy is not None:
            dxs.append(out["dx"])
            for kname, gval in out["grads"].items():
                grads[kname] = grads.get(kname, 0.0) + gval
    res = {"y": np.stack(ys)}
    if dy is not None:
        res["dx"] = np.stack(dxs)
        res["grads"] = grads
    return res


def stack(x, ws, sp: Spec, dy=None):
    """L layers applied in sequence, y = layer_L(... layer_1(x)), each with its
    own weights ws[l] ("Training memory", §3: the model is L such layers; the
    checkpointing schedule changes what is kept, never the values). The
    backward runs the layers in reverse, each layer's dx being the cotangent
    of the layer below. Returns {"y"} and, with dy, "dx" and "grads" (a list
    of per-layer gradient dicts)."""
    hs = [np.asarray(x, dtype=np.float64)]
    for w in ws:
        hs.append(layer(hs[-1], w, sp)["y"])
    if dy is None:
        return {"y": hs[-1]}
    g = np.asarray(dy, dtype=np.float64)
    grads = [None] * len(ws)
    for li in range(len(ws) - 1, -1, -1):
        out = layer(hs[li], ws[li], sp, dy=g)
        grads[li] = out["grads"]
        g = out["dx"]
    return {"y": hs[-1], "dx": g, "grads": grads}
