"""CPU oracle for the blockwise LM head with cross-entropy loss: forward and
backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. The HIP
library never calls it, and it shares no code with the HIP path.

What it computes
----------------
"Blockwise Parallel Transformer for Long Context Large Models", §3.4 (the
walkthrough's handling of the cross-entropy loss): the output layer maps every
position's hidden vector to one score per vocabulary entry (the logits) and
the loss of a position is -log softmax(logits)[target]; blockwise evaluation
gives the same values without holding all positions' logits at once. "Training
memory: model states, activations and checkpointing", §3 (the logits): the
loss is computed in fp32 (here float64). Written plainly, per row i:

    logits_i = z_i W                         (W is [h, V], y = x W convention)
    lse_i    = m_i + log sum_j exp(logits_ij - m_i),  m_i = max_j logits_ij
    loss_i   = lse_i - logits_i[t_i]

A target outside [0, V) (e.g. -1 for padding) marks an ignored row: loss 0 and
no gradient.

Backward ("Training memory", §2 per-operation rules: the softmax rule and the
linear rule), with g_i the cotangent of loss_i:

    dlogits_ij = g_i (softmax(logits_i)_j - [j == t_i])     (0 for ignored rows)
    dz = dlogits W^T,   dW = z^T dlogits

Rows are evaluated in groups of ROW_GROUP so that only a group's logits exist
at a time (the definition is per row, so grouping changes nothing else).

Pins: tests/test_oracle_lm_head.py (PyTorch linear + cross_entropy with
autograd, central finite differences, the W = 0 closed form, invariance of the
loss and dz under adding one vector to every column of W, row grouping).
"""
from __future__ import annotations

import numpy as np

__all__ = ["lm_head_ce", "ROW_GROUP"]

ROW_GROUP = 2048


def lm_head_ce(z, w, targets, g=None):
    """Per-row loss (and, with the cotangent g of the losses, dz and dW).

    z [n, h], w [h, V], targets int [n]. Returns {"loss": [n], "lse": [n]} and
    with g also "dz" [n, h] and "dw" [h, V]. Everything in float64."""
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    n, _ = z.shape
    V = w.shape[1]
    valid = (t >= 0) & (t < V)
    loss = np.zeros(n)
    lse = np.zeros(n)
    dz = dw = None
    if g is not None:
        g = np.asarray(g, dtype=np.float64)
        dz = np.zeros_like(z)
        dw = np.zeros_like(w)
    for a in range(0, n, ROW_GROUP):
        b = min(a + ROW_GROUP, n)
        logits = z[a:b] @ w
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        ssum = e.sum(axis=1, keepdims=True)
        lse[a:b] = (m + np.log(ssum))[:, 0]
        rows = np.arange(b - a)
        tv = np.where(valid[a:b], t[a:b], 0)
        loss[a:b] = np.where(valid[a:b], lse[a:b] - logits[rows, tv], 0.0)
        if g is None:
            continue
        p = e / ssum
        p[rows, tv] -= 1.0
        dl = p * np.where(valid[a:b], g[a:b], 0.0)[:, None]
        dz[a:b] = dl @ w.T
        dw += z[a:b].T @ dl
    out = {"loss": loss, "lse": lse}
    if g is not None:
        out["dz"] = dz
        out["dw"] = dw
    return out
