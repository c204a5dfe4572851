"""Pins for the LM-head cross-entropy oracle (oracle/lm_head_oracle.py), each
independent of the oracle's own code: PyTorch's linear and cross_entropy with
autograd, central finite differences, the W = 0 closed form, shift invariance
of the softmax, and row grouping."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import lm_head_oracle as lmo


def _case(n=37, h=16, V=48, seed=3, ignore=(5, 20)):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, h))
    w = rng.standard_normal((h, V)) / np.sqrt(h)
    t = rng.integers(0, V, n)
    for i in ignore:
        t[i] = -1
    g = rng.standard_normal(n)
    return z, w, t, g


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("row_group", [lmo.ROW_GROUP, 5])
def test_matches_torch_cross_entropy_and_autograd(row_group, monkeypatch):
    monkeypatch.setattr(lmo, "ROW_GROUP", row_group)
    z, w, t, g = _case()
    out = lmo.lm_head_ce(z, w, t, g)
    tz = torch.tensor(z, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    logits = F.linear(tz, tw.T)
    loss = F.cross_entropy(logits, torch.tensor(t), reduction="none", ignore_index=-1)
    assert _rel(out["loss"], loss.detach().numpy()) < 1e-13
    assert _rel(out["lse"], torch.logsumexp(logits, dim=1).detach().numpy()) < 1e-13
    (loss * torch.tensor(g)).sum().backward()
    assert _rel(out["dz"], tz.grad.numpy()) < 1e-12
    assert _rel(out["dw"], tw.grad.numpy()) < 1e-12
    # ignored rows: no loss, no gradient
    assert out["loss"][5] == 0.0 and np.all(out["dz"][5] == 0.0)


def test_central_differences():
    z, w, t, g = _case(n=7, h=5, V=9, ignore=(2,))
    out = lmo.lm_head_ce(z, w, t, g)
    eps = 1e-6

    def obj(zz, ww):
        return float(np.dot(lmo.lm_head_ce(zz, ww, t)["loss"], g))

    for arr, grad in ((z, out["dz"]), (w, out["dw"])):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            orig = arr[idx]
            arr[idx] = orig + eps
            fp = obj(z, w)
            arr[idx] = orig - eps
            fm = obj(z, w)
            arr[idx] = orig
            num[idx] = (fp - fm) / (2 * eps)
        assert _rel(grad, num) < 1e-6


def test_zero_weights_closed_form():
    """W = 0: every logit is 0, so loss = ln V on valid rows, dz = 0 and
    dW = z^T ((1/V) - onehot(t)) g."""
    z, w, t, g = _case()
    V = w.shape[1]
    out = lmo.lm_head_ce(z, np.zeros_like(w), t, g)
    valid = t >= 0
    assert np.allclose(out["loss"][valid], np.log(V), rtol=0, atol=1e-14)
    assert np.all(out["loss"][~valid] == 0.0)
    assert np.all(out["dz"] == 0.0)
    dl = np.full((len(t), V), 1.0 / V)
    dl[np.arange(len(t)), np.where(valid, t, 0)] -= 1.0
    dl *= np.where(valid, g, 0.0)[:, None]
    assert _rel(out["dw"], z.T @ dl) < 1e-13


def test_column_shift_invariance():
    """Adding one vector u to every column of W shifts each row's logits by a
    constant (z_i . u): the loss and dz do not change (softmax is
    shift-invariant and each row of dlogits sums to zero)."""
    z, w, t, g = _case()
    u = np.random.default_rng(9).standard_normal(w.shape[0])
    a = lmo.lm_head_ce(z, w, t, g)
    b = lmo.lm_head_ce(z, w + u[:, None], t, g)
    assert _rel(b["loss"], a["loss"]) < 1e-12
    assert _rel(b["dz"], a["dz"]) < 1e-11


def test_out_of_range_targets_are_ignored():
    z, w, t, g = _case(ignore=())
    V = w.shape[1]
    t2 = t.copy()
    t2[[1, 4]] = [V, -7]
    out = lmo.lm_head_ce(z, w, t2, g)
    assert out["loss"][1] == 0.0 and out["loss"][4] == 0.0
    assert np.all(out["dz"][[1, 4]] == 0.0)
