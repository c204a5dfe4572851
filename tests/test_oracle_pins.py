"""Pins for the CPU oracle, each independent of the oracle's own code.

* PyTorch library routines (layer_norm, rms_norm, linear, gelu, silu,
  scaled_dot_product_attention; RoPE as a complex multiplication) composed into
  the layer, and autograd through them, pin the forward and the hand-derived
  backward.
* Central finite differences of L = <y, dy> pin every gradient on tiny shapes.
* An independent blockwise online-softmax recurrence ("Blockwise Parallel
  Transformer for Long Context Large Models", §3.4 and Algorithm 1: running
  max, numerator and denominator rescaled per key-value block) pins attention
  for many block sizes.
* Closed forms and invariants: causal row 0, uniform attention as a prefix mean,
  softmax rows summing to one, GQA as replicated MHA, head permutation, RoPE
  identities, norm statistics, causality.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as wl
from oracle import bpt_oracle as orc

torch.set_default_dtype(torch.float64)


def _shape(name="t", s=8, h=8, H=2, Hkv=2, d=4, f=16, norm="layernorm", ffn="gelu",
           bias=True, rope=None, causal=True, window=0):
    return wl.LayerShape(name, 9, "f32", 1, s, h, H, Hkv, d, f, norm, ffn, bias, causal, rope,
                         s, s, H, window=window)


def _weights(sh, seed_shift=0):
    ws = wl.make_weights(sh.replace(wid=sh.wid + seed_shift), bias_std=0.2, norm_std=0.2)
    return {k: v.f64() for k, v in ws.items()}


def _inputs(sh, batch=1):
    sh = sh.replace(batch=batch)
    return wl.make_x(sh).f64(), wl.make_dy(sh).f64()


VARIANTS = {
    "gpt-relu": dict(norm="layernorm", ffn="relu", bias=True),
    "gpt-gelu": dict(norm="layernorm", ffn="gelu", bias=True),
    "llama-gqa-rope-swiglu": dict(norm="rmsnorm", ffn="swiglu", bias=False, H=4, Hkv=2, h=16,
                                   rope=10000.0),
    "llama-gqa-swiglu": dict(norm="rmsnorm", ffn="swiglu", bias=False, H=4, Hkv=1, h=16),
    "noncausal-gelu": dict(norm="layernorm", ffn="gelu", bias=True, causal=False),
    "window-gqa-rope": dict(norm="rmsnorm", ffn="swiglu", bias=False, H=4, Hkv=2, h=16,
                            rope=10000.0, window=3),
}


# ----------------------------------------------------------------- torch composition
def _torch_layer(x, w, sh):
    """The same layer assembled from PyTorch library routines (float64, CPU)."""
    H, Hkv, d, h = sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.hidden
    b, s, _ = x.shape
    if sh.norm == "layernorm":
        xn = F.layer_norm(x, (h,), w["n1_g"], w["n1_b"], eps=sh.norm_eps)
    else:
        xn = F.rms_norm(x, (h,), w["n1_g"], eps=sh.norm_eps)
    qkv = F.linear(xn, w["w_qkv"].T, w.get("b_qkv"))
    q, k, v = torch.split(qkv, [H * d, Hkv * d, Hkv * d], dim=-1)
    q = q.reshape(b, s, H, d)
    k = k.reshape(b, s, Hkv, d)
    v = v.reshape(b, s, Hkv, d)
    if sh.rope_base is not None:
        pos = torch.arange(s, dtype=torch.float64)
        inv = sh.rope_base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
        rot = torch.polar(torch.ones(s, d // 2), pos[:, None] * inv[None, :])[None, :, None, :]

        def apply(t):
            tc = torch.view_as_complex(t.reshape(*t.shape[:-1], d // 2, 2).contiguous())
            return torch.view_as_real(tc * rot).reshape(t.shape)
        q, k = apply(q), apply(k)
    G = H // Hkv
    k = k.repeat_interleave(G, dim=2)
    v = v.repeat_interleave(G, dim=2)
    if sh.window:
        i = torch.arange(s)[:, None]
        j = torch.arange(s)[None, :]
        mask = (j <= i) & (i - j < sh.window)
        o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2),
                                           v.transpose(1, 2), attn_mask=mask)
    else:
        o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2),
                                           v.transpose(1, 2), is_causal=sh.causal)
    o = o.transpose(1, 2).reshape(b, s, H * d)
    h1 = x + F.linear(o, w["w_o"].T, w.get("b_o"))
    if sh.norm == "layernorm":
        z = F.layer_norm(h1, (h,), w["n2_g"], w["n2_b"], eps=sh.norm_eps)
    else:
        z = F.rms_norm(h1, (h,), w["n2_g"], eps=sh.norm_eps)
    if sh.ffn == "swiglu":
        u = F.silu(F.linear(z, w["w_1"].T, w.get("b_1"))) * F.linear(z, w["w_3"].T)
    elif sh.ffn == "gelu":
        u = F.gelu(F.linear(z, w["w_1"].T, w.get("b_1")))
    else:
        u = F.relu(F.linear(z, w["w_1"].T, w.get("b_1")))
    return h1 + F.linear(u, w["w_2"].T, w.get("b_2"))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("row_group", [orc.ROW_GROUP, 5])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_layer_matches_torch_library_and_autograd(variant, row_group, monkeypatch):
    # row_group 5 splits the 24 query rows into groups of 5 (the last one
    # ragged), each against only the keys up to its last row when causal.
    monkeypatch.setattr(orc, "ROW_GROUP", row_group)
    kw = dict(VARIANTS[variant])
    sh = _shape(s=24, d=8, f=48, **{**kw, "h": kw.get("h", 16)})
    w = _weights(sh)
    x, dy = _inputs(sh, batch=2)
    out = orc.layer(x, w, orc.spec_of(sh), dy=dy)

    tw = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    tx = torch.tensor(x, requires_grad=True)
    ty = _torch_layer(tx, tw, sh)
    assert _rel(out["y"], ty.detach().numpy()) < 1e-12
    (ty * torch.tensor(dy)).sum().backward()
    assert _rel(out["dx"], tx.grad.numpy()) < 1e-10
    assert set(out["grads"]) == set(w)
    for name, g in out["grads"].items():
        assert _rel(g, tw[name].grad.numpy()) < 1e-10, name


# ----------------------------------------------------------------- finite differences
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_backward_central_differences(variant):
    kw = dict(VARIANTS[variant])
    sh = _shape(**kw)
    w = _weights(sh, seed_shift=1)
    x, dy = _inputs(sh)
    sp = orc.spec_of(sh)
    out = orc.layer(x, w, sp, dy=dy)

    def loss(xx, ww):
        return float((orc.layer(xx, ww, sp)["y"] * dy).sum())

    eps = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd[idx] = (loss(xp, w) - loss(xm, w)) / (2 * eps)
    assert _rel(out["dx"], fd) < 1e-6
    for name, val in w.items():
        fdw = np.zeros_like(val)
        for idx in np.ndindex(val.shape):
            wp = dict(w)
            wm = dict(w)
            wp[name] = val.copy()
            wm[name] = val.copy()
            wp[name][idx] += eps
            wm[name][idx] -= eps
            fdw[idx] = (loss(x, wp) - loss(x, wm)) / (2 * eps)
        assert _rel(out["grads"][name], fdw) < 1e-6, name


# ----------------------------------------------------------------- blockwise recurrence
def _blockwise_attention(q, k, v, cq, ckv, causal):
    """Attention computed as the pages' blockwise schedule: an outer loop over
    query blocks, an inner loop over key-value blocks carrying a running max,
    an unnormalised numerator and a denominator; each new block's max rescales
    the carries by exp(old - new); the output is numerator / denominator."""
    s, d = q.shape
    out = np.zeros_like(q)
    for q0 in range(0, s, cq):
        qi = q[q0:q0 + cq]
        rows = np.arange(q0, min(q0 + cq, s))
        num = np.zeros_like(qi)
        den = np.zeros((len(rows), 1))
        run_max = np.full((len(rows), 1), -np.inf)
        for k0 in range(0, s, ckv):
            cols = np.arange(k0, min(k0 + ckv, s))
            sc = qi @ k[cols].T / np.sqrt(d)
            if causal:
                sc = np.where(rows[:, None] >= cols[None, :], sc, -np.inf)
            blk_max = sc.max(axis=1, keepdims=True)
            new_max = np.maximum(run_max, blk_max)
            safe = np.where(np.isfinite(new_max), new_max, 0.0)
            corr = np.where(np.isfinite(run_max), np.exp(run_max - safe), 0.0)
            e = np.exp(sc - safe)
            num = num * corr + e @ v[cols]
            den = den * corr + e.sum(axis=1, keepdims=True)
            run_max = new_max
        out[q0:q0 + cq] = num / den
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("cq,ckv", [(1, 1), (3, 16), (16, 3), (64, 64), (17, 200), (200, 200)])
def test_blockwise_recurrence_equals_oracle(cq, ckv, causal):
    rng = np.random.default_rng(3)
    s, d = 200, 16
    q, k, v = (rng.standard_normal((s, d)) * 1.5 for _ in range(3))
    ref = orc.attention_probs(q, k, np.arange(s), causal) @ v
    assert np.max(np.abs(_blockwise_attention(q, k, v, cq, ckv, causal) - ref)) < 1e-12


def test_attention_matches_sdpa():
    rng = np.random.default_rng(4)
    s, d = 96, 32
    q, k, v = (rng.standard_normal((s, d)) for _ in range(3))
    for causal in (True, False):
        ref = F.scaled_dot_product_attention(*(torch.tensor(t)[None] for t in (q, k, v)),
                                             is_causal=causal)[0].numpy()
        got = orc.attention_probs(q, k, np.arange(s), causal) @ v
        assert np.max(np.abs(got - ref)) < 1e-13


# ----------------------------------------------------------------- closed forms, invariants
def test_softmax_rows_and_shift_invariance():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    p = orc.attention_probs(q, k, np.arange(40), True)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14
    assert np.all(np.triu(p, 1) == 0.0)
    # Adding a per-row constant to every score leaves P unchanged: shift q by a
    # vector orthogonal to nothing is not available, so shift via an extra key
    # coordinate: append a column c_i to q and 1 to every k.
    c = rng.standard_normal((40, 1)) * 5
    q2 = np.concatenate([q, c * np.sqrt(9 / 8)], axis=1)
    k2 = np.concatenate([k * np.sqrt(9 / 8), np.ones((40, 1))], axis=1)
    p2 = orc.attention_probs(q2, k2, np.arange(40), True)
    assert np.max(np.abs(p2 - p)) < 1e-13


def test_causal_row0_and_prefix_mean():
    sh = _shape(s=16, h=16, H=2, d=8, f=32)
    w = _weights(sh)
    x, _ = _inputs(sh)
    sp = orc.spec_of(sh)
    # Uniform attention: W_Q = 0 and b_Q = 0 make every score 0, so the
    # attention output at row i is the mean of v_0..v_i.
    w0 = dict(w)
    w0["w_qkv"] = w["w_qkv"].copy()
    w0["w_qkv"][:, :16] = 0.0
    w0["b_qkv"] = w["b_qkv"].copy()
    w0["b_qkv"][:16] = 0.0
    w0["w_o"] = np.eye(16)
    w0["b_o"] = np.zeros(16)
    w0["w_2"] = np.zeros_like(w["w_2"])
    w0["b_2"] = np.zeros(16)
    y = orc.layer(x, w0, sp)["y"][0]
    xn, _, _ = orc.norm_forward(x[0], w["n1_g"], w["n1_b"], "layernorm", 1e-5)
    vv = xn @ w["w_qkv"][:, 32:] + w["b_qkv"][32:]
    prefix = np.cumsum(vv, axis=0) / np.arange(1, 17)[:, None]
    assert np.max(np.abs((y - x[0]) - prefix)) < 1e-12
    # Row 0 attends only to itself: its attention output is v_0 exactly.
    assert np.max(np.abs((y - x[0])[0] - vv[0])) < 1e-13


def test_causality_future_rows_do_not_matter():
    sh = _shape(s=20, h=16, H=2, d=8, f=32)
    w = _weights(sh)
    x, _ = _inputs(sh)
    sp = orc.spec_of(sh)
    y = orc.layer(x, w, sp)["y"]
    x2 = x.copy()
    x2[0, 11:] += 3.0
    y2 = orc.layer(x2, w, sp)["y"]
    assert np.array_equal(y[0, :11], y2[0, :11])
    assert np.max(np.abs(y[0, 11:] - y2[0, 11:])) > 1e-3


def test_gqa_equals_replicated_mha():
    sh = _shape(s=20, h=32, H=4, Hkv=2, d=8, f=32, norm="rmsnorm", ffn="swiglu", bias=False,
                rope=500000.0)
    w = _weights(sh)
    x, dy = _inputs(sh)
    out = orc.layer(x, w, orc.spec_of(sh), dy=dy)
    H, Hkv, d = 4, 2, 8
    G = H // Hkv
    wq = w["w_qkv"][:, :H * d]
    wk = w["w_qkv"][:, H * d:(H + Hkv) * d].reshape(-1, Hkv, d)
    wv = w["w_qkv"][:, (H + Hkv) * d:].reshape(-1, Hkv, d)
    rep = lambda t: np.repeat(t, G, axis=1).reshape(t.shape[0], -1)
    w_mha = dict(w)
    w_mha["w_qkv"] = np.concatenate([wq, rep(wk), rep(wv)], axis=1)
    sh_mha = sh.replace(n_kv_heads=H)
    out2 = orc.layer(x, w_mha, orc.spec_of(sh_mha), dy=dy)
    assert np.max(np.abs(out["y"] - out2["y"])) < 1e-12
    assert np.max(np.abs(out["dx"] - out2["dx"])) < 1e-12
    # The GQA K/V weight gradient is the replicated gradient summed over G.
    gk = out2["grads"]["w_qkv"][:, H * d:2 * H * d].reshape(-1, Hkv, G, d).sum(axis=2)
    assert np.max(np.abs(out["grads"]["w_qkv"][:, H * d:(H + Hkv) * d]
                         - gk.reshape(-1, Hkv * d))) < 1e-12


def test_head_permutation_invariance():
    sh = _shape(s=16, h=32, H=4, Hkv=4, d=8, f=32)
    w = _weights(sh)
    x, dy = _inputs(sh)
    sp = orc.spec_of(sh)
    perm = np.array([2, 0, 3, 1])
    d, H = 8, 4
    cols = np.concatenate([np.concatenate([np.arange(p * d, (p + 1) * d) + part * H * d
                                           for p in perm]) for part in range(3)])
    wp = dict(w)
    wp["w_qkv"] = w["w_qkv"][:, cols]
    wp["b_qkv"] = w["b_qkv"][cols]
    wp["w_o"] = w["w_o"][np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])]
    a = orc.layer(x, w, sp, dy=dy)
    b = orc.layer(x, wp, sp, dy=dy)
    assert np.max(np.abs(a["y"] - b["y"])) < 1e-12
    assert np.max(np.abs(a["dx"] - b["dx"])) < 1e-12


def test_rope_identities():
    rng = np.random.default_rng(6)
    t = rng.standard_normal((5, 3, 16))
    assert np.array_equal(orc.rope_rotate(t[:1], [0], 500000.0), t[:1])
    pos = np.array([0, 7, 1000, 65535, 12345])
    r = orc.rope_rotate(t, pos, 500000.0)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(t, axis=-1), atol=1e-12)
    assert np.max(np.abs(orc.rope_rotate(r, pos, 500000.0, sign=-1.0) - t)) < 1e-12
    # Relative position: <R_p q, R_r k> depends only on p - r.
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    for p, r_, shift in [(10, 3, 100), (65535, 0, -60000), (5, 5, 777)]:
        d1 = np.sum(orc.rope_rotate(q, [p], 1e4) * orc.rope_rotate(k, [r_], 1e4))
        d2 = np.sum(orc.rope_rotate(q, [p + shift], 1e4) * orc.rope_rotate(k, [r_ + shift], 1e4))
        assert abs(d1 - d2) < 1e-9


def test_norm_statistics():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((7, 64)) * 3 + 1
    out, _, _ = orc.norm_forward(x, np.ones(64), np.zeros(64), "layernorm", 1e-5)
    var = x.var(axis=1)
    assert np.max(np.abs(out.mean(axis=1))) < 1e-13
    assert np.max(np.abs(out.var(axis=1) - var / (var + 1e-5))) < 1e-12
    out, _, _ = orc.norm_forward(x, np.ones(64), None, "rmsnorm", 0.0)
    assert np.max(np.abs(np.sqrt((out ** 2).mean(axis=1)) - 1.0)) < 1e-13
    # LayerNorm's input gradient is orthogonal to the all-ones vector per row.
    _, xhat, rstd = orc.norm_forward(x, np.ones(64), np.zeros(64), "layernorm", 1e-5)
    dx, _, _ = orc.norm_backward(rng.standard_normal((7, 64)), xhat, rstd, np.ones(64),
                                 "layernorm")
    assert np.max(np.abs(dx.sum(axis=1))) < 1e-12


@pytest.mark.parametrize("row_group", [orc.ROW_GROUP, 3])
@pytest.mark.parametrize("variant", ["gpt-gelu", "llama-gqa-rope-swiglu", "noncausal-gelu"])
def test_row_subset_matches_dense(variant, row_group, monkeypatch):
    """The rows/sparse-cotangent mode (used at full sizes) equals the dense layer
    with dy zero outside the chosen rows."""
    monkeypatch.setattr(orc, "ROW_GROUP", row_group)
    kw = dict(VARIANTS[variant])
    sh = _shape(s=40, d=8, f=48, **{**kw, "h": kw.get("h", 16)})
    w = _weights(sh)
    x, dy = _inputs(sh)
    rows = np.array([0, 3, 17, 38])
    sp = orc.spec_of(sh)
    dy_masked = np.zeros_like(dy)
    dy_masked[:, rows] = dy[:, rows]
    dense = orc.layer(x, w, sp, dy=dy_masked)
    sub = orc.layer(x, w, sp, dy=dy[:, rows], rows=rows)
    assert np.max(np.abs(sub["y"] - dense["y"][:, rows])) < 1e-12
    assert np.max(np.abs(sub["dx"] - dense["dx"])) < 1e-12
    for name in dense["grads"]:
        assert np.max(np.abs(sub["grads"][name] - dense["grads"][name])) < 1e-12, name


def test_stack_central_differences():
    """A stack of two layers (own weights each): central differences of
    <y, dy> for the input and every parameter element of both layers."""
    sh = _shape(norm="layernorm", ffn="gelu", bias=True, s=6, h=8, f=12)
    ws = [_weights(sh, seed_shift=3), _weights(sh, seed_shift=4)]
    x, dy = _inputs(sh)
    sp = orc.spec_of(sh)
    out = orc.stack(x, ws, sp, dy=dy)
    eps = 1e-6

    def obj():
        return float((orc.stack(x, ws, sp)["y"] * dy).sum())

    def fd(arr):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            orig = arr[idx]
            arr[idx] = orig + eps
            fp = obj()
            arr[idx] = orig - eps
            fm = obj()
            arr[idx] = orig
            num[idx] = (fp - fm) / (2 * eps)
        return num

    assert _rel(out["dx"], fd(x)) < 1e-6
    for li in range(2):
        for name in ("w_qkv", "w_o", "w_1", "w_2", "n1_g", "n2_b", "b_qkv"):
            assert _rel(out["grads"][li][name], fd(ws[li][name])) < 1e-6, (li, name)
    # one layer is the layer itself
    one = orc.stack(x, ws[:1], sp, dy=dy)
    ref = orc.layer(x, ws[0], sp, dy=dy)
    assert np.array_equal(one["y"], ref["y"]) and np.array_equal(one["dx"], ref["dx"])


def test_sliding_window_closed_forms():
    """Window 1: each row sees only itself, so the attention output of a row
    is that row's value vector; a window of s or more is plain causal
    attention, bit for bit."""
    sh = _shape(s=12, d=4, f=16, window=1)
    w = _weights(sh)
    x, dy = _inputs(sh)
    w0 = dict(w)
    w0["w_o"] = np.eye(w["w_o"].shape[0])
    w0["b_o"] = np.zeros_like(w["b_o"])
    w0["w_2"] = np.zeros_like(w["w_2"])
    w0["b_2"] = np.zeros_like(w["b_2"])
    y = orc.layer(x, w0, orc.spec_of(sh))["y"]
    xn, _, _ = orc.norm_forward(x[0], w["n1_g"], w["n1_b"], "layernorm", 1e-5)
    H, d = sh.n_heads, sh.head_dim
    v = (xn @ w["w_qkv"] + w["b_qkv"])[:, 2 * H * d:]
    assert np.max(np.abs((y[0] - x[0]) - v)) < 1e-12
    full = _shape(s=12, d=4, f=16)
    a = orc.layer(x, w, orc.spec_of(full), dy=dy)
    b = orc.layer(x, w, orc.spec_of(full.replace(window=12)), dy=dy)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["dx"], b["dx"])


# ----------------------------------------------------------------- dropout
def test_philox_known_answers(repo_root):
    import json
    import os
    kat = json.load(open(os.path.join(repo_root, "tests", "golden", "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        c = [int(x, 16) for x in v["counter"]]
        k = [int(x, 16) for x in v["key"]]
        out = orc.philox4x32_10(*[np.array([x]) for x in c], *k)
        assert [int(o[0]) for o in out] == [int(x, 16) for x in v["output"]]


def test_dropout_mask_statistics():
    """Keep fraction within 4 standard deviations of 1 - t/256 and the bytes
    behind the masks uniform (chi-square over 256 bins), for two heads,
    batch entries and seeds."""
    for p, head, batch, seed in [(0.1, 0, 0, 1), (0.5, 3, 1, 2 ** 40 + 7)]:
        thr = orc.dropout_threshold(p)
        keep = orc.dropout_keep(np.arange(512), 512, head, batch, seed, thr)
        n = keep.size
        q = 1 - thr / 256
        assert abs(keep.mean() - q) < 4 * np.sqrt(q * (1 - q) / n)
    # byte uniformity of the underlying generator over consecutive counters
    c = np.arange(1 << 14)
    words = orc.philox4x32_10(c, c * 0 + 5, c * 0, c * 0, 123, 456)
    by = np.concatenate([(w[:, None] >> np.arange(0, 32, 8, dtype=np.uint64)) & 0xFF
                         for w in [np.asarray(x) for x in words]]).ravel()
    hist = np.bincount(by.astype(np.int64), minlength=256)
    exp = by.size / 256
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)


def _torch_attention_layer_with_masks(x, w, sh, masks, scale):
    """The layer of _torch_layer with explicit attention (library softmax)
    and the given dropout masks applied to the probabilities."""
    H, Hkv, d, h = sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.hidden
    b, s, _ = x.shape
    xn = F.layer_norm(x, (h,), w["n1_g"], w["n1_b"], eps=sh.norm_eps)
    qkv = F.linear(xn, w["w_qkv"].T, w.get("b_qkv"))
    q, k, v = torch.split(qkv, [H * d, Hkv * d, Hkv * d], dim=-1)
    G = H // Hkv
    q = q.reshape(b, s, H, d).transpose(1, 2)
    k = k.reshape(b, s, Hkv, d).repeat_interleave(G, dim=2).transpose(1, 2)
    v = v.reshape(b, s, Hkv, d).repeat_interleave(G, dim=2).transpose(1, 2)
    sc = q @ k.transpose(-1, -2) / d ** 0.5
    sc = sc.masked_fill(~torch.ones(s, s, dtype=torch.bool).tril(), float("-inf"))
    pr = torch.softmax(sc, dim=-1) * masks * scale
    o = (pr @ v).transpose(1, 2).reshape(b, s, H * d)
    h1 = x + F.linear(o, w["w_o"].T, w.get("b_o"))
    z = F.layer_norm(h1, (h,), w["n2_g"], w["n2_b"], eps=sh.norm_eps)
    u = F.gelu(F.linear(z, w["w_1"].T, w.get("b_1")))
    return h1 + F.linear(u, w["w_2"].T, w.get("b_2"))


def test_dropout_matches_torch_with_the_same_masks():
    """The layer with attention dropout equals the PyTorch composition fed the
    oracle's masks as data (forward and autograd gradients), which pins the
    hand-derived dropout backward; two sequences get different masks."""
    sh = _shape(s=24, h=16, H=4, Hkv=2, d=4, f=32).replace(dropout_p=0.25, seed=99)
    w = _weights(sh)
    x, dy = _inputs(sh, batch=2)
    out = orc.layer(x, w, orc.spec_of(sh), dy=dy)
    thr = orc.dropout_threshold(sh.dropout_p)
    masks = torch.tensor(np.stack([
        np.stack([orc.dropout_keep(np.arange(24), 24, hq, bi, sh.seed, thr)
                  for hq in range(sh.n_heads)]) for bi in range(2)]).astype(np.float64))
    assert 0 < float(masks.mean()) < 1 and not torch.equal(masks[0], masks[1])
    tw = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    tx = torch.tensor(x, requires_grad=True)
    ty = _torch_attention_layer_with_masks(tx, tw, sh, masks, 256.0 / (256 - thr))
    assert _rel(out["y"], ty.detach().numpy()) < 1e-12
    (ty * torch.tensor(dy)).sum().backward()
    assert _rel(out["dx"], tx.grad.numpy()) < 1e-10
    for name, g in out["grads"].items():
        assert _rel(g, tw[name].grad.numpy()) < 1e-10, name
    nodrop = orc.layer(x, w, orc.spec_of(sh.replace(dropout_p=0.0)))
    assert _rel(out["y"], nodrop["y"]) > 1e-3
