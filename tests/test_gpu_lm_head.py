"""GPU parity of the blockwise LM head with cross-entropy (through the C ABI)
against the float64 oracle (oracle/lm_head_oracle.py).

* Reduced shapes in fp32 and bf16: three row chunks (the last ragged), some
  ignored rows; loss, dz and dW per tensor and per row / 32 x 32 tile.
* Peaked logits (W_head scaled 16x): the row log-sum-exp is dominated by a few
  columns far from the block maxima of the others.
* dW accumulation across calls; bitwise reproducibility.
* The fused forward + backward call: bit for bit the two calls' results
  (with and without the saved state, dz or dW alone, accumulating), guard
  regions around its outputs and workspace.
* The benchmarked shape (131072 rows, hidden 2048, vocabulary 50304): loss at
  sampled rows, and the backward from a cotangent on those rows only (dz must
  be exactly zero elsewhere; dW is the sum over the sampled rows).

Bars: fp32 max relative L2 1e-5; bf16 relative L2 1e-2 per tensor; local
(row / tile) errors within 5x, as in the layer's parity tests.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from harness import TOL, local_max, over_bar, rel_l2, to_host64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(t):
    if t.dtype == "bf16":
        return torch.from_numpy(t.storage.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(t.storage).cuda()


class LmInputs:
    def __init__(self, sh, w_scale=1.0, dloss_rows=None):
        self.sh = sh
        self.z = wl.make_z(sh)
        self.w = wl.make_w_head(sh)
        if w_scale != 1.0:
            self.w = wl.scaled(self.w, w_scale)
        self.t = wl.make_targets(sh)
        self.g = wl.make_dloss(sh, dloss_rows)


def _run_gpu(inp, accumulate_into=None):
    import memory_efficient_long_amd as bpt
    sh = inp.sh
    cfg = bpt.LmHeadConfig(sh.rows, sh.hidden, sh.vocab, sh.chunk_rows, sh.dtype)
    z, w = _dev(inp.z), _dev(inp.w)
    t = torch.from_numpy(inp.t).cuda()
    g = torch.from_numpy(inp.g).cuda()
    loss, saved = bpt.lm_head_forward(cfg, z, w, t)
    dz, dw = bpt.lm_head_backward(cfg, z, w, t, saved, g)
    torch.cuda.synchronize()
    return {"loss": loss, "saved": saved, "dz": dz, "dw": dw}


def _run_fused(inp, saved=True, dz=True, dw=True, dw_init=None):
    import memory_efficient_long_amd as bpt
    sh = inp.sh
    cfg = bpt.LmHeadConfig(sh.rows, sh.hidden, sh.vocab, sh.chunk_rows, sh.dtype)
    d = cfg.desc()
    z, w = _dev(inp.z), _dev(inp.w)
    t = torch.from_numpy(inp.t).cuda()
    g = torch.from_numpy(inp.g).cuda()
    loss = torch.empty(sh.rows, dtype=torch.float32, device="cuda")
    sv = torch.empty(bpt.bpt_lm_head_saved_size(d), dtype=torch.uint8, device="cuda") if saved else None
    dzt = torch.empty_like(z) if dz else None
    dwt = None
    if dw:
        dwt = (dw_init.clone() if dw_init is not None
               else torch.empty(sh.hidden, sh.vocab, dtype=torch.float32, device="cuda"))
    ws = torch.empty(bpt.bpt_lm_head_workspace_size(d, 2), dtype=torch.uint8, device="cuda")
    st = bpt.bpt_lm_head_forward_backward(d, z, w, t, g, loss, sv, dzt, dwt, ws,
                                          accumulate=dw_init is not None)
    assert st == 0, bpt.bpt_last_error()
    torch.cuda.synchronize()
    return {"loss": loss, "saved": sv, "dz": dzt, "dw": dwt}


def _errs(gpu, ref, rows=None):
    loss = to_host64(gpu["loss"])
    if rows is not None:
        loss = loss[rows]
    e = {"loss": rel_l2(loss, ref["loss"]), "loss@row": local_max(loss[:, None],
                                                                  ref["loss"][:, None], True)}
    for k in ("dz", "dw"):
        got = to_host64(gpu[k]).reshape(ref[k].shape)
        e[k] = rel_l2(got, ref[k])
        e[k + ("@row" if k == "dz" else "@tile")] = local_max(got, ref[k], k == "dz")
    return e


@pytest.mark.parametrize("name", ["lmhead-small-f32", "lmhead-small-bf16"])
@pytest.mark.parametrize("w_scale", [1.0, 16.0])
def test_lm_head_matches_oracle(name, w_scale):
    from oracle import lm_head_oracle as lmo
    sh = wl.LM_HEADS[name]
    _say(f"[lm-head] {name} rows={sh.rows} h={sh.hidden} V={sh.vocab} chunk={sh.chunk_rows} "
         f"W x{w_scale}")
    inp = LmInputs(sh, w_scale)
    gpu = _run_gpu(inp)
    ref = lmo.lm_head_ce(inp.z.f64(), inp.w.f64(), inp.t, inp.g.astype(np.float64))
    errs = _errs(gpu, ref)
    _say(f"  errs {errs}")
    bad = over_bar(errs, sh.dtype)
    assert not bad, bad
    # ignored rows: exactly zero loss and zero dz
    ign = inp.t < 0
    assert np.all(to_host64(gpu["loss"])[ign] == 0.0)
    assert np.all(to_host64(gpu["dz"])[ign] == 0.0)


@pytest.mark.parametrize("case", ["one-tile", "all-ignored"])
def test_lm_head_degenerate(case):
    """Fewer rows than one tile with the smallest vocabulary (one column
    tile), and a chunk whose every target is ignored (zero loss and dz)."""
    from oracle import lm_head_oracle as lmo
    base = wl.LM_HEADS["lmhead-small-bf16"]
    if case == "one-tile":
        sh = base.replace(name="lmhead-one-tile", rows=37, hidden=64, vocab=64, chunk_rows=64,
                          ignore_every=0)
    else:
        sh = base.replace(name="lmhead-all-ignored", rows=200, chunk_rows=64, ignore_every=1)
    _say(f"[lm-head] {sh.name} rows={sh.rows} h={sh.hidden} V={sh.vocab}")
    inp = LmInputs(sh)
    gpu = _run_gpu(inp)
    ref = lmo.lm_head_ce(inp.z.f64(), inp.w.f64(), inp.t, inp.g.astype(np.float64))
    if case == "all-ignored":
        assert np.all(to_host64(gpu["loss"]) == 0.0) and np.all(to_host64(gpu["dz"]) == 0.0)
        assert np.all(to_host64(gpu["dw"]) == 0.0)
        return
    errs = _errs(gpu, ref)
    _say(f"  errs {errs}")
    bad = over_bar(errs, sh.dtype)
    assert not bad, bad


def test_lm_head_accumulate_and_reproducible():
    import memory_efficient_long_amd as bpt
    sh = wl.LM_HEADS["lmhead-small-bf16"]
    inp = LmInputs(sh)
    a = _run_gpu(inp)
    b = _run_gpu(inp)
    for k in ("loss", "saved", "dz", "dw"):
        assert torch.equal(a[k], b[k]), k
    cfg = bpt.LmHeadConfig(sh.rows, sh.hidden, sh.vocab, sh.chunk_rows, sh.dtype)
    z, w = _dev(inp.z), _dev(inp.w)
    t = torch.from_numpy(inp.t).cuda()
    g = torch.from_numpy(inp.g).cuda()
    dw = a["dw"].clone()
    dz2, dw2 = bpt.lm_head_backward(cfg, z, w, t, a["saved"], g, dw_head=dw, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dz2, a["dz"])
    err = (dw2.double() - 2 * a["dw"].double()).norm() / (2 * a["dw"].double()).norm()
    assert err < 1e-6


@pytest.mark.parametrize("name", ["lmhead-small-f32", "lmhead-small-bf16"])
@pytest.mark.parametrize("w_scale", [1.0, 16.0])
def test_lm_head_fused_equals_two_calls(name, w_scale):
    """The fused call forms each chunk's dlogits from the stored fp32 logits
    with the backward epilogue's arithmetic: its loss, saved state, dz and dW
    equal the forward + backward calls' bit for bit (and so meet the oracle
    bars those calls are held to, checked here again)."""
    from oracle import lm_head_oracle as lmo
    sh = wl.LM_HEADS[name]
    _say(f"[lm-head fused] {name} W x{w_scale}")
    inp = LmInputs(sh, w_scale)
    two = _run_gpu(inp)
    fused = _run_fused(inp)
    for k in ("loss", "saved", "dz", "dw"):
        assert torch.equal(two[k], fused[k]), k
    ref = lmo.lm_head_ce(inp.z.f64(), inp.w.f64(), inp.t, inp.g.astype(np.float64))
    errs = _errs(fused, ref)
    _say(f"  errs {errs}")
    bad = over_bar(errs, sh.dtype)
    assert not bad, bad


def test_lm_head_fused_options():
    """Without the saved state, with dz or dW alone, and accumulating into dW:
    the same bits as the full fused call (twice dW when accumulating onto it)."""
    sh = wl.LM_HEADS["lmhead-small-bf16"]
    _say(f"[lm-head fused options] {sh.name}")
    inp = LmInputs(sh)
    full = _run_fused(inp)
    a = _run_fused(inp, saved=False)
    assert torch.equal(a["loss"], full["loss"]) and torch.equal(a["dz"], full["dz"])
    assert torch.equal(a["dw"], full["dw"])
    b = _run_fused(inp, dw=False)
    assert torch.equal(b["dz"], full["dz"]) and torch.equal(b["saved"], full["saved"])
    c = _run_fused(inp, dz=False)
    assert torch.equal(c["dw"], full["dw"])
    e = _run_fused(inp, dw_init=full["dw"])
    assert torch.equal(e["dz"], full["dz"])
    err = (e["dw"].double() - 2 * full["dw"].double()).norm() / (2 * full["dw"].double()).norm()
    assert err < 1e-6


def test_lm_head_no_writes_outside_outputs():
    """loss, saved, dz, dW and both workspaces, each sized exactly, between
    guard regions that must come back untouched."""
    import memory_efficient_long_amd as bpt
    sh = wl.LM_HEADS["lmhead-small-bf16"]
    _say(f"[lm-head guards] {sh.name}")
    inp = LmInputs(sh)
    cfg = bpt.LmHeadConfig(sh.rows, sh.hidden, sh.vocab, sh.chunk_rows, sh.dtype)
    d = cfg.desc()
    z, w = _dev(inp.z), _dev(inp.w)
    t = torch.from_numpy(inp.t).cuda()
    g = torch.from_numpy(inp.g).cuda()
    guard = 4096
    bufs = []

    def guarded(numel, dtype, shape=None):
        buf = torch.full((numel + 2 * guard,), 7, dtype=dtype, device="cuda")
        bufs.append(buf)
        v = buf[guard:guard + numel]
        return v.view(shape) if shape is not None else v

    loss = guarded(sh.rows, torch.float32)
    saved = guarded(bpt.bpt_lm_head_saved_size(d), torch.uint8)
    ws_f = guarded(bpt.bpt_lm_head_workspace_size(d, False), torch.uint8)
    ws_b = guarded(bpt.bpt_lm_head_workspace_size(d, True), torch.uint8)
    dz = guarded(z.numel(), z.dtype, z.shape)
    dw = guarded(sh.hidden * sh.vocab, torch.float32, (sh.hidden, sh.vocab))
    assert bpt.bpt_lm_head_forward(d, z, w, t, loss, saved, ws_f) == 0
    assert bpt.bpt_lm_head_backward(d, z, w, t, saved, g, dz, dw, ws_b, False) == 0
    torch.cuda.synchronize()
    for buf in bufs:
        assert torch.all(buf[:guard] == 7) and torch.all(buf[-guard:] == 7)
    ref = _run_gpu(inp)
    assert torch.equal(loss, ref["loss"]) and torch.equal(dz, ref["dz"])
    assert torch.equal(dw, ref["dw"])
    # the fused call: the same outputs and its own workspace, each guarded
    n0 = len(bufs)
    loss2 = guarded(sh.rows, torch.float32)
    saved2 = guarded(bpt.bpt_lm_head_saved_size(d), torch.uint8)
    ws_fb = guarded(bpt.bpt_lm_head_workspace_size(d, 2), torch.uint8)
    dz2 = guarded(z.numel(), z.dtype, z.shape)
    dw2 = guarded(sh.hidden * sh.vocab, torch.float32, (sh.hidden, sh.vocab))
    assert bpt.bpt_lm_head_forward_backward(d, z, w, t, g, loss2, saved2, dz2, dw2, ws_fb) == 0
    torch.cuda.synchronize()
    for buf in bufs[n0:]:
        assert torch.all(buf[:guard] == 7) and torch.all(buf[-guard:] == 7)
    assert torch.equal(loss2, ref["loss"]) and torch.equal(saved2, ref["saved"])
    assert torch.equal(dz2, ref["dz"]) and torch.equal(dw2, ref["dw"])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_lm_head_full_size_sampled_rows():
    from oracle import lm_head_oracle as lmo
    sh = wl.LM_HEADS["lmhead-gpt1b-s128k"]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(sh.rows, 16, replace=False),
                                     np.arange(sh.rows - 8, sh.rows)]))
    _say(f"[lm-head full] {sh.name}: rows {rows.tolist()}")
    inp = LmInputs(sh, dloss_rows=rows)
    gpu = _run_gpu(inp)
    z = inp.z.f64()
    ref = lmo.lm_head_ce(z[rows], inp.w.f64(), inp.t[rows], inp.g[rows].astype(np.float64))
    dz_full = np.zeros((sh.rows, sh.hidden))
    dz_full[rows] = ref["dz"]
    ref_full = {"loss": ref["loss"], "dz": dz_full, "dw": ref["dw"]}
    errs = _errs(gpu, ref_full, rows=rows)
    errs = {k: v for k, v in errs.items() if "@" not in k or k == "loss@row"}
    _say(f"  errs {errs}")
    bad = over_bar(errs, sh.dtype)
    assert not bad, bad
    other = np.ones(sh.rows, bool)
    other[rows] = False
    assert np.all(to_host64(gpu["dz"])[other] == 0.0)
    # the fused call at full size: the same bits as the two calls
    _say("  fused call at full size")
    fused = _run_fused(inp)
    for k in ("loss", "saved", "dz", "dw"):
        assert torch.equal(gpu[k], fused[k]), k
