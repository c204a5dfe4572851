"""The memory-accounting helper against the values the pages print
("Training memory: model states, activations and checkpointing": §4 worked
example, §5 printed outputs of both code blocks, §3 checkpoint-every-k
example), stored with their citation in tests/golden/."""
import json
import os

import pytest

from memory_efficient_long_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "page3_printed_values.json")))


def test_worked_example_totals():
    we = GOLD["worked_example"]
    L, h, a, V, s, b = we["L"], we["h"], we["a"], we["V"], we["s"], we["b"]
    no_flash = acc.peak_bytes(L, h, a, V, s, b, flash=False)
    flash = acc.peak_bytes(L, h, a, V, s, b, flash=True)
    assert no_flash["psi"] == we["psi"]
    assert round(12 * L * h * h / no_flash["psi"], 3) == we["ratio_12Lh2_over_psi"]
    assert round(no_flash["states"] / acc.GB, 1) == we["states_GB"]
    assert round(no_flash["activations"] / acc.GB, 1) == we["act_GB_no_flash"]
    assert round(flash["activations"] / acc.GB, 1) == we["act_GB_flash"]
    assert round(no_flash["logits"] / acc.GB, 1) == we["logits_GB"]
    assert round(no_flash["total"] / acc.GB, 1) == we["total_GB_no_flash"]
    assert round(flash["total"] / acc.GB, 1) == we["total_GB_flash"]


def test_layer_parameter_counts():
    for h, n in GOLD["params_per_gpt_layer"].items():
        assert acc.params_gpt_layer(int(h)) == n


def test_saved_sbh_predictions():
    p = GOLD["saved_sbh_predictions"]
    h, a, s, b = p["h"], p["a"], p["s"], p["b"]
    assert acc.sbh_per_layer(h, a, s, "vanilla") == p["vanilla"]
    assert acc.sbh_per_layer(h, a, s, "flash") == p["flash"]
    assert acc.sbh_per_layer(h, a, s, "full_checkpoint") == p["full_checkpoint"]
    sbh = s * b * h
    assert acc.activation_bytes_per_layer(s, b, h, a) / sbh == p["vanilla"]
    assert acc.activation_bytes_per_layer(s, b, h, a, flash=True) / sbh == p["flash"]
    assert acc.full_checkpoint_bytes_per_layer(s, b, h) / sbh == p["full_checkpoint"]


def test_checkpoint_every_k_example():
    """L = 80 with c = 2 sbh and A = 34 sbh: M(1) = 194 sbh, M(2) = 148 sbh,
    and the best k is sqrt(L / 17) (§3, checkpoint every k layers)."""
    ck = GOLD["checkpoint_every_k"]
    L, c, A = ck["L"], ck["c_sbh"], ck["A_sbh"]
    assert acc.checkpoint_every_k(L, 1, c, A) == ck["M1_sbh"]
    assert acc.checkpoint_every_k(L, 2, c, A) == ck["M2_sbh"]
    assert acc.best_k(L, c, A) == pytest.approx((L / 17) ** 0.5)
    assert min(range(1, 9), key=lambda k: acc.checkpoint_every_k(L, k, c, A)) == 2
    # below L = 34 one layer per segment is best
    assert min(range(1, 9), key=lambda k: acc.checkpoint_every_k(33, k, c, A)) == 1
