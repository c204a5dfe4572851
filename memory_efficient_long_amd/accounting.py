"""Memory accounting of a transformer layer, as the pages state it.

Formulas of "Training memory: model states, activations and checkpointing":
§3 parameters (12h^2 + 13h per GPT layer; embedding Vh shared with the output
layer; final LayerNorm 2h), model states (16 bytes per parameter with
mixed-precision Adam), the activation theorem (sbh(34 + 5as/h) bytes per
pre-LN GPT layer with dropout; about 34sbh with FlashAttention; 2sbh with
full checkpointing), the logits (4sbV bytes, fp32), and checkpointing every k
layers (M(k) = (L/k) c + k A, best k = sqrt(L c / A)). "Blockwise Parallel
Transformer for Long Context Large Models", §3.4 memory analysis: a BPT layer
keeps about 2bsh (its output) for the backward.

Used by the benchmark to state the pages' predictions beside the library's
measured bytes per token; pinned by the worked example's printed values
(tests/test_accounting.py).
"""
from __future__ import annotations

import math

GB = 1e9   # the pages' unit: 1 GB = 10^9 bytes


def params_gpt_layer(h: int) -> int:
    """W_Q, W_K, W_V, W_O with biases (4h^2 + 4h), the 4h MLP with biases
    (8h^2 + 5h) and two LayerNorms with scale and shift (4h)."""
    return 12 * h * h + 13 * h


def params_gpt(L: int, h: int, V: int) -> int:
    """L layers, the token embedding shared with the output layer (Vh) and the
    final LayerNorm (2h)."""
    return L * params_gpt_layer(h) + V * h + 2 * h


def model_state_bytes(psi: int) -> int:
    """bf16 weights and gradients, fp32 master weights and both Adam moments."""
    return 16 * psi


def activation_bytes_per_layer(s: int, b: int, h: int, a: int, flash: bool = False) -> int:
    """34 sbh for everything linear in s, plus the 5 a s^2 b attention core
    (softmax output, dropout mask and output) unless a fused attention keeps
    no s x s matrix."""
    return 34 * s * b * h + (0 if flash else 5 * a * s * s * b)


def logits_bytes(s: int, b: int, V: int) -> int:
    return 4 * s * b * V


def full_checkpoint_bytes_per_layer(s: int, b: int, h: int) -> int:
    """Only the layer input, in 16 bits."""
    return 2 * s * b * h


def peak_bytes(L: int, h: int, a: int, V: int, s: int, b: int, flash: bool) -> dict:
    """Model states + L layers of activations + logits (no buffers)."""
    psi = params_gpt(L, h, V)
    out = {"psi": psi, "states": model_state_bytes(psi),
           "activations": L * activation_bytes_per_layer(s, b, h, a, flash),
           "logits": logits_bytes(s, b, V)}
    out["total"] = out["states"] + out["activations"] + out["logits"]
    return out


def sbh_per_layer(h: int, a: int, s: int, scheme: str) -> float:
    """Bytes per layer in units of sbh: 'vanilla' 34 + 5as/h, 'flash' 34,
    'full_checkpoint' 2, 'bpt' 2 (its output, the BPT memory analysis)."""
    return {"vanilla": 34 + 5 * a * s / h, "flash": 34.0, "full_checkpoint": 2.0,
            "bpt": 2.0}[scheme]


def checkpoint_every_k(L: int, k: int, c: float, A: float) -> float:
    """Peak of L/k stored segment inputs of size c plus one rebuilt segment of
    k layers of activations A."""
    return L / k * c + k * A


def best_k(L: int, c: float, A: float) -> float:
    return math.sqrt(L * c / A)
