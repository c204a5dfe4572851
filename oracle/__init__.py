"""CPU oracle for the Blockwise Parallel Transformer layer (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the HIP library and its Python binding never do.
"""
from .bpt_oracle import Spec, spec_of, layer, norm_forward, norm_backward, rope_rotate, attention_probs  # noqa: F401
