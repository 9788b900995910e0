"""CPU oracle for the fused gate-up SwiGLU forward and backward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package. The product package
(``swiglu_activation_amd``) never imports it, and this package imports nothing
from the product: the two share no code. Inputs come from ``synth``.

Everything here is plain float64 numpy written from the definitions, with no
blocking, fusion or reformulation. See ``oracle.swiglu`` for the sources.
"""

from .swiglu import (  # noqa: F401
    G0,
    bf16_bits_to_f64,
    bf16_ordinal,
    bf16_ulp_distance,
    oracle_bwd,
    oracle_bwd_bias_scale,
    oracle_fc1,
    oracle_fc1_swiglu,
    oracle_fwd,
    oracle_fwd_bias_scale,
    round_f64_to_bf16_bits,
    sigmoid,
    silu,
    silu_grad,
    split_gate_up,
    widen,
)
