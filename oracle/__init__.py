"""CPU oracle for the FlashNorm norm-then-project path (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the
package entry file and the ``cpu_baseline`` leg of the benchmark may import
this package.  The GPU library never calls it, and it shares no code with the
GPU library: both sides only read the seeded inputs of ``synth``.

What it computes is the *textbook* RMSNorm followed by a bias-free linear
layer, with the gain still separate and the division done before the matmul
(the unfolded, undeferred form).  FlashNorm is an exact rewrite of exactly
that computation (FlashNorm: Fast Normalization for Transformers, Abstract,
points (i) and (ii)), so the definition itself is the oracle.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, hand-derived golden cases in ``tests/golden/``,
library routines on special cases and brute force on tiny inputs.  No
function is left unpinned.
"""

from .reference import (  # noqa: F401
    deferred_on_folded,
    deferred_fp8_act,
    deferred_on_quantized,
    dequantize_fp8,
    e4m3_code,
    e4m3_value,
    fold_weights,
    glu_deferred_on_folded,
    glu_deferred_fp8_act,
    glu_deferred_on_quantized,
    glu_fp8_act,
    fold_layernorm,
    head_rmsnorm,
    layernorm,
    layernorm_deferred_on_folded,
    latent_dropped_on_folded,
    layernorm_linear,
    linear_latent_norm,
    linear_qknorm,
    linear_qknorm_rope,
    norm_glu_ffn,
    norm_linear,
    norm_linear_fp8_act,
    qknorm_dropped_on_folded,
    quantize_fp8_per_channel,
    rms,
    rmsnorm,
    rope,
    rope_angles,
    round_to_bf16,
    round_to_e4m3,
    round_to_f32,
    silu,
)
from .compare import row_metrics, check_close  # noqa: F401
