"""CPU oracle for the AWQ W4A16 hot path -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The library under
``weight_only_int4_stats_amd`` never imports it, and this package imports
nothing from there: the two share no code.

The oracle is a plain, slow, step-by-step NumPy implementation of what the
method computes, written from these pages (cited by title and section):

* "AWQ Math" (aicassindra.com transformer-math series) -- the formulas;
* "AWQ > Benefits and Practical Considerations" and "AWQ > Limitations"
  (mbrenndoerfer.com) -- storage format and the inference-time dequantization;
* "AWQ vs. GPTQ: Understanding Weight Quantization Principles" -- process order.

Floating point runs in float64 except where a step is defined in float32 or
float16 (the quantizer's scale and codes, the candidate scales); those steps use
NumPy float32/float16 element operations, which are IEEE-754 correctly rounded
(NumPy never contracts a*b+c into an FMA).  Every function cites its passage.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
except the value of the chosen exponent on realistic random layers (no page
prints a search result) -- that is "parity unpinned" beyond the brute-force,
special-case and monotonicity pins listed in that test module.
"""
from .awq import (  # noqa: F401
    GROUP, NBITS, QMAX,
    act_mean_abs, act_fixed_point_sums,
    candidate_scales,
    fp16_round_up, scale_columns, unscale_activation,
    code_max, group_quant_params, quantize_codes, dequantize,
    quantize_layer, pack_codes, unpack_codes,
    search_losses, search_losses_operand_model, choose_candidate, search_scales,
    w4a16_matmul, w4a16_matmul_rows,
    round_bf16, round_storage, fold_scales,
    salient_channels,
    symmetric_rtn,
)
