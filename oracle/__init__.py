"""Plain fp64 CPU oracle of the GPTQ per-layer quantization solver.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test-suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or constants); the only
thing both sides consume is the seeded synthetic input generator, which holds
none of the method's arithmetic.

Every function is written from the pages' description of the method (cited in
each docstring by page title and section), in float64, as slow and obvious
code.  Pins that tie it to something other than itself live in
``tests/test_oracle_pins.py``.
"""
from .gptq_oracle import (  # noqa: F401
    NotPositiveDefinite,
    NonFinite,
    InvalidArgument,
    hessian,
    act_order_permutation,
    damp_hessian,
    inverse_hessian_upper,
    quant_params,
    quantize_column,
    tie_margin,
    sweep,
    static_group_params,
    gptq_quantize,
    pack,
    unpack,
    pack_permuted,
    dequant_matmul,
    round_to_dtype,
    quantize_block_chain,
    dequantize,
    layer_loss,
    words_per_row,
)
