"""CPU oracle for the weight-only quantized linear layer (test infrastructure).

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product path (the HIP library and its Python
binding) never imports, links or runs anything from here.
"""

from .wq_oracle import (  # noqa: F401
    SUPPORTED_BITS,
    group_of_channel,
    act_order_perm,
    rtn_quantize,
    pack,
    unpack,
    dequant,
    dequant_fp64_path,
    awq_alpha_grid,
    awq_channel_scales,
    awq_fold_weight,
    awq_scale_act,
    awq_search,
    awq_clip_ratios,
    awq_clip_search,
    gptq_quantize,
    linear_ref,
    silu_mul_ref,
    quantize_linear_layer,
    f64_to_f16_nearest,
)
