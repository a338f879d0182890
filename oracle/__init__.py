"""CPU oracle for the GPTQ layer quantizer (test infrastructure only).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports or calls it.
"""
from .gptq_oracle import (  # noqa: F401
    NotPositiveDefinite,
    hessian,
    hessian_rows,
    act_order_perm,
    damp_and_permute,
    inverse_cholesky_upper,
    grid_params,
    quantize_values,
    gptq_quantize,
    rtn_quantize,
    unpermute_codes,
    group_index,
    dequantize,
    layer_loss,
    obs_loss,
    pack_codes,
    unpack_codes,
    packed_words_per_row,
    dequantize_packed,
    dequant_matmul,
    dequant_matmul_bound,
    asymmetric_target,
    asymmetric_target_from_hessians,
    gptaq_layer,
    lowrank_basis,
    lowrank_hessian,
    lowrank_compensation,
    gptq_lora_layer,
    refine_codes,
    lora_refine,
    gptq_layer,
)
from . import decoder_oracle  # noqa: F401,E402
