"""One-shot GPTQ quantization of linear layers on AMD Instinct MI355X (gfx950).

The computation lives in libgptq.so (hand-written HIP kernels behind a
C ABI, declared in include/gptq.h); this package is its Python binding.
"""
from ._lib import (  # noqa: F401
    GptqError,
    bits_for_levels,
    gptaq_quantize_linear,
    gptq_asym_target,
    gptq_dequant_gemm,
    gptq_dequant_gemv,
    gptq_hessian_accumulate,
    gptq_hessian_accumulate_noalloc,
    gptq_hessian_pair_accumulate,
    gptq_lora_quantize_linear,
    gptq_lora_refine,
    gptq_lowrank_basis,
    gptq_lowrank_compensation,
    gptq_lowrank_hessian,
    gptq_pack,
    gptq_prepare_hinv,
    gptq_quantize_layer,
    gptq_quantize_linear,
    gptq_refine_codes,
    load,
    packed_words,
)
