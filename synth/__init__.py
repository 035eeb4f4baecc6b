"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark."""
from .workloads import (CONFIGS, CONFIG_ORDER, FORMAT_ORDER, INT4, INT4_G128, MXFP4, NVFP4, SIGMOID,
                        SOFTMAX, WIDE_ORDER, LayerConfig,
                        LayerWeights, QMat, bf16_bits_to_f32, f32_to_bf16_bits, make_layer,
                        make_tokens, quantize_int4, quantize_int4_g64, quantize_mxfp4_g32,
                        quantize_nvfp4_g16)

__all__ = [
    "CONFIGS", "CONFIG_ORDER", "FORMAT_ORDER", "INT4", "INT4_G128", "MXFP4", "NVFP4", "SIGMOID",
    "SOFTMAX", "WIDE_ORDER", "LayerConfig",
    "LayerWeights",
    "QMat", "bf16_bits_to_f32", "f32_to_bf16_bits", "make_layer", "make_tokens",
    "quantize_int4", "quantize_int4_g64", "quantize_mxfp4_g32", "quantize_nvfp4_g16",
]
