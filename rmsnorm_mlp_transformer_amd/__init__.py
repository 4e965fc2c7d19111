"""MI355X-native (gfx950) fused LayerNorm/RMSNorm-MLP library.

The computation lives in libtemi355x.so (hand-written HIP kernels behind a C
ABI, declared in include/te_mi355x.h); this package is its Python binding.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (EXPORTED, LIB_PATH, Fp8Meta, QuantizerSet, TEError,  # noqa: F401
                       act_type_of, activation, activation_codes, dact_dbias, dact_dbias_quantize, dequantize,
                       is_gated, layernorm, layernorm_bwd, layernorm_dense, layernorm_mlp, layernorm_mlp_bwd,
                       make_saved,
                       noop_quantizer_set, quantize, te_last_error, te_timing_collect,
                       te_timing_enable, te_timing_reset, te_version)
