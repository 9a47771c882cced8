"""DeepSeekMoE layer forward on MI355X (gfx950): Python binding of the HIP
library libmoe_mi355x.so, whose C ABI is include/moe.h."""
from ._binding import (  # noqa: F401
    LIB_PATH, MOE_ACT_QUANT_E4M3_1X128, MOE_ACT_QUANT_NONE, MOE_BF16, MOE_ERR_HIP, MOE_ERR_INVALID_ARG,
    MOE_ERR_OOM, MOE_ERR_UNSUPPORTED, MOE_F32, MOE_FP8_E4M3, MOE_OK, MOE_PATH_AUTO, MOE_PATH_GROUPED, MOE_PATH_STREAM, MoEError, MoELayer, MoeParams,
    MoeWeightGrads, MoeWeights, bias_update, create_cfg, declared_functions, load_library, load_stats, make_params,
    quantize_e4m3_1x128, status_string,
)
