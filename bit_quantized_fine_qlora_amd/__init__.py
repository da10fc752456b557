"""MI355X-native QLoRA adapted-linear hot path (NF4 + double quantization + LoRA).

The compute lives in libqlora.so (hand-written HIP for gfx950, C ABI in
include/qlora.h); this package is a thin torch binding over it.
"""

from .api import (  # noqa: F401
    GroupedForward,
    QLORA_OP_BWD,
    QLORA_OP_BWD_DROPOUT,
    QLORA_OP_FWD,
    QTYPE_NF4,
    QTYPE_UNIFORM4,
    QTYPE_EDGE_MEAN4,
    QTYPE_INT4,
    QuantizedWeight,
    AdamStep,
    adam_step,
    alloc_quantized,
    dequant_dq,
    dequant_nf4_dq,
    linear_bwd,
    linear_check,
    linear_fwd,
    linear_fwd_static,
    linear_fwd_grouped,
    merge_adapter,
    level_table,
    nf4_table,
    profile_enable,
    profile_query,
    quantize_dq,
    quantize_dq_grouped,
    quantize_nf4_dq,
    workspace_bytes,
)
from ._lib import LIB_PATH, QloraError  # noqa: F401
