"""CPU oracle for the FP8 decode-step hot path (test infrastructure only).

This package is the plain, slow, obviously-correct reference that the HIP
kernels are checked against.  It is NOT part of the product path: only the
tests, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library or its
Python binding, and neither imports the other.

Everything is NumPy in float64 (exact for every dequantised FP8 operand),
except where the method fixes a narrower precision (the fp32 scale division of
block-scaled quantisation and the fp32 rounding of the SwiGLU output before it
is re-quantised).

Sources, by page title:
  * "How We Made Our Text-to-Speech API Free: The Inference Engineering Behind
    S2.1 Pro" (and its Chinese original) -- sections "FP8 Quantization
    Strategy", "Kernel Benchmark Results", "Why cuBLAS Wasn't Enough",
    "What's Open Source".
  * "Fish Speech KV Cache 推理优化记录" (Fish Speech KV-cache optimisation
    notes) -- section 4 (the bottleneck), section 5 (keep capacity, read the
    active prefix), section 7 (tests).
  * The OCP 8-bit floating point specification and the OCP Microscaling (MX)
    specification, which the first page names for its e4m3 / UE8M0 formats.

Parity status of each function is stated in its module header.
"""

from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_encode,
    e4m3_decode,
    quant_block_fp32,
    quant_act_1x128,
    quant_weight_128x128,
    quant_mx_1x32,
    dequant_block_fp32,
    dequant_mx_1x32,
)
from .mlp import linear_dequant, swiglu, swiglu_mlp  # noqa: F401
from .attention import gqa_decode_attention, kv_len_schedule, mx_kv_store  # noqa: F401
from .dual_ar import (  # noqa: F401
    RMS_EPS,
    round_bf16,
    rmsnorm,
    fp8_linear,
    dequant_weight,
    attention_block,
    mlp_block,
    decoder_layer,
    embed_sum,
    greedy_code,
    dual_ar_step,
)
