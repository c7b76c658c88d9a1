"""CPU oracle of the DeepSeekMoE layer forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy (fp64) implementation of what the
layer computes, written from the DeepSeek-V3 pages:

* "DeepSeek_V3_Report: Annotation", section "DeepSeekMoE with
  Auxiliary-Loss-Free Load Balancing", eq. (12)-(16); sections "Node-Limited
  Routing" and "No Token-Dropping"; section "Fine-Grained Quantization",
  "Increasing Accumulation Precision", "Mantissa over Exponents" and "Online
  Quantization" of the FP8 framework; the SwiGLU paragraph.
* "DeepSeek V3 / V4 Infra" (blog digest), section on V3 FP8 (1x128 activation
  tiles, 128x128 weight blocks, promotion every 128 elements), the 6hd
  FLOP count per token-expert pair, and the V4 post-training FP4 (MXFP4)
  expert weights (``mxfp4.py``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library never calls it, links
it or shares code with it; the two meet only through the seeded inputs of
``moe_inputs``.

Parity pins: every function here is pinned by a CPU test in
``tests/test_oracle_*.py`` against something other than itself (brute force,
closed forms, invariants, or a library routine). The absolute output values of
the full layer have no worked example on the pages: beyond those pins they
are "parity unpinned".
"""
from .accumulation import keep_bits, limited_precision_gemm  # noqa: F401
from .backward import (  # noqa: F401
    ffn_backward, ffn_backward_fp8, gate_backward, layer_backward, requant_cols_pow2, round_bf16,
)
from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode  # noqa: F401
from .mxfp4 import (  # noqa: F401
    e2m1_decode, e2m1_encode, quantize_mxfp4, dequantize_mxfp4, pack_e2m1, unpack_e2m1, mxfp4_to_e4m3_blocks,
)
from .moe import (  # noqa: F401
    affinity, balance_stats, route, permute, swiglu_ffn, quantize_tiles, quantize_blocks,
    dequantize_tiles, dequantize_blocks, ffn_fp8, ffn_quantised_acts, ffn_mxfp4, combine, bias_update,
    expert_ffn, layer_forward,
)
