"""CPU oracle for the quantized GEMM -- TEST INFRASTRUCTURE, not part of the product.

A plain, slow, obviously correct reference written from the Humming pages (the
vLLM/Ant Group announcement and the AIREITER benchmark write-up) and the OCP
format specifications.  It shares no code with the HIP library and imports
nothing from it.  Only ``tests/``, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import it; the library never does.

Pins (tests marked ``not gpu``) tie every function to something other than
itself: torch's e4m3 / e8m0 / bf16 decoders, the OCP e2m1 value set, the
e0m7 = INT8-without--128 identity, numpy's bit unpacking, exact rational brute
force, integer GEMM special cases and closed forms; the MXFP8 quantizer and the
MoE output stage are pinned by hand-worked cases, exact round trips, brute
force over the e4m3 values and closed forms (tests/test_oracle_quantize.py).
The 1-, 2- and 8-bit integer, e0m and e4m3 weight formats, the W8A8 block
scales and the per-token FP8 activations are pinned by integer GEMMs on the
raw codes, torch's e4m3 values, exact rational sums and closed forms
(tests/test_oracle_gemm.py); the FP8 quantizer by hand-worked cases, exact
round trips and torch's fp32 division and e4m3 cast.  No function here is
"parity unpinned".
"""
from . import formats, quantize, reference  # noqa: F401
from .reference import (  # noqa: F401
    A_BF16, A_FP8_BLOCK, A_FP8_TOKEN, A_MXFP4, A_MXFP8, FP8_BLOCK, W_E0M3, W_E0M7, W_FP8, W_INT1, W_INT2,
    W_INT3, W_INT4, W_INT8, W_MXFP4, W_UINT1, W_UINT2, W_UINT3, W_UINT4, W_UINT8,
    dequant_activations, dequant_weights, dequant_weights_fp8_block, gemm, gemm_exact, moe_counts,
    moe_gemm, moe_offsets, moe_sorted_pairs, normwise_error, qg_gemm, round_bf16,
)
