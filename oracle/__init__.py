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
force over the e4m3 values and closed forms (tests/test_oracle_quantize.py).  No function here is
"parity unpinned".
"""
from . import formats, quantize, reference  # noqa: F401
from .reference import (  # noqa: F401
    A_BF16, A_MXFP8, W_INT3, W_INT4, W_MXFP4, W_UINT3, W_UINT4,
    dequant_activations, dequant_weights, gemm, gemm_exact, moe_counts, moe_gemm,
    moe_offsets, moe_sorted_pairs, normwise_error, qg_gemm, round_bf16,
)
