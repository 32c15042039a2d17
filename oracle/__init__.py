"""FP64 CPU oracle for the block-scaled FP4 top-k MoE forward and the
group16 -> group32 FP4 requantisation.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
statement of what the HIP path computes.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``block_scaled_fp4_topk_amd``) never imports, calls or links
anything here, and this package never imports the product path: the two share
no code.  The only thing both sides consume is the seeded input generator in
``synth`` (which holds none of the method's arithmetic).

Sources (the pages):
  [P1] DeepGEMM commit log, branch ``cch/deepgemm-glm52-nvfp4-group16``
       (commits on ``requant_fp4_to_gran_k`` and the group16 capability gate).
  [P2] "GLM-5.2 NVFP4 group16 MegaMoE notes" (sections Context, Current patch
       scope, Remaining kernel work, Requantization path, Validation target).
  [P3] b12x ``moe/fused/w4a16/prepare.py`` ("Local NVFP4/BF16 weight
       preparation for the CuTeDSL W4A16 path"), cited by function name.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library decoders, invariants and brute force on tiny
inputs.  No function is "parity unpinned".
"""

from .formats import (  # noqa: F401
    E2M1_VALUES,
    e2m1_decode,
    e4m3_decode,
    ue8m0_decode,
    unpack_fp4,
    pack_fp4,
    rne_e2m1_magnitude,
    rne_e4m3,
    rne_bf16,
    dequant_fp4,
    bf16_bits_decode,
)
from .requant import requant_g16_to_g32, requant_block  # noqa: F401
from .moe import route, moe_forward, quantize_h_a8, quantize_a4, silu, h_decision_band, h_decision_margin, decision_radius  # noqa: F401
