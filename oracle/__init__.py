"""fp64 CPU oracle of the Flux MMDiT block forward and the rectified-flow objective.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library shares no code with
it and never calls it: there is no CPU fallback anywhere in the product path.

Every function is the plain definition written out in numpy float64 (a matmul,
an exp, an erf are library primitives), following the Flux pages:
  * "Flux architecture deep dive" -- Flow matching framework, Model
    components (MMDiT layer, Flux single block, Output processing),
    Mathematical formulation (Flow matching objective, 3D RoPE mathematics),
    Implementation details (Adaptive layer normalization, Attention).
  * "Flux model API reference" -- FluxConfig key parameters, AdaLN, RMSNorm,
    EmbedND, apply_flow_matching_noise, compute_flow_matching_loss.
  * "FP8 training for Flux models" -- Configuration (E4M3, delayed scaling),
    in fp8_oracle; the "mxfp8" recipe (block-scaled E4M3 in the OCP MX
    format) in mx_oracle.
  * the backward pass of the blocks under the rectified-flow loss (the chain
    rule of the forward definitions, written out by hand) in backward_oracle.
Where the pages leave a step open the oracle takes one stated reading; the
readings are listed in the design notes and repeated next to the code.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (closed forms, invariants, page-printed constants and
a pure-Python brute force on tiny inputs); the backward by central finite
differences of the forward in tests/test_backward_oracle_pins.py.
"""
from .flux_oracle import *  # noqa: F401,F403
from . import fp8_oracle  # noqa: F401
from . import mx_oracle  # noqa: F401
from . import backward_oracle  # noqa: F401
