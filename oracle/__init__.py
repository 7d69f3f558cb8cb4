"""CPU oracle for the MoE-layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers, tables or constant generators) and
imports nothing from the product package.

Source of truth, cited below as [MCore-MoE]: the web page "Scalable Training of
Mixture-of-Experts Models with Megatron Core" (paperlayer.ai summary of arXiv
2603.07685v2).  The relevant passages are in its section 2 ("Megatron-Core MoE
Architecture": the Route, Dispatch, Expert Computation and Combine bullets) and
section 5 ("Reduced-Precision Training in FP8/FP4 for MoE": the Selective
precision and Platform-specific recipes bullets).  The FP8 codec follows the
OCP 8-bit Floating Point specification (E4M3 "FN" encoding), cited as [OCP-FP8].

Numerics: floating-point math is float64 unless a step fixes the precision
(the router keys are fp32 per [MCore-MoE] section 5, Selective precision, and
the FP8 quantizer's scale arithmetic is fp32).
"""

from .moe_oracle import *  # noqa: F401,F403
from . import fp8  # noqa: F401
