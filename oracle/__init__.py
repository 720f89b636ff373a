"""CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this package. The GPU library never imports, links or calls it,
and it imports nothing from the GPU library: the two share only the seeded
input generators in ``synth`` (which hold none of the layer's arithmetic).

Every function is plain numpy in float64, written for a reader to check by eye
against the pages it cites; see ``oracle.moe``.
"""
from .moe import *  # noqa: F401,F403
