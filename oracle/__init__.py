"""CPU oracle for the MoE expert-MLP path.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition of what the GPU path computes, evaluated in float64 with numpy.
Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``mixture_experts_expert_top_amd``) never does and shares no code with it.

Sources (cited by page title and section):
  * "Efficient MoE Training for Biological Foundation Models" (NVIDIA
    Developer Blog, mirrored) -- Challenge 1 (per-expert loop, split_sizes,
    GroupedLinear gate_up of width 2*intermediate), Challenge 2 (MXFP8: one
    scale per 32 consecutive values), Challenge 3 (GroupedLinear ->
    ScaledSwiGLU -> GroupedLinear, the routing probabilities act as scales).
  * "How MoE Architecture Cuts Costs and Boosts Efficiency: Efficient
    Training of Biological Foundation Models" -- section "Why Biology Is
    Especially Well-Suited for MoE" (top-K router over per-expert scores)
    and "Engineering Challenges of Efficient Training" (load balance).
  * the hgpu.org abstract of an MXFP4 MoE training recipe on Hopper (FP8
    GEMMs, MXFP4 activations and payloads, FP4 row blocks converted to
    column blocks with new scales).

Every function is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_mx_pins.py``, ``tests/test_oracle_mx_layer_pins.py``,
``tests/test_oracle_router_pins.py``, ``tests/test_oracle_mx4_pins.py`` and
``tests/test_oracle_mx4_layer_pins.py`` (brute force, closed forms, library
routines, finite differences, exhaustive codec sweeps, independent
formulations of the MXFP8 and MXFP4-activation layers).
See each module header for what is and is not pinned.
"""

from . import moe_mx, moe_ref, mx4_ref, mx_ref  # noqa: F401
