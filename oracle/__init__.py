"""CPU oracle of the MoE layer hot path (plain numpy, fp64).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py are the only callers.  It shares no code with
the HIP library or its binding and imports nothing from them; the only
module both sides use is ``workloads`` (seeded input data, no arithmetic
of the layer).

Every function is pinned by a CPU test in tests/test_oracle_*.py against a
closed form, an invariant, a brute-force or a finite-difference check; none
is "parity unpinned".
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (assign, bf16_bits, bf16_rne, capacity, combine,
                         combine_bwd, expert_ffn_bwd, expert_ffn_fwd,
                         fp32_rne, gelu_tanh, gelu_tanh_grad, layer_bwd,
                         layer_fwd, permute, route, route_bwd, router_dz,
                         router_logits, rounder, softmax, to_f64,
                         topk_select, unpermute_bwd)
