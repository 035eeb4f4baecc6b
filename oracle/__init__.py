"""CPU oracle of the routed 4-bit MoE FFN layer under an expert budget.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke entry
point and the benchmark's CPU-baseline leg may import, call or execute anything
in this package.  The HIP library never routes through it and shares no code,
table or constant with it.

The oracle is the plain definition of what the layer computes: the paging,
budget and wave machinery of the library only move bytes, so the oracle keeps
every expert "resident" and has no notion of slots (a predictor or cache may
reorder work but never change what is computed: ro99/strata README, list of
enforced rules).  Floating point is fp64 except where a float decides an
integer: the router logits that select experts are formed in fp32 in one fixed
summation order, the same order the GPU kernel uses, so that both sides take
the top-k decision on identical values.

Parity status of each function (what pins it, see tests/test_oracle_pins.py):
  dequant_int4_g64      pinned (hand-packed blocks, closed form)
  dequant_mxfp4_g32     pinned (E2M1 bit definition, E8M0 exponent field)
  router_logits_fp32    pinned (fp64 bound, exact small-integer case, hand-derived
                        rounding cases for the per-lane and butterfly order)
  select_topk           pinned (brute force sorted() on tiny inputs)
  routing_weights       pinned (closed forms: k=2 softmax is a logistic, ties 1/k)
  permute               pinned (brute force, permutation invariants)
  expert_ffn            pinned (one-hot input picks weight columns; SwiGLU closed form)
  moe_forward           pinned (isolation per expert, identical experts, relabelling)
  ResidencyModel        pinned (OrderedDict LRU simulator, hand-worked traces)
"""
from .moe import (dequant_int4_g64, dequant_mxfp4_g32, dequant_qmat, expert_ffn, moe_forward,
                  permute, router_logits_fp32, routing_weights, select_topk)
from .residency import ResidencyModel

__all__ = [
    "dequant_int4_g64", "dequant_mxfp4_g32", "dequant_qmat", "expert_ffn", "moe_forward", "permute",
    "router_logits_fp32", "routing_weights", "select_topk", "ResidencyModel",
]
