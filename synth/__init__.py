"""Seeded synthetic inputs (shapes, value distributions, Zipf routing bias).

Feeds both the fp64 oracle and the HIP path; holds none of the method's
arithmetic.  See ``recipes`` for the workloads and ``philox`` for the
counter-based generator behind the expert weights.
"""
from .recipes import (WORKLOADS, TINY, DEC35, DEC80, BAT80, POOL80, DEC80I8, BAT80I8, Workload,  # noqa: F401
                      expert_raw, random_affine_bias, router_weights, router_bias, tokens,
                      zipf_bias, f32_to_bf16_bits, f32_to_f16_bits, GdnWorkload, GDN80, GDN_TINY,
                      gdn_inputs, gdn_state)
