"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and shapes them into the input formats the
decode path consumes (bf16 activations, fp32 master weights, fp32 router
logits).  It holds none of the method's arithmetic: no quantisation, no
dequantisation, no GEMV, no routing.  Both the CPU oracle and the HIP path
receive the same arrays from here and each side quantises the fp32 master
weights with its own code.

Every tensor is drawn from its own PCG64 stream keyed by
``SeedSequence(seed, spawn_key=(workload, tensor, expert))`` so that any single
expert of a 256-expert bank can be regenerated on its own, in any order.
"""
from .synth import *  # noqa: F401,F403
