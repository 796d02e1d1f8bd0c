"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package holds no step of the sparse-attention method itself: it only draws
random tensors, rounds them to the storage formats the method reads (bf16, OCP fp8
e4m3 with a per-token scale, OCP MXFP4 rows) and prepares positions (rotary embedding of the
attention inputs for the small multi-head workload, which happens before the
attention layer sees its inputs).
"""
from .inputs import *  # noqa: F401,F403
