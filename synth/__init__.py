"""Seeded synthetic workloads (shapes, weights, token and label ids).

Shared by the oracle and the GPU path; contains no scoring arithmetic.
"""
from .configs import (PAGE_TOKENS, PARITY_WORKLOADS, WORKLOADS, ModelShape, Request, TreeSpec, Workload,
                      workload)
from .gen import Branch, Instance, Weights, make_instance, make_weights
