"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This package only *makes* input bytes (weights, hidden rows, planted edits, state
snapshots).  It holds none of the arithmetic of the speculative cycle: no logits,
no softmax, no acceptance rule, no sampling and no dequantisation used by either
side.  Both the oracle and the HIP path read the bytes it returns.
"""
from .inputs import *  # noqa: F401,F403
