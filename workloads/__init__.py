"""Seeded synthetic inputs for the speculative-decoding step.

This package only draws random inputs (contexts, logits, drafter outputs,
uniforms, tree weights).  It contains none of the step's arithmetic, so both
the CPU oracle and the HIP path can consume exactly the same arrays.
"""
from .synth import *  # noqa: F401,F403
