"""Seeded synthetic inputs for the MoE-layer hot path.

This package only draws random numbers and lays bytes out; it holds none of
the layer's arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP path
(``bit_routed_expert_tf_amd``) consume what it produces.
"""
from .gen import *  # noqa: F401,F403
