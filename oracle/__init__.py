"""fp64 CPU oracle for the q4 MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package.  It shares no code with the HIP
path (``bit_routed_expert_tf_amd``) and never imports it; the only module both
sides use is ``synth`` (seeded input draws and byte layout).

Parity status of each function is listed in ``oracle/ref.py``.
"""
from .ref import *  # noqa: F401,F403
