"""Plain fp64 CPU oracle for the InfLLM-V2 sparse-attention forward path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product library.
"""
from .infv2_oracle import *  # noqa: F401,F403
