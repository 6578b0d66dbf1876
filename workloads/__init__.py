"""Seeded synthetic inputs for the routed-MoE-over-slot-cache path.

This package is shared by the CPU oracle (``oracle/``), the tests, ``bench.py``
and the HIP path's Python driver.  It draws random numbers and lays them out;
it holds none of the method's arithmetic (no routing, dedup, LRU, align,
format decode or expert MLP).
"""
from .synth import *  # noqa: F401,F403
