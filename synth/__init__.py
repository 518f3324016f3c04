"""Seeded synthetic inputs for the DFlash 2 draft -> select -> verify cycle.

This module serves both the CPU oracle and the HIP library (tests, smoke and
bench feed the same arrays to each).  It holds none of the method's
arithmetic: it only draws random numbers, rounds them to the storage type and
shapes planted-token structure.  See ``synth.inputs`` for the recipe.
"""

from .inputs import CONFIGS, make, make_conv, make_lattice, bf16_bits, bf16_value  # noqa: F401
