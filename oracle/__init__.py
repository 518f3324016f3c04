"""CPU oracle for the DFlash 2 draft -> select -> verify hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``block_draft_select_amd``) and imports nothing from it.

Everything here is plain NumPy in float64 on inputs widened exactly from their
storage type (bf16 bit patterns or float32), with explicit per-stream loops, so
that a reader can check each step against the pages by eye:

* ``oracle.philox``  -- Philox4x32-10 counter-based generator and the uniform
  conversions the sampler contract uses.
* ``oracle.dflash``  -- top-K candidate extraction, the context gate, adjacent
  pair scores, the lattice trace, the rejection-sampling verify, and the
  decision margins the input guard uses.
* ``oracle.conv``    -- the two-tap dynamic depthwise convolution of the
  drafter's block representations.
* ``oracle.viterbi`` -- the global max-sum path through the candidate
  lattice (a variant of the greedy trace).

Pinned by ``tests/test_oracle_*.py`` against known-answer vectors, closed
forms, brute-force enumeration and chi-square tests (see each function's
docstring for its pin).  Parity unpinned: the numerical values of the pair
score, because the pages' formula was lost in extraction; only the reading
documented in ``oracle.dflash.pair_scores`` fixes them.
"""

from . import philox  # noqa: F401
from . import dflash  # noqa: F401
from . import conv  # noqa: F401
from . import viterbi  # noqa: F401
