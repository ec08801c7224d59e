"""CPU fp64 oracle of the LoGRA sketch hot path -- TEST INFRASTRUCTURE.

This package is the slow, plain reference implementation that the HIP
library is checked against.  It shares no code with the library.  Only the
test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import it; the product path never does.

Every function cites the passage of the pages it follows (see the module
docstrings).  Pins that tie it to something other than itself live in
``tests/test_oracle_pins.py``.  One detail is "parity unpinned": the placement
of RowAdam's relative epsilon (invisible at eps = 1e-8).
"""
from . import philox  # noqa: F401
from .logra import *  # noqa: F401,F403
