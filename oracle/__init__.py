"""CPU oracle of the Engram layer forward. TEST INFRASTRUCTURE: only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does."""
from . import engram_oracle  # noqa: F401
from .engram_oracle import *  # noqa: F401,F403
