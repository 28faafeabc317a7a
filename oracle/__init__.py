"""CPU oracle for the TTQ per-prompt hot path — test infrastructure only.

Imported by the tests, by the smoke check and by the benchmark's CPU-baseline
leg; never by the product path.  See ``ttq_oracle`` for the definitions and
the readings of the source pages they follow.
"""
from .ttq_oracle import *  # noqa: F401,F403
from .ttq_oracle import __all__  # noqa: F401
