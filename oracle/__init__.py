"""CPU oracle for the Fathom plane-prefix scan -- test infrastructure only.

Importable by tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .fathom_oracle import *  # noqa: F401,F403
