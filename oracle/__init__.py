"""fp64 CPU oracle of the Compressor operator: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never imports it.
"""
from .compressor_oracle import *  # noqa: F401,F403
