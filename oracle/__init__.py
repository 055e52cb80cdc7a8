"""CPU oracle for the W4A4 + LoRA linear layer (test infrastructure only).

Only the tests, the package's ``smoke()`` check and the benchmark's CPU
baseline may import this package; the product path never does.
"""
from .w4a4_oracle import *  # noqa: F401,F403
