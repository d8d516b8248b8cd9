"""CPU oracle for the GPT-2 training step. TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference the HIP library is checked against. It shares no
code with the library. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import it; the product path never does.
"""
from .gpt2_oracle import *  # noqa: F401,F403
