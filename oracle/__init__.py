"""CPU oracle for InfLLM v2 block-sparse attention (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package; the product path never does.
"""
from .infllmv2_oracle import *  # noqa: F401,F403
