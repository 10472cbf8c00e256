"""CPU oracle for the Gated DeltaNet state layer (test infrastructure only).

Imported only by tests/, __graft_entry__.smoke() and the CPU-baseline leg of
bench.py; the GPU library never imports it.
"""
from .gdn_oracle import *  # noqa: F401,F403
from .gdn_oracle import __all__  # noqa: F401
