"""CPU oracle of the routed-MoE MLP forward.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it; the HIP library and its
Python binding never do, and nothing here imports them.

  moe_oracle  vectorised NumPy float64 rendering of every step
  loops       pure-Python rendering (tiny inputs) used to check the first
"""
from . import moe_oracle, loops  # noqa: F401
from .moe_oracle import forward, take_rows  # noqa: F401
