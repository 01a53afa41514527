"""CPU oracle -- test infrastructure only (tests/, __graft_entry__.smoke(), bench.py cpu_baseline)."""
from . import sa_oracle  # noqa: F401
