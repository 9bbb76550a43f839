"""Float64 CPU oracle of MSA decode -- test infrastructure only (tests,
__graft_entry__.smoke and bench.py's cpu_baseline leg). The library path
never imports this package."""
from . import msa_oracle  # noqa: F401
