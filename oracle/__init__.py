"""CPU oracle (test infrastructure): see kvq_oracle.py.  Only tests/, the
smoke check and bench.py's CPU-baseline leg may import this package."""
from . import kvq_oracle  # noqa: F401
