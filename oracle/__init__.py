"""CPU oracle (test infrastructure only): see q4moe_oracle."""
from . import q4moe_oracle  # noqa: F401
