"""Float64 CPU oracle (test infrastructure only; see gdr_oracle)."""
from .gdr_oracle import forward, backward, rel_l2, head_map  # noqa: F401
