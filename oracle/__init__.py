"""Float64 CPU oracle (test infrastructure only; see pc_oracle)."""
from .pc_oracle import (forward, backward, em_step, em_step_corrected, lowrank_effective,  # noqa: F401
                        lowrank_param_ranges, lowrank_scale)
