"""Seeded synthetic workloads (circuit structures and inputs) for the sum-layer
hot path.  Shared by the float64 oracle and by the HIP path's tests and
benchmark; holds no arithmetic of the method itself."""
from .circuits import (Circuit, InputCat, InputExternal, Product, Sum, SumGroup,  # noqa: F401
                       hmm, hclt, dense_layer, block_sparse, random_block_layer, prufer_tree, pd,
                       node_ranges)
from .inputs import (softmax_rows_params, uniform_tokens, external_values,  # noqa: F401
                     uniform_flows, lowrank_factors, lowrank_sigma_for_spread)
from .configs import CONFIGS, make_config  # noqa: F401
