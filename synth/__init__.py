"""Seeded synthetic inputs for the ResidualKV hot path.

This package holds the workload shapes and the random-number recipes that
both the HIP path and the CPU oracle consume.  It contains none of the
method's arithmetic (no distances, selection, means, residuals or
quantisation): it only draws K, V and queries.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .kvgen import gen_head_kv, gen_instance_kv, gen_queries, seed_for  # noqa: F401
