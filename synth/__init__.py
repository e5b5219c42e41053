"""Seeded synthetic inputs for the RaggedShard shard step.

This package generates *inputs only*: bucket tensor lists (shapes and
RaggedShard block geometry), the bucket layout a planner hands to the shard
step, and seeded random parameter / gradient values.  It holds none of the
optimizer's arithmetic.  Both the GPU path's tests and the CPU oracle's tests
draw their inputs from here; neither side imports the other.
"""

from .configs import (CONFIGS, HPARAMS, TensorDef, Config, get_config,  # noqa: F401
                      toy_variants)
from .layout import Layout, plan_p0  # noqa: F401
