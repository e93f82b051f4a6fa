"""Seeded synthetic decision-request workloads.

This package only draws inputs: tree structures (trunk, branches, deeper
forks, cached histories), the flat stream layout, and the random tensors of
every segment.  It holds none of the method's arithmetic (no visibility rule,
no attention, no recurrence), so both the fp64 oracle and the HIP path can
consume the same inputs without sharing any code of the method.
"""
from .trees import Seg, Tree, build_tree, subtree_path, random_tree  # noqa: F401
from .tensors import draw_inputs, draw_conv, to_bf16, Inputs, ConvInputs  # noqa: F401
from .configs import WORKLOADS, make_config  # noqa: F401
