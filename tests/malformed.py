"""Malformed rounds and the error class each must raise.  Shared by the
oracle's error tests and the host validator's tests; the two sides have
their own error codes, compared through these class names."""
import numpy as np

# (name, tok_seg, seg_parent, seg_fork, seg_cached_len, expected class)
CASES = [
    ("seg_out_of_range", [0, 0, 2], [-1, 0], [0, 2], [0, 0], "seg_range"),
    ("negative_seg", [0, -2], [-1, 0], [0, 1], [0, 0], "seg_range"),
    # -1 marks tail padding of a capacity bucket on the GPU side; before a
    # live token it is malformed on both sides
    ("padding_before_live", [-1, 0, 1], [-1, 0], [0, 1], [0, 0], "seg_range"),
    ("noncontiguous", [0, 1, 0], [-1, 0], [0, 1], [0, 0], "noncontig"),
    ("parent_out_of_range", [0, 1], [-1, 5], [0, 1], [0, 0], "parent"),
    ("self_parent", [0, 1], [-1, 1], [0, 0], [0, 0], "parent"),
    ("cycle", [0, 1, 2], [2, 0, 1], [0, 1, 1], [0, 0, 0], "cycle"),
    ("fork_past_parent_end", [0, 0, 1], [-1, 0], [0, 3], [0, 0], "fork"),
    ("negative_fork", [0, 0, 1], [-1, 0], [0, -1], [0, 0], "fork"),
    ("root_with_fork", [0, 1], [-1, 0], [2, 1], [0, 0], "fork"),
    ("live_segment_without_tokens", [0, 0], [-1, 0], [0, 1], [0, 0], "empty"),
    ("cached_with_tokens", [0, 1], [-1, 0], [0, 3], [3, 0], "empty"),
    ("cached_below_live", [0], [-1, 0], [0, 1], [0, 4], "cached"),
    ("fork_inside_cached", [1, 1], [-1, 0], [0, 2], [5, 0], "cached"),
]


def arrays(case):
    name, ts, par, fk, cl, kind = case
    return (np.array(ts, np.int32), np.array(par, np.int32), np.array(fk, np.int32),
            np.array(cl, np.int32), kind)
