"""MI355X (gfx950) library for exact state forking of decision-request trees:
ForkAttention and forked Gated DeltaNet behind a C ABI (include/forkgdn.h).

The HIP library ``libforkgdn.so`` is the only implementation; this package
marshals torch tensors into its calls (``api``) and plans page tables for
rounds (``rounds``).
"""
from . import _lib  # noqa: F401
from .api import (TreeMeta, alloc_workspace, fk_read_status, fk_strerror,  # noqa: F401
                  fk_token_positions, fk_tree_build, fk_tree_validate_host, fk_workspace_bytes,
                  fork_attn_forward, fork_attn_forward_noalloc, fork_attn_forward_rule, fork_attn_readout,
                  gdn_checkpoint_resume, gdn_checkpoint_save, gdn_conv_forward,
                  gdn_fork_forward,
                  kv_append, make_tree_meta, fk_peak_mfma_bf16, fk_proj_gemm)
from .rounds import Bucket, RoundPlan, bucket_for, capacities, plan_arrays, plan_round  # noqa: F401,E402
from .graph import BucketRound, GraphFamily, StepGraph  # noqa: F401,E402
