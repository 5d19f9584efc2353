"""lossless_draft_verification_amd: batched lossless verification of
speculative-decoding drafts on AMD Instinct MI355X (gfx950).

The work happens in libspecverify.so (hand-written HIP, C ABI in
include/specverify.h); this package is a thin ctypes binding over torch
device tensors and the current HIP stream.
"""
from ._lib import (  # noqa: F401
    BF16, DRAFT_ONEHOT, DRAFT_PROBS, F32, FLAG_BLOCK, FLAG_DECIDE_ONLY, FLAG_KF_ROWS, FLAG_FP64_RACE, FLAG_FUSED, FLAG_PHASED, FLAG_STATS_ONLY, MAX_BATCH, MAX_DRAFT, MAX_NODES,
    MAX_VOCAB, REQ_BAD_DRAFT_ID, REQ_BAD_TEMPERATURE, REQ_BAD_TREE, REQ_INTERNAL, REQ_NONFINITE, REQ_OK,
    LIB_PATH, PLAN_MAX_SLOTS, PreparedChain, PreparedPlan, SpecVerifyError, Workspace, abi_version, chain_workspace_bytes, compact_kv, default_workspace, lib, plan_budget, plan_workspace_bytes,
    row_stats, row_stats_workspace_bytes, status_string, tree_workspace_bytes, verify_chain, verify_chain_noalloc,
    verify_tree, SCRATCH_BYTES, SCRATCH_MAX_BATCH, PreparedTree, stream_read,
)
