"""Seeded synthetic inputs for tree-attention verification.

This package only *draws inputs*: draft trees, draft/target tokens, prefix
lengths and q/k/v tensors.  It holds none of the verification arithmetic
(no masks, no attention, no acceptance walk, no compaction), so both the CPU
oracle and the HIP path can be fed from it without sharing any of the method.
``make_paged`` only places a workload's rows into a pool of token slots; ``make_stochastic``
draws next-token distributions, drafted tokens and uniforms for sampling-mode acceptance;
``make_draft_levels`` draws the drafter's per-level candidates (tokens and confidences) that
EAGLE-2 tree construction consumes; ``make_lm_head`` draws a drafter LM head (low-rank factors,
shuffled rows, the full head) and hidden states.  The workload trees themselves are inputs of the
verification step, drawn by a float64 expand-and-rerank recipe in ``eagle2_tree``; the
device-side tree construction is checked against the oracle on ``make_draft_levels`` inputs,
never against these trees.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    PagedLayout,
    StochasticInputs,
    Workload,
    WorkloadSpec,
    DraftLevels,
    LM_HEADS,
    LmHeadInputs,
    make_draft_levels,
    make_lm_head,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_paged,
    make_stochastic,
    make_workload,
    random_parent,
    worked_tree_parent,
)
