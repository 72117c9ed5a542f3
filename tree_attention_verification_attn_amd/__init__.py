"""Tree-attention verification of speculative draft trees on AMD Instinct MI355X (gfx950).

The computation lives in libtreeverify.so (hand-written HIP kernels behind the C ABI in
include/tree_verify.h); this package only builds and binds it.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    TV_BAD_LEN,
    TV_BAD_PAGE,
    TV_BAD_PATH,
    TV_BAD_TOKEN,
    TV_BAD_TREE,
    TV_BF16,
    TV_ERR_HIP,
    TV_ERR_INVALID_ARG,
    TV_ERR_UNSUPPORTED,
    TV_ERR_WORKSPACE,
    TV_F32,
    TV_OK,
    TV_OVERFLOW,
    TV_SYNC_TIMEOUT,
    TreeVerifyError,
    kv_commit_paged,
    kv_compact_accepted,
    lib_path,
    load_library,
    profile_accept_stochastic,
    profile_attn_main,
    status_string,
    tree_accept,
    tree_accept_stochastic,
    tree_accept_stochastic_workspace_size,
    tree_build_mask,
    tree_verify_attn,
    tree_verify_attn_paged,
    tree_verify_attn_workspace_size,
    tree_verify_step,
)
